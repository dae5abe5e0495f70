"""The planner and the C ABI (host C++) under AddressSanitizer and
UndefinedBehaviorSanitizer.

A g++ -fsanitize=address,undefined build of the library's host code (linked
with the regular device-code object) is loaded, in a child process that
preloads the gcc ASan runtime, in place of the in-tree build; the planner and
ABI tests run against it.  Any heap overflow, use after free or undefined
behaviour in plan building, validation, list export or error paths aborts the
child.  CPU only: no kernel is launched."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    try:
        p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                           text=True, timeout=30).stdout.strip()
    except (OSError, subprocess.SubprocessError):
        return None
    return p if p and os.path.isabs(p) and os.path.exists(p) else None


def test_planner_and_abi_under_asan_ubsan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    sys.path.insert(0, ROOT)
    from prefill_decode_amd import build
    lib = build.build_sanitized(verbose=False)
    env = dict(os.environ, LD_PRELOAD=rt, POD_ATTN_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # the instrumented build is the one the binding loads
    chk = subprocess.run(
        [sys.executable, "-c",
         "from prefill_decode_amd import binding as B\nB.lib()\n"
         "print(any(B._LIB_PATH in l for l in open('/proc/self/maps')))"],
        env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert chk.returncode == 0 and chk.stdout.strip().endswith("True"), chk.stderr[-2000:]
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "tests/test_plan.py", "tests/test_abi.py", "-q", "-x",
         "-m", "not gpu", "-p", "no:cacheprovider"],
        env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout
