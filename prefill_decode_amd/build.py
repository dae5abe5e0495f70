"""Builds libpod_attn.so in-tree (hipcc for gfx950, g++ for the host C++).

    python -m prefill_decode_amd.build          # or __graft_entry__.build()

Outputs ``prefill_decode_amd/libpod_attn.so``; objects go to ``_build/``.
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpod_attn.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

# Packed fp32 instructions are disabled (hipcc forms them on its own).  The
# atomic optimizer is off: it turns a one-lane claim into a wave-aggregated
# atomic whose result is read at once, which would stall every prefetched
# work claim for the atomic's full latency.  No arithmetic here produces or
# tests a NaN (masked scores are -inf, every -inf - -inf is guarded), so NaN
# semantics are not honoured: a float max then needs no canonicalising move
# of its inputs (eight fewer VALU instructions per prefill softmax half).
HIP_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
             "-fno-honor-nans",
             "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__",
             f"-I{ROCM}/include"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "--hip-link" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = True, save_isa: bool = False) -> str:
    """Compiles every source and links ``libpod_attn.so``; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    kern_obj = os.path.join(BUILD, "kernels.o")
    cmd = [HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "kernels.hip"), "-o", kern_obj]
    if save_isa:
        cmd[1:1] = ["-save-temps=obj"]
    _run(cmd, verbose)
    objs.append(kern_obj)
    cxx = shutil.which("g++") or "g++"
    for src in ("api.cpp", "plan.cpp"):
        obj = os.path.join(BUILD, src.replace(".cpp", ".o"))
        _run([cxx, *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


# Host-side sanitizer build: the planner and the C ABI (host C++ only) are
# compiled with AddressSanitizer and UndefinedBehaviorSanitizer by g++ and
# linked with the regular device-code object.  Loaded into a Python process
# that preloads the gcc ASan runtime (see tests/test_sanitizers.py).
SAN_DIR = os.path.join(BUILD, "sanitize")
SAN_LIB = os.path.join(SAN_DIR, "libpod_attn.so")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined"]


def build_sanitized(verbose: bool = False) -> str:
    """Builds _build/sanitize/libpod_attn.so (host code instrumented); returns its path."""
    kern_obj = os.path.join(BUILD, "kernels.o")
    if not os.path.exists(kern_obj):
        build(verbose)
    os.makedirs(SAN_DIR, exist_ok=True)
    cxx = shutil.which("g++") or "g++"
    objs = [kern_obj]
    for src in ("api.cpp", "plan.cpp"):
        obj = os.path.join(SAN_DIR, src.replace(".cpp", ".o"))
        _run([cxx, *CXX_FLAGS, *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    _run([cxx, "-shared", "-fPIC", *SAN_FLAGS, *objs, "-o", SAN_LIB,
          f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"], verbose)
    return SAN_LIB


if __name__ == "__main__":
    build(verbose=True, save_isa="--isa" in sys.argv)
    if "--sanitize" in sys.argv:
        build_sanitized(verbose=True)
