"""C ABI: the library loads without a GPU, exports every declared symbol, and
rejects invalid arguments with status codes (no compute calls here)."""

import ctypes as C
import math
import os
import re

import numpy as np
import pytest

from prefill_decode_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    src = open(os.path.join(ROOT, "include", "pod_attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pod_attn_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    declared = _declared_symbols()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(B.EXPORTED)


def _plan_status(params, qo, kv, dkv, tuning=None):
    lib = B.lib()
    qo, kv, dkv = (np.ascontiguousarray(np.asarray(x, np.int32)) for x in (qo, kv, dkv))
    h = C.c_void_p(0)
    dev = B.DeviceDesc(256, 8)
    st = lib.pod_attn_plan_host(C.byref(params), len(qo), B._ptr(qo), B._ptr(kv), len(dkv),
                                B._ptr(dkv), C.byref(tuning) if tuning else None,
                                C.byref(dev), C.byref(h))
    if h.value:
        lib.pod_attn_plan_destroy(h)
    return st


OK, INV, UNS = 0, 1, 2


@pytest.mark.parametrize("case,expect", [
    (dict(qo=[5], kv=[4], dkv=[]), INV),                    # qo > kv
    (dict(qo=[0], kv=[4], dkv=[]), INV),                    # qo = 0
    (dict(qo=[], kv=[], dkv=[0]), INV),                     # decode kv = 0
    (dict(qo=[], kv=[], dkv=[-3]), INV),
    (dict(qo=[4], kv=[4], dkv=[7]), OK),
    (dict(qo=[], kv=[], dkv=[]), OK),                       # empty batch is valid
    (dict(hq=6, hkv=4), INV),                               # Hq % Hkv != 0
    (dict(hq=0, hkv=1), INV),
    (dict(head_dim=64), UNS),
    (dict(page_size=12), INV),
    (dict(page_size=0), INV),
    (dict(page_size=2048), INV),
    (dict(page_size=1), OK),
    (dict(page_size=8), OK),
    (dict(sm_scale=0.0), INV),
    (dict(sm_scale=-1.0), INV),
    (dict(sm_scale=float("nan")), INV),
    (dict(sm_scale=float("inf")), INV),
    (dict(layout=7), INV),
    (dict(causal=2), INV),
    (dict(qo=[3], kv=[1 << 25], dkv=[]), UNS),
    (dict(kv_dtype=2), INV),                                # unknown dtype
    (dict(kv_dtype=1), OK),                                 # FP8 cache, hybrid batch
    (dict(kv_dtype=1, qo=[], kv=[]), OK),                   # FP8 decode-only
    (dict(kv_dtype=1, qo=[], kv=[], page_size=8), UNS),     # FP8 needs pages >= 16
    (dict(kv_dtype=1, page_size=8), UNS),                   # (also with a prefill)
])
def test_plan_validation(case, expect):
    p = B.make_params(case.get("hq", 8), case.get("hkv", 2), "paged",
                      case.get("page_size", 16), True,
                      case.get("sm_scale", 1 / math.sqrt(128)), case.get("head_dim", 128))
    if "layout" in case:
        p.kv_layout = case["layout"]
    if "causal" in case:
        p.causal = case["causal"]
    if "kv_dtype" in case:
        p.kv_dtype = case["kv_dtype"]
    st = _plan_status(p, case.get("qo", [4]), case.get("kv", [9]), case.get("dkv", [5]))
    assert st == expect, (st, B.last_error())
    if st != OK:
        assert B.last_error()


@pytest.mark.parametrize("tun,expect", [
    (dict(wgs_per_cu=4), UNS), (dict(wgs_per_cu=3), UNS), (dict(wgs_per_cu=2), OK),
    (dict(prefill_quarters_per_cu=9), INV), (dict(prefill_quarters_per_cu=-2), INV),
    (dict(prefill_kv_splits=-1), INV), (dict(decode_kv_splits=-1), INV),
    (dict(sched_mode=4), INV), (dict(match_sequential=2), INV),
    (dict(sched_mode=B.SCHED_COLOCATE, prefill_quarters_per_cu=8), OK),
])
def test_tuning_validation(tun, expect):
    p = B.make_params(8, 2)
    st = _plan_status(p, [4], [9], [5], B.make_tuning(**tun))
    assert st == expect, (st, B.last_error())


def test_null_length_arrays_rejected():
    lib = B.lib()
    p = B.make_params(8, 2)
    h = C.c_void_p(0)
    dev = B.DeviceDesc(256, 8)
    st = lib.pod_attn_plan_host(C.byref(p), 2, None, None, 0, None, None, C.byref(dev),
                                C.byref(h))
    assert st == INV and not h.value
    st = lib.pod_attn_plan_host(C.byref(p), 0, None, None, 3, None, None, C.byref(dev),
                                C.byref(h))
    assert st == INV and not h.value
    st = lib.pod_attn_plan_host(None, 0, None, None, 0, None, None, C.byref(dev), C.byref(h))
    assert st == INV
    st = lib.pod_attn_plan_host(C.byref(p), 0, None, None, 0, None, None, None, C.byref(h))
    assert st == INV
    bad = B.DeviceDesc(0, 8)
    st = lib.pod_attn_plan_host(C.byref(p), 0, None, None, 0, None, None, C.byref(bad),
                                C.byref(h))
    assert st == INV


def test_host_plan_cannot_run_and_null_handles():
    lib = B.lib()
    pl = B.plan_host(B.make_params(8, 2), [4], [9], [5])
    t = B.Tensors()
    st = lib.pod_attn_run(pl.handle, C.byref(t), None)
    assert st == INV and "workspace" in B.last_error()
    st = lib.pod_attn_sequential_run(pl.handle, C.byref(t), None)
    assert st == INV
    assert lib.pod_attn_run(None, C.byref(t), None) == INV
    assert lib.pod_attn_run(pl.handle, None, None) == INV
    assert lib.pod_attn_plan_info(None, None) == INV
    cnt = C.c_size_t(0)
    assert lib.pod_attn_plan_export(pl.handle, 99, None, 0, C.byref(cnt)) == INV
    assert lib.pod_attn_read_trace(pl.handle, None, 0, C.byref(cnt), None) == INV
    assert lib.pod_attn_probe_hwid(0, None, None) == INV
    lib.pod_attn_plan_destroy(None)   # no-op
    info = pl.info()
    # 8 q heads over 2 KV heads: two items of 4 packed heads x 1 position block
    assert info["workspace_bytes"] > 0 and info["prefill_items"] == 2
    pl.destroy()


def test_one_hip_runtime_whatever_the_import_order():
    # the library loaded before torch must not bring a second HIP runtime
    # into the process (one of two would not see the device)
    import subprocess
    import sys
    code = ("import prefill_decode_amd.binding as B\nB.lib()\nimport torch\n"
            "print(len({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0, r.stderr[-500:]
    assert r.stdout.strip().splitlines()[-1] == "1", r.stdout


def test_plan_refuses_partials_beyond_int32():
    """A batch whose split partials would outgrow their int32 indices (one
    non-causal chunk of 2^19 rows, 64 query heads, 64 forced KV splits:
    2^31 partial rows) is refused with POD_ERR_UNSUPPORTED; one row fewer
    per tile's share (2^19 - 64 rows) plans."""
    p = B.make_params(64, 8, causal=False)
    t = B.make_tuning(prefill_kv_splits=64, match_sequential=1)
    n = 1 << 19
    st = _plan_status(p, [n], [n], [], t)
    assert st == UNS and "2^31 - 1 split partials" in B.last_error(), (st, B.last_error())
    assert _plan_status(p, [n - 64], [n - 64], [], t) == OK, B.last_error()
