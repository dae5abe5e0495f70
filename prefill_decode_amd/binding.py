"""ctypes binding of libpod_attn.so (argument marshalling only).

Every step of the attention runs in the library's HIP kernels; this module
only converts Python/torch arguments into the C ABI of ``include/pod_attn.h``.
The library is loaded on first use and its absence is an error (there is no
fallback path).
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional, Sequence

import numpy as np

# POD_ATTN_LIB selects another build of the same library (the host-sanitizer
# build in the tests); by default the in-tree build is loaded.
_LIB_PATH = os.environ.get("POD_ATTN_LIB") or \
    os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpod_attn.so")
_lib = None

POD_OK = 0
STATUS = {0: "POD_OK", 1: "POD_ERR_INVALID_ARGUMENT", 2: "POD_ERR_UNSUPPORTED",
          3: "POD_ERR_WORKSPACE_TOO_SMALL", 4: "POD_ERR_HIP", 5: "POD_ERR_INTERNAL"}
KV_CONTIGUOUS, KV_PAGED = 0, 1
KV_BF16, KV_FP8_E4M3 = 0, 1
SCHED_AUTO, SCHED_COLOCATE, SCHED_ORDERED, SCHED_SPLIT = 0, 1, 2, 3
FLAG_TRACE = 0x1
FLAG_BATCHED_PREFILL = 0x2
FLAG_ONE_UNIT_PER_WG = 0x4

# every function the header declares
EXPORTED = ("pod_attn_plan", "pod_attn_plan_host", "pod_attn_run", "pod_attn_run_events",
            "pod_attn_sequential_run", "pod_attn_streams_run", "pod_attn_batched_prefill_run",
            "pod_attn_merge",
            "pod_attn_plan_info", "pod_attn_plan_export", "pod_attn_read_trace",
            "pod_attn_plan_destroy", "pod_attn_last_error", "pod_attn_probe_hwid",
            "pod_attn_probe_read_bw", "pod_attn_plan_scratch", "pod_attn_plan_shared_prefix",
            "pod_attn_plan_shared_prefix_host")


class PodError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Params(C.Structure):
    _fields_ = [("num_qo_heads", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("kv_layout", C.c_int32), ("page_size", C.c_int32),
                ("causal", C.c_int32), ("sm_scale", C.c_float), ("kv_dtype", C.c_int32)]


class Tuning(C.Structure):
    _fields_ = [("wgs_per_cu", C.c_int32), ("prefill_quarters_per_cu", C.c_int32),
                ("prefill_kv_splits", C.c_int32), ("decode_kv_splits", C.c_int32),
                ("match_sequential", C.c_int32), ("sched_mode", C.c_int32),
                ("flags", C.c_uint32)]


class DeviceDesc(C.Structure):
    _fields_ = [("num_cus", C.c_int32), ("num_xcds", C.c_int32)]


class PlanInfo(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "prefill_items", "decode_items", "decode_groups", "merge_tasks",
        "seq_prefill_items", "seq_decode_items", "seq_merge_tasks",
        "prefill_splits_max", "decode_splits_max", "wgs_per_cu",
        "prefill_quarters_per_cu", "sched_mode", "one_unit_per_wg", "num_partials",
        "trace_records", "runs_sequential")] + \
        [("workspace_bytes", C.c_uint64)]


class TraceRecord(C.Structure):
    _fields_ = [("block", C.c_int32), ("cu_slot", C.c_int32), ("role", C.c_int32),
                ("unit", C.c_int32), ("t_start", C.c_uint64), ("t_end", C.c_uint64)]


class Tensors(C.Structure):
    _fields_ = [("q_prefill", C.c_void_p), ("q_decode", C.c_void_p), ("k", C.c_void_p),
                ("v", C.c_void_p), ("kv_indptr", C.c_void_p), ("page_indptr", C.c_void_p),
                ("page_indices", C.c_void_p), ("o_prefill", C.c_void_p),
                ("o_decode", C.c_void_p), ("lse_prefill", C.c_void_p),
                ("lse_decode", C.c_void_p), ("k_scale", C.c_void_p), ("v_scale", C.c_void_p)]


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m prefill_decode_amd.build` (no fallback exists)")
        # torch first: its bundled HIP runtime (same soname as the system's)
        # then serves the library too.  Loaded first, the library would pull
        # the system runtime in beside torch's, and one of the two would not
        # see the device.
        import torch  # noqa: F401
        L = C.CDLL(_LIB_PATH)
        i32p = C.POINTER(C.c_int32)
        L.pod_attn_plan.argtypes = [C.POINTER(Params), C.c_int32, i32p, i32p, C.c_int32, i32p,
                                    C.POINTER(Tuning), C.c_void_p, C.c_size_t,
                                    C.POINTER(C.c_size_t), C.c_void_p, C.POINTER(C.c_void_p)]
        L.pod_attn_plan_shared_prefix.argtypes = [C.POINTER(Params), C.c_int32, i32p, i32p,
                                                  C.c_int32, i32p, C.POINTER(Tuning),
                                                  C.c_void_p, C.c_size_t,
                                                  C.POINTER(C.c_size_t), C.c_void_p,
                                                  C.POINTER(C.c_void_p)]
        L.pod_attn_plan_shared_prefix_host.argtypes = [C.POINTER(Params), C.c_int32, i32p,
                                                       i32p, C.c_int32, i32p,
                                                       C.POINTER(Tuning),
                                                       C.POINTER(DeviceDesc),
                                                       C.POINTER(C.c_void_p)]
        L.pod_attn_plan_scratch.argtypes = [C.POINTER(Params), C.c_int32, i32p, i32p,
                                            C.c_int32, i32p, C.POINTER(Tuning), C.c_void_p,
                                            C.POINTER(C.c_void_p)]
        L.pod_attn_plan_host.argtypes = [C.POINTER(Params), C.c_int32, i32p, i32p, C.c_int32,
                                         i32p, C.POINTER(Tuning), C.POINTER(DeviceDesc),
                                         C.POINTER(C.c_void_p)]
        L.pod_attn_run.argtypes = [C.c_void_p, C.POINTER(Tensors), C.c_void_p]
        L.pod_attn_run_events.argtypes = [C.c_void_p, C.POINTER(Tensors), C.c_void_p,
                                          C.c_void_p, C.c_void_p]
        L.pod_attn_sequential_run.argtypes = [C.c_void_p, C.POINTER(Tensors), C.c_void_p]
        L.pod_attn_streams_run.argtypes = [C.c_void_p, C.POINTER(Tensors), C.c_void_p,
                                           C.c_void_p]
        L.pod_attn_batched_prefill_run.argtypes = [C.c_void_p, C.POINTER(Tensors), C.c_void_p]
        L.pod_attn_merge.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p,
                                     C.c_void_p, C.c_void_p]
        L.pod_attn_plan_info.argtypes = [C.c_void_p, C.POINTER(PlanInfo)]
        L.pod_attn_plan_export.argtypes = [C.c_void_p, C.c_int32, i32p, C.c_size_t,
                                           C.POINTER(C.c_size_t)]
        L.pod_attn_read_trace.argtypes = [C.c_void_p, C.POINTER(TraceRecord), C.c_size_t,
                                          C.POINTER(C.c_size_t), C.c_void_p]
        L.pod_attn_plan_destroy.argtypes = [C.c_void_p]
        L.pod_attn_plan_destroy.restype = None
        L.pod_attn_last_error.restype = C.c_char_p
        L.pod_attn_probe_hwid.argtypes = [C.c_int32, C.c_void_p, C.c_void_p]
        L.pod_attn_probe_read_bw.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int32,
                                             C.c_void_p]
        for name in EXPORTED:
            if name not in ("pod_attn_plan_destroy", "pod_attn_last_error"):
                getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def last_error() -> str:
    return lib().pod_attn_last_error().decode()


def _check(st: int):
    if st != POD_OK:
        raise PodError(st, last_error())


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.POINTER(C.c_int32)) if a.size else None


def make_params(num_qo_heads, num_kv_heads, layout="paged", page_size=16, causal=True,
                sm_scale=None, head_dim=128, kv_dtype="bf16") -> Params:
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(head_dim)
    lay = KV_PAGED if layout in ("paged", KV_PAGED) else KV_CONTIGUOUS
    dt = KV_FP8_E4M3 if kv_dtype in ("fp8_e4m3", KV_FP8_E4M3) else KV_BF16
    return Params(int(num_qo_heads), int(num_kv_heads), int(head_dim), lay, int(page_size),
                  1 if causal else 0, float(sm_scale), dt)


def make_tuning(wgs_per_cu=0, prefill_quarters_per_cu=-1, prefill_kv_splits=0,
                decode_kv_splits=0, match_sequential=0, sched_mode=SCHED_AUTO,
                flags=0) -> Tuning:
    return Tuning(wgs_per_cu, prefill_quarters_per_cu, prefill_kv_splits, decode_kv_splits,
                  match_sequential, sched_mode, flags)


class Plan:
    """A plan (host object) plus, for device plans, its torch workspace."""

    def __init__(self, handle, workspace=None, batch_keys=None):
        self._h = C.c_void_p(handle)
        self.workspace = workspace

    @property
    def handle(self):
        return self._h

    def info(self) -> Dict[str, int]:
        inf = PlanInfo()
        _check(lib().pod_attn_plan_info(self._h, C.byref(inf)))
        return {n: getattr(inf, n) for n, _ in PlanInfo._fields_}

    def export(self, which: int) -> np.ndarray:
        cnt = C.c_size_t(0)
        _check(lib().pod_attn_plan_export(self._h, which, None, 0, C.byref(cnt)))
        out = np.zeros(cnt.value, dtype=np.int32)
        _check(lib().pod_attn_plan_export(self._h, which, _ptr(out), out.size, C.byref(cnt)))
        return out

    def read_trace(self, stream=None) -> np.ndarray:
        cnt = C.c_size_t(0)
        s = _stream(stream)
        _check(lib().pod_attn_read_trace(self._h, None, 0, C.byref(cnt), s))
        buf = (TraceRecord * cnt.value)()
        _check(lib().pod_attn_read_trace(self._h, buf, cnt.value, C.byref(cnt), s))
        return np.array([(r.block, r.cu_slot, r.role, r.unit, r.t_start, r.t_end) for r in buf],
                        dtype=np.int64).reshape(-1, 6)

    def destroy(self):
        if self._h is not None and self._h.value:
            lib().pod_attn_plan_destroy(self._h)
        self._h = C.c_void_p(0)

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def _stream(stream):
    if stream is None:
        import torch
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


def plan_host(params: Params, prefill_qo: Sequence[int], prefill_kv: Sequence[int],
              decode_kv: Sequence[int], tuning: Optional[Tuning] = None,
              num_cus: int = 256, num_xcds: int = 8) -> Plan:
    """Plans without a GPU (host inspection); the plan cannot run."""
    qo, kv, dk = _i32(prefill_qo), _i32(prefill_kv), _i32(decode_kv)
    h = C.c_void_p(0)
    dev = DeviceDesc(num_cus, num_xcds)
    _check(lib().pod_attn_plan_host(C.byref(params), len(qo), _ptr(qo), _ptr(kv), len(dk),
                                    _ptr(dk), C.byref(tuning) if tuning else None,
                                    C.byref(dev), C.byref(h)))
    return Plan(h.value)


def plan(params: Params, prefill_qo: Sequence[int], prefill_kv: Sequence[int],
         decode_kv: Sequence[int], tuning: Optional[Tuning] = None, device="cuda",
         stream=None) -> Plan:
    """Plans for the current device; allocates the workspace as a torch
    uint8 tensor on `device` and uploads the plan's work lists into it."""
    import torch
    qo, kv, dk = _i32(prefill_qo), _i32(prefill_kv), _i32(decode_kv)
    need = C.c_size_t(0)
    s = _stream(stream)
    tp = C.byref(tuning) if tuning else None
    _check(lib().pod_attn_plan(C.byref(params), len(qo), _ptr(qo), _ptr(kv), len(dk), _ptr(dk),
                               tp, None, 0, C.byref(need), s, None))
    ws = torch.empty(max(int(need.value), 256), dtype=torch.uint8, device=device)
    h = C.c_void_p(0)
    _check(lib().pod_attn_plan(C.byref(params), len(qo), _ptr(qo), _ptr(kv), len(dk), _ptr(dk),
                               tp, C.c_void_p(ws.data_ptr()), ws.numel(), C.byref(need), s,
                               C.byref(h)))
    return Plan(h.value, workspace=ws)


def plan_shared_prefix_host(params: Params, decode_kv: Sequence[int],
                            prefix_group: Sequence[int], prefix_len: Sequence[int],
                            tuning: Optional[Tuning] = None, num_cus: int = 256,
                            num_xcds: int = 8) -> Plan:
    """Shared-prefix plan without a GPU (host inspection); it cannot run."""
    dk, pg, pln = _i32(decode_kv), _i32(prefix_group), _i32(prefix_len)
    h = C.c_void_p(0)
    dev = DeviceDesc(num_cus, num_xcds)
    _check(lib().pod_attn_plan_shared_prefix_host(C.byref(params), len(dk), _ptr(dk), _ptr(pg),
                                                  len(pln), _ptr(pln),
                                                  C.byref(tuning) if tuning else None,
                                                  C.byref(dev), C.byref(h)))
    return Plan(h.value)


def plan_shared_prefix(params: Params, decode_kv: Sequence[int], prefix_group: Sequence[int],
                       prefix_len: Sequence[int], tuning: Optional[Tuning] = None,
                       device="cuda", stream=None) -> Plan:
    """Shared-prefix (packed) decode plan; allocates its torch workspace."""
    import torch
    dk, pg, pln = _i32(decode_kv), _i32(prefix_group), _i32(prefix_len)
    need = C.c_size_t(0)
    s = _stream(stream)
    tp = C.byref(tuning) if tuning else None
    _check(lib().pod_attn_plan_shared_prefix(C.byref(params), len(dk), _ptr(dk), _ptr(pg),
                                             len(pln), _ptr(pln), tp, None, 0, C.byref(need),
                                             s, None))
    ws = torch.empty(max(int(need.value), 256), dtype=torch.uint8, device=device)
    h = C.c_void_p(0)
    _check(lib().pod_attn_plan_shared_prefix(C.byref(params), len(dk), _ptr(dk), _ptr(pg),
                                             len(pln), _ptr(pln), tp, C.c_void_p(ws.data_ptr()),
                                             ws.numel(), C.byref(need), s, C.byref(h)))
    return Plan(h.value, workspace=ws)


def plan_scratch(params: Params, prefill_qo: Sequence[int], prefill_kv: Sequence[int],
                 decode_kv: Sequence[int], tuning: Optional[Tuning] = None,
                 stream=None) -> Plan:
    """Plans for the current device into the library's static scratch (no
    device allocation; see pod_attn_plan_scratch for the sharing rules)."""
    qo, kv, dk = _i32(prefill_qo), _i32(prefill_kv), _i32(decode_kv)
    h = C.c_void_p(0)
    _check(lib().pod_attn_plan_scratch(C.byref(params), len(qo), _ptr(qo), _ptr(kv), len(dk),
                                       _ptr(dk), C.byref(tuning) if tuning else None,
                                       _stream(stream), C.byref(h)))
    return Plan(h.value)


def _dp(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def make_tensors(q_prefill=None, q_decode=None, k=None, v=None, kv_indptr=None,
                 page_indptr=None, page_indices=None, o_prefill=None, o_decode=None,
                 lse_prefill=None, lse_decode=None, k_scale=None, v_scale=None) -> Tensors:
    return Tensors(_dp(q_prefill), _dp(q_decode), _dp(k), _dp(v), _dp(kv_indptr),
                   _dp(page_indptr), _dp(page_indices), _dp(o_prefill), _dp(o_decode),
                   _dp(lse_prefill), _dp(lse_decode), _dp(k_scale), _dp(v_scale))


def run(p: Plan, tensors: Tensors, stream=None):
    """Fused prefill+decode attention (asynchronous on the stream)."""
    _check(lib().pod_attn_run(p.handle, C.byref(tensors), _stream(stream)))


def run_events(p: Plan, tensors: Tensors, before_fused, after_fused, stream=None):
    """`run` recording two torch.cuda.Event objects (timing enabled) on the
    stream immediately around the fused kernel's launch."""
    for e in (before_fused, after_fused):
        if not e.cuda_event:          # torch creates the HIP event on first record
            e.record()
    _check(lib().pod_attn_run_events(p.handle, C.byref(tensors), _stream(stream),
                                     C.c_void_p(before_fused.cuda_event),
                                     C.c_void_p(after_fused.cuda_event)))


def sequential_run(p: Plan, tensors: Tensors, stream=None):
    """Prefill kernel, then decode kernel, then merge (asynchronous)."""
    _check(lib().pod_attn_sequential_run(p.handle, C.byref(tensors), _stream(stream)))


def streams_run(p: Plan, tensors: Tensors, decode_stream, stream=None):
    """Prefill kernel on `stream`, decode kernel on `decode_stream`, merge on
    `stream` after both (asynchronous)."""
    _check(lib().pod_attn_streams_run(p.handle, C.byref(tensors), _stream(stream),
                                      _stream(decode_stream)))


def batched_prefill_run(p: Plan, tensors: Tensors, stream=None):
    """Every request through the prefill kernel (decodes as one-row chunks),
    then the merge; the plan needs FLAG_BATCHED_PREFILL (asynchronous)."""
    _check(lib().pod_attn_batched_prefill_run(p.handle, C.byref(tensors), _stream(stream)))


def merge(part_o, part_lse, o, lse=None, stream=None):
    """Log-sum-exp merge of fp32 partials [rows, splits, 128] / LSEs [rows,
    splits] (natural log) into bf16 o [rows, 128] and fp32 lse [rows]."""
    rows, splits = int(part_lse.shape[0]), int(part_lse.shape[1])
    assert tuple(part_o.shape) == (rows, splits, 128) and part_o.is_contiguous()
    assert part_lse.is_contiguous() and tuple(o.shape) == (rows, 128) and o.is_contiguous()
    _check(lib().pod_attn_merge(_dp(part_o), _dp(part_lse), rows, splits, _dp(o), _dp(lse),
                                _stream(stream)))


def probe_hwid(num_blocks: int, device="cuda", stream=None) -> np.ndarray:
    import torch
    out = torch.zeros(2 * num_blocks, dtype=torch.int32, device=device)
    _check(lib().pod_attn_probe_hwid(num_blocks, C.c_void_p(out.data_ptr()), _stream(stream)))
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(-1, 2)


def probe_read_bw(buf, sink, num_blocks=2048, stream=None):
    """Enqueues one read of the whole device tensor `buf` (the HBM read-rate
    probe); `sink` is a device uint32/int32 tensor of at least one element."""
    _check(lib().pod_attn_probe_read_bw(_dp(buf), buf.numel() * buf.element_size(), _dp(sink),
                                        int(num_blocks), _stream(stream)))


# ---------------------------------------------------------------------------
# Convenience over a batch dict (prefill_decode_amd.inputs layout)
# ---------------------------------------------------------------------------

class BatchRunner:
    """Owns the device tensors of one batch and its plan; `run()` /
    `sequential_run()` write into ``o_prefill``/``o_decode``/``lse_*``."""

    def __init__(self, batch: Dict, tuning: Optional[Tuning] = None, device="cuda"):
        import torch
        self.batch = batch
        b = batch
        self.params = make_params(b["num_qo_heads"], b["num_kv_heads"], b["layout"],
                                  b["page_size"], b["causal"], b["sm_scale"], b["head_dim"],
                                  b.get("kv_dtype", "bf16"))

        def dev(x, dtype=None):
            if isinstance(x, torch.Tensor):
                return x.to(device)
            if isinstance(x, np.ndarray) and x.dtype == np.uint16:
                return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device) \
                    .view(torch.bfloat16)
            if isinstance(x, np.ndarray) and x.dtype in (np.uint8, np.float32):
                return torch.from_numpy(np.ascontiguousarray(x)).to(device)
            return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.int32))) \
                .to(device)

        self.q_prefill = dev(b["q_prefill"])
        self.q_decode = dev(b["q_decode"])
        self.k = dev(b["k_cache"])
        self.v = dev(b["v_cache"])
        self.kv_indptr = dev(b["kv_indptr"]) if "kv_indptr" in b else None
        self.page_indptr = dev(b["page_indptr"]) if "page_indptr" in b else None
        self.page_indices = dev(b["page_indices"]) if "page_indices" in b else None
        self.k_scale = dev(b["k_scale"]) if "k_scale" in b else None
        self.v_scale = dev(b["v_scale"]) if "v_scale" in b else None
        hq = b["num_qo_heads"]
        self.o_prefill = torch.empty_like(self.q_prefill)
        self.o_decode = torch.empty_like(self.q_decode)
        self.lse_prefill = torch.empty(self.q_prefill.shape[0], hq, dtype=torch.float32,
                                       device=device)
        self.lse_decode = torch.empty(self.q_decode.shape[0], hq, dtype=torch.float32,
                                      device=device)
        if b.get("prefix_groups"):
            # decode-only batch with shared prefixes: the packed plan
            nd = len(b["decode_kv_len"])
            grp = np.full(nd, -1, dtype=np.int32)
            plen = []
            for gi, (members, pl_) in enumerate(b["prefix_groups"]):
                grp[list(members)] = gi
                plen.append(pl_)
            self.plan = plan_shared_prefix(self.params, b["decode_kv_len"], grp, plen, tuning,
                                           device=device)
        else:
            self.plan = plan(self.params, b["prefill_qo_len"], b["prefill_kv_len"],
                             b["decode_kv_len"], tuning, device=device)
        self.tensors = make_tensors(self.q_prefill, self.q_decode, self.k, self.v,
                                    self.kv_indptr, self.page_indptr, self.page_indices,
                                    self.o_prefill, self.o_decode, self.lse_prefill,
                                    self.lse_decode, self.k_scale, self.v_scale)

    def run(self, stream=None):
        run(self.plan, self.tensors, stream)

    def run_events(self, before_fused, after_fused, stream=None):
        run_events(self.plan, self.tensors, before_fused, after_fused, stream)

    def sequential_run(self, stream=None):
        sequential_run(self.plan, self.tensors, stream)

    def streams_run(self, decode_stream, stream=None):
        streams_run(self.plan, self.tensors, decode_stream, stream)

    def batched_prefill_run(self, stream=None):
        batched_prefill_run(self.plan, self.tensors, stream)

    def outputs(self):
        """Host copies: O as float64 (from bf16) and LSE as float64."""
        import torch
        return {
            "o_prefill": self.o_prefill.float().cpu().double().numpy(),
            "lse_prefill": self.lse_prefill.cpu().double().numpy(),
            "o_decode": self.o_decode.float().cpu().double().numpy(),
            "lse_decode": self.lse_decode.cpu().double().numpy(),
        }
