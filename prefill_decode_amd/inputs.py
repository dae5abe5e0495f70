"""Seeded synthetic hybrid batches (inputs only; none of the attention math).

This module is the one piece shared by the GPU library's tests/bench and the
CPU oracle: it draws request lengths, the paged-KV page table and the bf16
bit patterns of Q, K and V.  It computes nothing of the method itself.

Workloads (shapes of the hybrid batches the summary of "POD-Attention:
Unlocking Full Prefill-Decode Overlap for Faster LLM Inference" evaluates in
"The evaluation": contexts 4K-20K, prefill chunks 512-2K, Llama-2-7B /
Llama-3-8B-shaped layers).  No dataset is involved; every value is synthetic:

* ``tiny``      8 q / 8 kv heads; one causal chunk of 128 tokens at kv 384;
                4 decodes at kv 512; contiguous KV.
* ``llama3_8b`` 32/8; chunk 1024 at kv 4096; 64 decodes, kv ~ U[1024, 4096];
                paged (16-token pages, seeded random page order).
* ``llama2_7b`` 32/32 (MHA); chunk 512 at kv 12288; 128 decodes at kv 8192;
                paged.
* ``l70b_tp1``  64/8; chunk 2048 at kv 16384; 256 decodes, kv lognormal
                (median 4096, sigma 1, capped at 32768); paged.
* ``batched``   32/8; 4 chunks {128, 256, 512, 640} at kv ~ U[2048, 8192];
                192 decodes at kv ~ U[512, 16384]; paged.  ``n_dec`` sweeps
                {32, 64, 128, 256}.
* ``l70b_prefix`` 64/8, decode-only with shared prefixes (the workload class
                of [PAT]'s abstract: system prompts, templates, RAG shared
                across requests): 128 decodes in 16 groups of 8, each group
                sharing a 2048-token prefix (the same pages), each request
                with its own ~ U[64, 1024] tokens after it; paged.

Conventions: request order is all prefill requests, then all decodes;
``uniform in [a, b]`` is integers with both ends included; Q/K/V values are
i.i.d. N(0, 1) drawn in float32 and rounded to bfloat16 (nearest-even).

FP8 KV caches (``kv_dtype="fp8_e4m3"``, any batch): K and V are
drawn the same way in float32, each KV head gets the scale max|x| / 448 over
its pool (float32), and the cache holds x / scale encoded as OCP FP8 E4M3
(nearest, ties to even) -- so that the largest value of a head is the format's
largest finite value.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

HEAD_DIM = 128
PAGE_SIZE = 16
BF16_NAN = 0x7FC0
FP8_NAN = 0x7F              # E4M3: S.1111.111 is the only NaN pattern
FP8_MAX = 448.0

# rng stream tags
_TAG_LEN, _TAG_PAGES, _TAG_QP, _TAG_K, _TAG_V, _TAG_QD = 0, 1, 2, 3, 4, 5
_CHUNK_PAGES = 4096


@dataclass(frozen=True)
class BatchSpec:
    name: str
    num_qo_heads: int
    num_kv_heads: int
    prefill_qo_len: Tuple[int, ...]
    prefill_kv_len: Tuple[int, ...]
    decode_kv_len: Tuple[int, ...]
    layout: str = "paged"            # "paged" | "contiguous"
    page_size: int = PAGE_SIZE
    causal: bool = True
    sm_scale: float = 1.0 / math.sqrt(HEAD_DIM)
    seed: int = 0
    head_dim: int = HEAD_DIM
    random_pages: bool = True
    extra_pages: int = 3             # unreferenced pool pages (poisoned)
    kv_dtype: str = "bf16"           # "bf16" | "fp8_e4m3"
    # decode requests sharing a KV prefix: ((decode ids, prefix tokens), ..);
    # the members' first prefix tokens are the same pages (prefix tokens are
    # a multiple of page_size)
    prefix_groups: Tuple = ()

    @property
    def num_prefill(self) -> int:
        return len(self.prefill_qo_len)

    @property
    def num_decode(self) -> int:
        return len(self.decode_kv_len)

    @property
    def kv_lens(self) -> Tuple[int, ...]:
        return tuple(self.prefill_kv_len) + tuple(self.decode_kv_len)

    def num_pages_of(self, kv_len: int) -> int:
        return -(-kv_len // self.page_size)


CONFIG_NAMES = ("tiny", "llama3_8b", "llama2_7b", "l70b_tp1", "batched")


def config_spec(name: str, n_dec: Optional[int] = None) -> BatchSpec:
    """The five workload shapes (module docstring), lengths drawn from their
    seeds.  ``n_dec`` (``batched`` only) selects a point of the decode-count
    sweep.  A name ending in ``_fp8`` gives that workload with an FP8 E4M3
    cache."""
    if name.endswith("_fp8"):
        base = config_spec(name[:-4], n_dec)
        return replace(base, name=base.name + "_fp8", kv_dtype="fp8_e4m3")
    if name == "tiny":
        return BatchSpec(name, 8, 8, (128,), (384,), (512,) * 4,
                         layout="contiguous", seed=1234, extra_pages=0)
    if name == "llama3_8b":
        seed = 1235
        rng = np.random.default_rng([seed, _TAG_LEN])
        dec = rng.integers(1024, 4096, size=64, endpoint=True)
        return BatchSpec(name, 32, 8, (1024,), (4096,), tuple(int(x) for x in dec),
                         seed=seed)
    if name == "llama2_7b":
        return BatchSpec(name, 32, 32, (512,), (12288,), (8192,) * 128, seed=1236)
    if name == "l70b_tp1":
        seed = 1237
        rng = np.random.default_rng([seed, _TAG_LEN])
        z = rng.standard_normal(256)
        dec = np.clip(np.rint(4096.0 * np.exp(z)), 1, 32768).astype(np.int64)
        return BatchSpec(name, 64, 8, (2048,), (16384,), tuple(int(x) for x in dec),
                         seed=seed)
    if name == "batched":
        nd = 192 if n_dec is None else int(n_dec)
        seed = 1238 if n_dec is None else 1238 + 1000 * nd
        rng = np.random.default_rng([seed, _TAG_LEN])
        pkv = rng.integers(2048, 8192, size=4, endpoint=True)
        dec = rng.integers(512, 16384, size=nd, endpoint=True)
        return BatchSpec(name if n_dec is None else f"batched_d{nd}", 32, 8,
                         (128, 256, 512, 640), tuple(int(x) for x in pkv),
                         tuple(int(x) for x in dec), seed=seed)
    if name == "l70b_prefix":
        seed = 1239
        rng = np.random.default_rng([seed, _TAG_LEN])
        own = rng.integers(64, 1024, size=128, endpoint=True)
        groups = tuple((tuple(range(8 * g, 8 * g + 8)), 2048) for g in range(16))
        return BatchSpec(name, 64, 8, (), (), tuple(2048 + int(x) for x in own), seed=seed,
                         prefix_groups=groups)
    raise ValueError(f"unknown config {name!r}")


def fp8_spec(name: str) -> BatchSpec:
    """Workload ``name`` with an FP8 E4M3 KV cache (same lengths and seed)."""
    return config_spec(name + "_fp8")


def decode_only_spec(name: str, kv_dtype: str = "bf16") -> BatchSpec:
    """The decodes of workload ``name`` alone (its prefill dropped), with a
    bf16 or an FP8 E4M3 cache."""
    base = config_spec(name)
    suffix = "_dec_fp8" if kv_dtype == "fp8_e4m3" else "_dec_bf16"
    return replace(base, name=base.name + suffix, prefill_qo_len=(), prefill_kv_len=(),
                   kv_dtype=kv_dtype)


def custom_spec(name: str, num_qo_heads: int, num_kv_heads: int,
                prefill: Sequence[Tuple[int, int]], decode_kv: Sequence[int],
                seed: int, **kw) -> BatchSpec:
    """A spec with explicit (qo_len, kv_len) prefill pairs and decode kv
    lengths (used for reduced-size parity cases and edge cases)."""
    return BatchSpec(name, num_qo_heads, num_kv_heads,
                     tuple(int(a) for a, _ in prefill), tuple(int(b) for _, b in prefill),
                     tuple(int(x) for x in decode_kv), seed=seed, **kw)


def with_scale(spec: BatchSpec, sm_scale: float, suffix: str = "_sharp") -> BatchSpec:
    return replace(spec, sm_scale=float(sm_scale), name=spec.name + suffix)


# ---------------------------------------------------------------------------
# bit-level helpers (input encoding, not attention arithmetic)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); finite inputs."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _fp8_e4m3_code_values() -> np.ndarray:
    """Values of the non-negative finite E4M3 codes 0x00 .. 0x7E, in code
    order (which is increasing order): exponent field 0 gives m * 2^-9,
    otherwise (1 + m/8) * 2^(e - 7)."""
    codes = np.arange(0x7F)
    e, m = codes >> 3, codes & 7
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))


_FP8_VALUES = _fp8_e4m3_code_values()


def f32_to_fp8_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Encode finite values with |x| <= 448 as E4M3 bytes, rounding to the
    nearest code and, on a tie, to the code with an even mantissa."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > FP8_MAX) or not np.all(np.isfinite(x)):
        raise ValueError("value outside the E4M3 range")
    v = _FP8_VALUES
    i = np.clip(np.searchsorted(v, a, side="left"), 1, len(v) - 1)   # v[i-1] < a <= v[i]
    lo, hi = v[i - 1], v[i]
    pick_hi = (a - lo > hi - a) | ((a - lo == hi - a) & (i % 2 == 0))
    code = np.where(a <= v[0], 0, np.where(pick_hi, i, i - 1)).astype(np.uint8)
    return (code | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)).astype(np.uint8)


def _fp8_pool(seed: int, tag: int, shape, chunk: int):
    """(E4M3 bytes, per-KV-head float32 scales) of an N(0, 1) float32 pool of
    shape [..., Hkv, d] drawn as the bf16 pools are."""
    lead = shape[0]
    x = np.empty(shape, dtype=np.float32)
    for c0 in range(0, lead, chunk):
        c1 = min(lead, c0 + chunk)
        rng = np.random.default_rng([seed, tag, c0 // chunk])
        x[c0:c1] = rng.standard_normal((c1 - c0,) + tuple(shape[1:]), dtype=np.float32)
    axes = tuple(range(x.ndim - 2)) + (x.ndim - 1,)
    scale = (np.max(np.abs(x), axis=axes) / np.float32(FP8_MAX)).astype(np.float32)
    # x / scale of a head's largest |x| rounds to 448 give or take an ulp
    return f32_to_fp8_e4m3_bits(np.clip(x / scale[:, None], -FP8_MAX, FP8_MAX)), scale


def _normal_bf16(seed: int, tag: int, shape, chunk: Optional[int] = None) -> np.ndarray:
    if chunk is None:
        rng = np.random.default_rng([seed, tag])
        return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    out = np.empty(shape, dtype=np.uint16)
    lead = shape[0]
    for c0 in range(0, lead, chunk):
        c1 = min(lead, c0 + chunk)
        rng = np.random.default_rng([seed, tag, c0 // chunk])
        out[c0:c1] = f32_to_bf16_bits(
            rng.standard_normal((c1 - c0,) + tuple(shape[1:]), dtype=np.float32))
    return out


def page_table(spec: BatchSpec):
    """(page_indptr [R+1] int32, page_indices [sum pages] int32, pool_pages).

    Pages are handed out in request order from a seeded permutation of the
    pool (or in order when ``random_pages`` is False); ``extra_pages``
    pool pages are referenced by no request.  A decode request of a prefix
    group starts with the group's shared prefix pages (handed out once, at the
    group's first member) and continues with pages of its own."""
    n_p = spec.num_prefill
    ps = spec.page_size
    shared_of = {}                      # decode id -> (group, prefix pages)
    for gi, (members, plen) in enumerate(spec.prefix_groups):
        if plen % ps or plen < 1:
            raise ValueError("a shared prefix is a positive whole number of pages")
        for m in members:
            if spec.decode_kv_len[m] < plen:
                raise ValueError("a member is shorter than its group's prefix")
            shared_of[int(m)] = (gi, plen // ps)
    npg = [spec.num_pages_of(L) for L in spec.kv_lens]
    own = list(npg)
    groups_seen = set()
    for m, (gi, pp) in shared_of.items():
        own[n_p + m] -= pp
        if gi not in groups_seen:
            groups_seen.add(gi)
            own[n_p + m] += pp           # the first member seen allocates them
    total = int(sum(own))
    pool = total + spec.extra_pages
    if spec.random_pages:
        perm = np.random.default_rng([spec.seed, _TAG_PAGES]).permutation(pool)
    else:
        perm = np.arange(pool)
    indptr = np.zeros(len(npg) + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(npg)
    indices = np.empty(int(indptr[-1]), dtype=np.int32)
    nxt = 0
    group_pages = {}
    for r, n in enumerate(npg):
        out = indices[indptr[r]:indptr[r + 1]]
        sh = shared_of.get(r - n_p) if r >= n_p else None
        k = 0
        if sh is not None:
            gi, pp = sh
            if gi not in group_pages:
                group_pages[gi] = perm[nxt:nxt + pp].astype(np.int32)
                nxt += pp
            out[:pp] = group_pages[gi]
            k = pp
        out[k:] = perm[nxt:nxt + (n - k)]
        nxt += n - k
    assert nxt == total
    return indptr, indices, pool


def _base_dict(spec: BatchSpec) -> Dict:
    return {
        "name": spec.name,
        "num_qo_heads": spec.num_qo_heads,
        "num_kv_heads": spec.num_kv_heads,
        "head_dim": spec.head_dim,
        "layout": spec.layout,
        "page_size": spec.page_size,
        "causal": spec.causal,
        "sm_scale": spec.sm_scale,
        "kv_dtype": spec.kv_dtype,
        "prefix_groups": spec.prefix_groups,
        "prefill_qo_len": np.array(spec.prefill_qo_len, dtype=np.int32),
        "prefill_kv_len": np.array(spec.prefill_kv_len, dtype=np.int32),
        "decode_kv_len": np.array(spec.decode_kv_len, dtype=np.int32),
    }


def make_batch_host(spec: BatchSpec, poison: bool = True) -> Dict:
    """A hybrid batch as host numpy arrays (bf16 as uint16 bit patterns).

    Keys: q_prefill [sum qo, Hq, d], q_decode [n_dec, Hq, d], k_cache and
    v_cache ([pool, page_size, Hkv, d] paged, or [sum kv, Hkv, d]
    contiguous), page_indptr/page_indices (paged) or kv_indptr
    (contiguous), plus the spec's scalars and lengths.  An FP8 batch holds
    E4M3 bytes (uint8) in k_cache / v_cache and float32 k_scale / v_scale
    [Hkv].  With ``poison``, KV slots that belong to no token (tails of last
    pages, unreferenced pages) hold NaN so that a reader of them is caught.
    """
    b = _base_dict(spec)
    hq, hkv, d = spec.num_qo_heads, spec.num_kv_heads, spec.head_dim
    sum_qo = int(sum(spec.prefill_qo_len))
    fp8 = spec.kv_dtype == "fp8_e4m3"
    nan = FP8_NAN if fp8 else BF16_NAN
    b["q_prefill"] = _normal_bf16(spec.seed, _TAG_QP, (sum_qo, hq, d))
    b["q_decode"] = _normal_bf16(spec.seed, _TAG_QD, (spec.num_decode, hq, d))

    def pools(shape, chunk):
        if fp8:
            b["k_cache"], b["k_scale"] = _fp8_pool(spec.seed, _TAG_K, shape, chunk)
            b["v_cache"], b["v_scale"] = _fp8_pool(spec.seed, _TAG_V, shape, chunk)
        else:
            b["k_cache"] = _normal_bf16(spec.seed, _TAG_K, shape, chunk=chunk)
            b["v_cache"] = _normal_bf16(spec.seed, _TAG_V, shape, chunk=chunk)

    if spec.layout == "contiguous":
        lens = np.array(spec.kv_lens, dtype=np.int64)
        indptr = np.zeros(len(lens) + 1, dtype=np.int32)
        indptr[1:] = np.cumsum(lens)
        n = int(indptr[-1])
        b["kv_indptr"] = indptr
        pools((n, hkv, d), 65536)
        return b
    indptr, indices, pool = page_table(spec)
    ps = spec.page_size
    b["page_indptr"] = indptr
    b["page_indices"] = indices
    pools((pool, ps, hkv, d), _CHUNK_PAGES)
    if poison:
        used = np.zeros(pool, dtype=bool)
        used[indices] = True
        b["k_cache"][~used] = nan
        b["v_cache"][~used] = nan
        for r, L in enumerate(spec.kv_lens):
            tail = L % ps
            if tail:
                last = indices[indptr[r + 1] - 1]
                b["k_cache"][last, tail:] = nan
                b["v_cache"][last, tail:] = nan
    return b


# ---------------------------------------------------------------------------
# Full-size batches generated on the device (torch's seeded generator) and a
# host copy of selected requests for the oracle.
# ---------------------------------------------------------------------------

def make_batch_device(spec: BatchSpec, device="cuda", poison: bool = False) -> Dict:
    """The same structure as :func:`make_batch_host`, with Q/K/V drawn on
    the device by torch's seeded generator (N(0,1) float32 rounded to
    bfloat16) and stored as torch.bfloat16 device tensors.  Page tables and
    lengths are the host arrays of :func:`page_table`.  Used for full-size
    workloads whose KV pool is too large to draw on the host."""
    import torch

    b = _base_dict(spec)
    hq, hkv, d = spec.num_qo_heads, spec.num_kv_heads, spec.head_dim
    gen = torch.Generator(device=device)

    def normal(tag, shape, chunk_rows=None):
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
        lead = shape[0]
        step = lead if not chunk_rows else chunk_rows
        for c0 in range(0, lead, max(1, step)):
            c1 = min(lead, c0 + step)
            gen.manual_seed(int(spec.seed) * 1000003 + tag * 7919 + c0 // max(1, step))
            out[c0:c1] = torch.randn((c1 - c0,) + tuple(shape[1:]), generator=gen,
                                     dtype=torch.float32, device=device).to(torch.bfloat16)
        return out

    def fp8_pool(tag, shape, chunk_rows):
        # float32 draws as for bf16, per-KV-head scale max|x| / 448, then
        # torch's E4M3 conversion (nearest, ties to even) of x / scale
        x = torch.empty(shape, dtype=torch.float32, device=device)
        for c0 in range(0, shape[0], chunk_rows):
            c1 = min(shape[0], c0 + chunk_rows)
            gen.manual_seed(int(spec.seed) * 1000003 + tag * 7919 + c0 // chunk_rows)
            x[c0:c1] = torch.randn((c1 - c0,) + tuple(shape[1:]), generator=gen,
                                   dtype=torch.float32, device=device)
        dims = tuple(range(x.dim() - 2)) + (x.dim() - 1,)
        scale = (x.abs().amax(dim=dims) / FP8_MAX).float()
        q = (x / scale[:, None]).clamp_(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn) \
            .view(torch.uint8)
        del x
        return q, scale

    sum_qo = int(sum(spec.prefill_qo_len))
    fp8 = spec.kv_dtype == "fp8_e4m3"
    b["q_prefill"] = normal(_TAG_QP, (sum_qo, hq, d))
    b["q_decode"] = normal(_TAG_QD, (spec.num_decode, hq, d))

    def pools(shape, chunk_rows):
        if fp8:
            b["k_cache"], b["k_scale"] = fp8_pool(_TAG_K, shape, chunk_rows)
            b["v_cache"], b["v_scale"] = fp8_pool(_TAG_V, shape, chunk_rows)
        else:
            b["k_cache"] = normal(_TAG_K, shape, chunk_rows)
            b["v_cache"] = normal(_TAG_V, shape, chunk_rows)

    if spec.layout == "contiguous":
        lens = np.array(spec.kv_lens, dtype=np.int64)
        indptr = np.zeros(len(lens) + 1, dtype=np.int32)
        indptr[1:] = np.cumsum(lens)
        b["kv_indptr"] = indptr
        n = int(indptr[-1])
        pools((n, hkv, d), 1 << 18)
        return b
    indptr, indices, pool = page_table(spec)
    b["page_indptr"] = indptr
    b["page_indices"] = indices
    pools((pool, spec.page_size, hkv, d), 16384)
    if poison:
        nan = torch.tensor(FP8_NAN, dtype=torch.uint8, device=device) if fp8 else \
            torch.tensor(float("nan"), dtype=torch.bfloat16, device=device)
        used = np.zeros(pool, dtype=bool)
        used[indices] = True
        unused = torch.from_numpy(np.nonzero(~used)[0]).to(device)
        if unused.numel():
            b["k_cache"][unused] = nan
            b["v_cache"][unused] = nan
        for r, L in enumerate(spec.kv_lens):
            tail = L % spec.page_size
            if tail:
                last = int(indices[indptr[r + 1] - 1])
                b["k_cache"][last, tail:] = nan
                b["v_cache"][last, tail:] = nan
    return b


def host_subset(batch_dev: Dict, prefill_ids: Sequence[int],
                decode_ids: Sequence[int]) -> Dict:
    """Host (uint16-bits) copy of a device batch restricted to the listed
    prefill requests and decode requests, with a compacted page pool, for
    the oracle.  Row and request order follow the given id lists."""
    import torch

    spec_keys = ["name", "num_qo_heads", "num_kv_heads", "head_dim", "layout",
                 "page_size", "causal", "sm_scale"]
    out = {k: batch_dev[k] for k in spec_keys}
    out["kv_dtype"] = batch_dev.get("kv_dtype", "bf16")
    for key in ("k_scale", "v_scale"):
        if key in batch_dev:
            v = batch_dev[key]
            out[key] = v.cpu().numpy() if hasattr(v, "cpu") else np.asarray(v)
    pqo = np.asarray(batch_dev["prefill_qo_len"])
    pkv = np.asarray(batch_dev["prefill_kv_len"])
    dkv = np.asarray(batch_dev["decode_kv_len"])
    n_p = len(pqo)
    offs = np.concatenate([[0], np.cumsum(pqo)])
    prefill_ids = [int(x) for x in prefill_ids]
    decode_ids = [int(x) for x in decode_ids]
    out["prefill_qo_len"] = pqo[prefill_ids].astype(np.int32)
    out["prefill_kv_len"] = pkv[prefill_ids].astype(np.int32)
    out["decode_kv_len"] = dkv[decode_ids].astype(np.int32)

    def bits(t):
        if t.dtype == torch.uint8:
            return t.contiguous().cpu().numpy()
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    qp = [bits(batch_dev["q_prefill"][int(offs[r]):int(offs[r + 1])]) for r in prefill_ids]
    hq, d = out["num_qo_heads"], out["head_dim"]
    out["q_prefill"] = np.concatenate(qp) if qp else np.zeros((0, hq, d), np.uint16)
    out["q_decode"] = bits(batch_dev["q_decode"][torch.tensor(decode_ids, dtype=torch.long)]) \
        if decode_ids else np.zeros((0, hq, d), np.uint16)
    reqs = prefill_ids + [n_p + i for i in decode_ids]
    if batch_dev["layout"] == "contiguous":
        ip = np.asarray(batch_dev["kv_indptr"])
        ks, vs, new_ip = [], [], [0]
        for r in reqs:
            ks.append(bits(batch_dev["k_cache"][int(ip[r]):int(ip[r + 1])]))
            vs.append(bits(batch_dev["v_cache"][int(ip[r]):int(ip[r + 1])]))
            new_ip.append(new_ip[-1] + int(ip[r + 1] - ip[r]))
        out["kv_indptr"] = np.array(new_ip, dtype=np.int32)
        out["k_cache"] = np.concatenate(ks)
        out["v_cache"] = np.concatenate(vs)
        return out
    ip = np.asarray(batch_dev["page_indptr"])
    idx = np.asarray(batch_dev["page_indices"])
    sel, new_ip = [], [0]
    for r in reqs:
        pg = idx[int(ip[r]):int(ip[r + 1])]
        sel.append(pg)
        new_ip.append(new_ip[-1] + len(pg))
    sel = np.concatenate(sel) if sel else np.zeros(0, np.int64)
    ti = torch.from_numpy(sel.astype(np.int64)).to(batch_dev["k_cache"].device)
    out["page_indptr"] = np.array(new_ip, dtype=np.int32)
    out["page_indices"] = np.arange(len(sel), dtype=np.int32)
    out["k_cache"] = bits(batch_dev["k_cache"][ti])
    out["v_cache"] = bits(batch_dev["v_cache"][ti])
    return out


def to_device(batch: Dict, device="cuda") -> Dict:
    """Copy a host batch's bit arrays to device torch.bfloat16 tensors and
    its index tables to device int32 tensors (lengths stay on the host)."""
    import torch

    out = dict(batch)
    for key in ("q_prefill", "q_decode", "k_cache", "v_cache"):
        a = np.ascontiguousarray(batch[key])
        if a.dtype == np.uint8:
            out[key] = torch.from_numpy(a).to(device)
        else:
            out[key] = torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    for key in ("k_scale", "v_scale"):
        if key in batch:
            out[key] = torch.from_numpy(np.ascontiguousarray(batch[key], np.float32)).to(device)
    return out
