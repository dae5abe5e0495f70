"""Plain float64 attention over a hybrid (prefill + decode) batch.

TEST INFRASTRUCTURE (see the package docstring): only tests, ``smoke()`` and
the bench's ``cpu_baseline`` leg may use it.

What is computed ([POD] "Why this problem is worth solving": each query token
takes a weighted combination of the keys and values of all earlier tokens in
the KV-cache; [POD] "The argument in one glance": prefill chunks and decode
tokens of one hybrid batch).  The pages give no formula; the oracle is the
textbook scaled-dot-product softmax attention, written out directly:

    for request r, query head h, query row i:
        kvh   = h // (Hq / Hkv)                          (reading R2)
        pos_i = kv_len_r - qo_len_r + i                  (reading R1)
        V_i   = {0..pos_i} if causal else {0..kv_len_r-1}
        s_ij  = sm_scale * <q_ih, k_j,kvh>               (reading R3)
        m_i   = max_{j in V_i} s_ij
        l_i   = sum_{j in V_i} exp(s_ij - m_i)
        O_ih  = sum_{j in V_i} exp(s_ij - m_i) * v_j,kvh / l_i
        LSE_ih = m_i + ln(l_i)                            (reading R4)

Readings of the pages (they are silent on each point):

* R1  causal alignment is bottom-right: a chunk of qo new tokens sits at the
      end of its kv_len-token context, so row i is absolute position
      kv_len - qo + i; a decode token is the qo = 1 case and sees all kv_len
      keys.
* R2  grouped-query heads map to KV heads in contiguous groups:
      kvh = h // (Hq / Hkv).
* R3  sm_scale multiplies the fp64 score; nothing is folded into Q.
* R4  LSE is the natural-log log-sum-exp of the *scaled* scores.
* R5  a split restricted to keys [b, e) with no visible key has O = 0 and
      LSE = -inf and carries zero weight in the merge.
* R6  an FP8 KV cache ("Prefill vs. Decode GPU Utilization Imbalance",
      section on quantization as a lever on the bandwidth and capacity
      problem, names quantized KV caches without fixing a format) holds OCP
      FP8 E4M3 bytes with one float32 scale per KV head for K and one for V:
      the key or value is the decoded byte times its head's scale, and the
      attention is that of the decoded values.

No online softmax, no tiling and no splitting is used in
:func:`attention_rows`; each row's softmax sees the whole row at once (max,
then exponentials and their sum).  A library matrix product is used for the
row-by-key score block and for the weighted sum of values.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# Element conversion
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bfloat16 bit patterns (uint16) to float64.

    A bfloat16 value is the upper 16 bits of an IEEE binary32 value, so
    shifting the pattern into the high half of a uint32 and reinterpreting it
    as float32 is exact; float32 -> float64 is exact too.
    """
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("expected uint16 bfloat16 bit patterns")
    f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def fp8_e4m3_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of OCP FP8 E4M3 bytes (uint8), from the format's
    definition: sign bit, 4 exponent bits with bias 7, 3 mantissa bits; an
    exponent field of 0 is subnormal (mantissa * 2^-6 / 8); S.1111.111 is NaN
    and the format has no infinities (reading R6)."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint8:
        raise TypeError("expected uint8 E4M3 bytes")
    b = bits.astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 0xF) & (m == 7), np.nan, mag)
    return sign * mag


# ---------------------------------------------------------------------------
# Small definitional helpers (kept separate so planted-mistake tests can
# replace them one at a time)
# ---------------------------------------------------------------------------

def kv_head_of(h: int, num_qo_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head ``h`` (reading R2: contiguous groups)."""
    group = num_qo_heads // num_kv_heads
    return h // group


def visible_key_count(pos: int, kv_len: int, causal: bool) -> int:
    """Number of keys visible to a query at absolute position ``pos``.

    Causal: keys 0..pos (reading R1); otherwise all ``kv_len`` keys.
    """
    if causal:
        return min(pos + 1, kv_len)
    return kv_len


def _row_positions(qo_len: int, kv_len: int) -> np.ndarray:
    """Absolute positions of a chunk's qo_len query rows (reading R1)."""
    return np.arange(kv_len - qo_len, kv_len, dtype=np.int64)


def _scores(q_h: np.ndarray, k_h: np.ndarray, sm_scale: float) -> np.ndarray:
    """s[i, j] = sm_scale * <q_i, k_j> for one head (reading R3)."""
    return sm_scale * (q_h @ k_h.T)


def _lse(m: np.ndarray, l: np.ndarray) -> np.ndarray:
    """Natural-log log-sum-exp from the row max and the shifted sum (R4)."""
    return m + np.log(l)


# ---------------------------------------------------------------------------
# Core definition
# ---------------------------------------------------------------------------

def attention_rows(q: np.ndarray, q_pos: Sequence[int], k: np.ndarray,
                   v: np.ndarray, causal: bool, sm_scale: float,
                   key_begin: int = 0, key_end: Optional[int] = None,
                   return_probs: bool = False):
    """Attention of query rows at absolute positions ``q_pos`` over one
    request's keys.

    Args:
      q:      float64 [n, Hq, d] query rows.
      q_pos:  [n] absolute position of each row in the request's sequence.
      k, v:   float64 [kv_len, Hkv, d] the request's keys and values.
      causal: bottom-right causal visibility (reading R1).
      sm_scale: score scale (reading R3).
      key_begin, key_end: restrict the softmax to keys in [key_begin,
        key_end) intersected with the visible set (a KV split).  The default
        is all keys.
      return_probs: also return the [n, Hq, kv_len] probability matrix.

    Returns (O [n, Hq, d] float64, LSE [n, Hq] float64[, P]).  Rows whose
    restricted visible set is empty get O = 0 and LSE = -inf (reading R5).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, hq, d = q.shape
    kv_len, hkv, dk = k.shape
    assert dk == d and v.shape == k.shape
    if key_end is None:
        key_end = kv_len
    key_begin = max(0, key_begin)
    key_end = min(kv_len, key_end)
    q_pos = np.asarray(q_pos, dtype=np.int64).reshape(n)

    o = np.zeros((n, hq, d), dtype=np.float64)
    lse = np.full((n, hq), NEG_INF, dtype=np.float64)
    probs = np.zeros((n, hq, kv_len), dtype=np.float64) if return_probs else None

    # visible[i, j]: key j in the softmax of row i
    vis_cnt = np.array([visible_key_count(int(p), kv_len, causal) for p in q_pos],
                       dtype=np.int64)
    j = np.arange(kv_len, dtype=np.int64)
    visible = (j[None, :] < vis_cnt[:, None]) & (j[None, :] >= key_begin) & \
              (j[None, :] < key_end)
    any_visible = visible.any(axis=1)

    for h in range(hq):
        kvh = kv_head_of(h, hq, hkv)
        s = _scores(q[:, h, :], k[:, kvh, :], sm_scale)        # [n, kv_len]
        s = np.where(visible, s, NEG_INF)
        m = np.max(s, axis=1)                                   # [n]
        m_safe = np.where(any_visible, m, 0.0)
        e = np.exp(s - m_safe[:, None])                         # exp(-inf) = 0
        l = np.sum(e, axis=1)
        ok = any_visible
        p = np.zeros_like(e)
        p[ok] = e[ok] / l[ok, None]
        o[:, h, :] = p @ v[:, kvh, :]
        lse[ok, h] = _lse(m[ok], l[ok])
        if return_probs:
            probs[:, h, :] = p
    if return_probs:
        return o, lse, probs
    return o, lse


def attention_partial(q, q_pos, k, v, causal, sm_scale, key_begin, key_end):
    """One KV split's partial (O, LSE): the softmax restricted to keys in
    [key_begin, key_end) ([POD] "Cap prefill splitting to avoid contention":
    splitting along the KV dimension).  Empty splits give (0, -inf)."""
    return attention_rows(q, q_pos, k, v, causal, sm_scale,
                          key_begin=key_begin, key_end=key_end)


def merge_partials(parts: Sequence[Tuple[np.ndarray, np.ndarray]]):
    """Combine split partials by log-sum-exp ([PAT] abstract: the final
    merge is an online-softmax combination of the partial results).

        LSE = M + ln sum_s exp(LSE_s - M),   M = max_s LSE_s
        O   = sum_s exp(LSE_s - LSE) * O_s

    Partials with LSE_s = -inf have weight zero.  If every partial is
    -inf the result is (0, -inf).
    """
    lses = np.stack([np.asarray(p[1], dtype=np.float64) for p in parts])   # [S, ...]
    os_ = np.stack([np.asarray(p[0], dtype=np.float64) for p in parts])    # [S, ..., d]
    m = np.max(lses, axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.exp(lses - m_safe[None])                                        # 0 for -inf
    tot = np.sum(w, axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, tot, 1.0)), NEG_INF)
    scale = np.where(finite[None], np.exp(lses - np.where(finite, lse, 0.0)[None]), 0.0)
    o = np.sum(scale[..., None] * os_, axis=0)
    return o, lse


# ---------------------------------------------------------------------------
# Batch level: gather each request's KV from the cache (own code, not shared
# with the GPU library) and apply the definition.
# ---------------------------------------------------------------------------

def gather_request_kv(batch: Dict, r: int, kv_len: int,
                      tokens: Optional[np.ndarray] = None):
    """Keys and values (float64 [kv_len, Hkv, d]) of request ``r`` (prefill
    requests first, then decodes) read from the batch's KV cache (bfloat16,
    or FP8 E4M3 bytes with per-KV-head scales, reading R6).

    Contiguous layout: rows kv_indptr[r] .. kv_indptr[r] + kv_len.
    Paged layout: the request's pages page_indices[page_indptr[r]:...] in
    order, page_size tokens each; token t lives in page t // page_size at
    slot t % page_size.
    """
    kc, vc = batch["k_cache"], batch["v_cache"]
    if tokens is None:
        tokens = np.arange(kv_len, dtype=np.int64)
    if batch["layout"] == "contiguous":
        rows = int(batch["kv_indptr"][r]) + tokens
        k = kc[rows]
        v = vc[rows]
    else:
        ps = int(batch["page_size"])
        pages = batch["page_indices"][int(batch["page_indptr"][r]):
                                      int(batch["page_indptr"][r + 1])]
        pg = pages[tokens // ps].astype(np.int64)
        sl = tokens % ps
        k = kc[pg, sl]
        v = vc[pg, sl]
    if batch.get("kv_dtype", "bf16") == "fp8_e4m3":
        # reading R6: decoded byte times the KV head's scale
        ks = np.asarray(batch["k_scale"], dtype=np.float64)
        vs = np.asarray(batch["v_scale"], dtype=np.float64)
        return (fp8_e4m3_bits_to_f64(k) * ks[None, :, None],
                fp8_e4m3_bits_to_f64(v) * vs[None, :, None])
    return bf16_bits_to_f64(k), bf16_bits_to_f64(v)


def _default_workers() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _run_jobs(jobs, workers):
    if workers <= 1 or len(jobs) <= 1:
        return [j() for j in jobs]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        futs = [ex.submit(j) for j in jobs]
        return [f.result() for f in futs]


def _prefill_offsets(batch):
    qo = np.asarray(batch["prefill_qo_len"], dtype=np.int64)
    return np.concatenate([[0], np.cumsum(qo)])


def _request_of_row(offs: np.ndarray, g: int) -> int:
    """Prefill request holding global query row ``g``: the r with
    offs[r] <= g < offs[r + 1] (``offs`` = [0, qo_0, qo_0 + qo_1, ...]).  A
    chunk's first row belongs to that chunk, not to the one before it."""
    return int(np.searchsorted(offs, g, side="right") - 1)


def batch_attention(batch: Dict, workers: Optional[int] = None,
                    row_block: int = 256) -> Dict[str, np.ndarray]:
    """Oracle outputs for every row of a hybrid batch.

    Returns float64 ``o_prefill`` [sum qo, Hq, d], ``lse_prefill``
    [sum qo, Hq], ``o_decode`` [n_dec, Hq, d], ``lse_decode`` [n_dec, Hq].
    Work is spread over a thread pool by (request, row block); the
    arithmetic of every row is :func:`attention_rows`.
    """
    if workers is None:
        workers = _default_workers()
    hq, d = int(batch["num_qo_heads"]), int(batch["head_dim"])
    causal, scale = bool(batch["causal"]), float(batch["sm_scale"])
    qo = np.asarray(batch["prefill_qo_len"], dtype=np.int64)
    pkv = np.asarray(batch["prefill_kv_len"], dtype=np.int64)
    dkv = np.asarray(batch["decode_kv_len"], dtype=np.int64)
    offs = _prefill_offsets(batch)
    n_p, n_d = len(qo), len(dkv)

    out = {
        "o_prefill": np.zeros((int(offs[-1]), hq, d)),
        "lse_prefill": np.zeros((int(offs[-1]), hq)),
        "o_decode": np.zeros((n_d, hq, d)),
        "lse_decode": np.zeros((n_d, hq)),
    }
    kv_cache: Dict[int, Tuple[np.ndarray, np.ndarray]] = {}

    def kv_of(r, L):
        if r not in kv_cache:
            kv_cache[r] = gather_request_kv(batch, r, L)
        return kv_cache[r]

    # gather serially (cheap), compute in parallel
    jobs = []
    for r in range(n_p):
        k, v = kv_of(r, int(pkv[r]))
        pos_all = _row_positions(int(qo[r]), int(pkv[r]))
        for b0 in range(0, int(qo[r]), row_block):
            b1 = min(int(qo[r]), b0 + row_block)
            rows = slice(int(offs[r]) + b0, int(offs[r]) + b1)

            def job(rows=rows, pos=pos_all[b0:b1], k=k, v=v):
                qf = bf16_bits_to_f64(batch["q_prefill"][rows])
                o, l = attention_rows(qf, pos, k, v, causal, scale)
                out["o_prefill"][rows] = o
                out["lse_prefill"][rows] = l
            jobs.append(job)
    for i in range(n_d):
        r = n_p + i

        def job(i=i, r=r):
            L = int(dkv[i])
            k, v = gather_request_kv(batch, r, L)
            qf = bf16_bits_to_f64(batch["q_decode"][i:i + 1])
            o, l = attention_rows(qf, [L - 1], k, v, causal, scale)
            out["o_decode"][i] = o[0]
            out["lse_decode"][i] = l[0]
        jobs.append(job)
    _run_jobs(jobs, workers)
    return out


def sample_batch_attention(batch: Dict, prefill_rows: Sequence[int],
                           decode_ids: Sequence[int],
                           workers: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Oracle outputs for a sample of rows only (for full-size batches).

    ``prefill_rows`` are global row indices into ``q_prefill``;
    ``decode_ids`` index the decode requests.  Each sampled row is computed
    by :func:`attention_rows` exactly as in :func:`batch_attention`.
    """
    if workers is None:
        workers = _default_workers()
    hq, d = int(batch["num_qo_heads"]), int(batch["head_dim"])
    causal, scale = bool(batch["causal"]), float(batch["sm_scale"])
    qo = np.asarray(batch["prefill_qo_len"], dtype=np.int64)
    pkv = np.asarray(batch["prefill_kv_len"], dtype=np.int64)
    dkv = np.asarray(batch["decode_kv_len"], dtype=np.int64)
    offs = _prefill_offsets(batch)
    n_p = len(qo)
    prefill_rows = [int(x) for x in prefill_rows]
    decode_ids = [int(x) for x in decode_ids]
    if any(g < 0 or g >= offs[-1] for g in prefill_rows) or \
            any(i < 0 or i >= len(dkv) for i in decode_ids):
        raise ValueError("sampled row or decode id out of range")
    res_p = {}
    res_d = {}

    by_req: Dict[int, List[int]] = {}
    for g in prefill_rows:
        by_req.setdefault(_request_of_row(offs, g), []).append(g)

    jobs = []
    for r, rows in by_req.items():
        def job(r=r, rows=rows):
            k, v = gather_request_kv(batch, r, int(pkv[r]))
            pos_all = _row_positions(int(qo[r]), int(pkv[r]))
            pos = [int(pos_all[g - offs[r]]) for g in rows]
            qf = bf16_bits_to_f64(batch["q_prefill"][np.array(rows)])
            o, l = attention_rows(qf, pos, k, v, causal, scale)
            for t, g in enumerate(rows):
                res_p[g] = (o[t], l[t])
        jobs.append(job)
    for i in decode_ids:
        def job(i=i):
            L = int(dkv[i])
            k, v = gather_request_kv(batch, n_p + i, L)
            qf = bf16_bits_to_f64(batch["q_decode"][i:i + 1])
            o, l = attention_rows(qf, [L - 1], k, v, causal, scale)
            res_d[i] = (o[0], l[0])
        jobs.append(job)
    _run_jobs(jobs, workers)
    out = {
        "prefill_rows": np.array(prefill_rows, dtype=np.int64),
        "o_prefill": np.stack([res_p[g][0] for g in prefill_rows]) if prefill_rows
        else np.zeros((0, hq, d)),
        "lse_prefill": np.stack([res_p[g][1] for g in prefill_rows]) if prefill_rows
        else np.zeros((0, hq)),
        "decode_ids": np.array(decode_ids, dtype=np.int64),
        "o_decode": np.stack([res_d[i][0] for i in decode_ids]) if decode_ids
        else np.zeros((0, hq, d)),
        "lse_decode": np.stack([res_d[i][1] for i in decode_ids]) if decode_ids
        else np.zeros((0, hq)),
    }
    return out
