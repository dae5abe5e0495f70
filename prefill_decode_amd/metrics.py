"""Algorithmic FLOP and byte counts of one hybrid batch (for the roofline).

Counts each Q, K, V, O and LSE byte once (K/V once per KV head), page
indices as int32, and only the visible (query, key) pairs:

    pairs(prefill r) = qo*(kv - qo) + qo*(qo + 1)/2   (causal; qo*kv otherwise)
    pairs(decode r)  = kv
    FLOPs            = 4 * d * Hq * sum(pairs)        (QK^T and PV, 2 flops/MAC)

Re-reads of K/V by several prefill tiles, split partials, masked MFMA work on
diagonal tiles and the padding of decode rows to 16 are overheads, not counted.
An FP8 KV cache counts one byte per K or V element plus its per-head scales.
A batch with shared prefixes counts each group's prefix K/V once (the pages
are shared; [PAT] abstract); ``bytes_unshared`` counts it once per member.
"""

import numpy as np

PEAK_BF16_FLOPS = 2.5e15     # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM_BYTES = 8.0e12      # MI355X HBM3E, B/s


def algorithmic_counts(b) -> dict:
    get = (lambda k: getattr(b, k)) if not isinstance(b, dict) else (lambda k: b[k])
    hq, hkv, d = get("num_qo_heads"), get("num_kv_heads"), get("head_dim")
    qo = np.asarray(get("prefill_qo_len"), dtype=np.float64)
    pkv = np.asarray(get("prefill_kv_len"), dtype=np.float64)
    dkv = np.asarray(get("decode_kv_len"), dtype=np.float64)
    causal = bool(get("causal"))
    pairs_p = float(np.sum(qo * (pkv - qo) + qo * (qo + 1) / 2)) if causal \
        else float(np.sum(qo * pkv))
    pairs_d = float(np.sum(dkv))
    paged = get("layout") == "paged"
    ps = get("page_size")
    rows_p, rows_d = float(np.sum(qo)), float(len(dkv))

    try:
        kv_elem = 1.0 if get("kv_dtype") == "fp8_e4m3" else 2.0
    except (AttributeError, KeyError):
        kv_elem = 2.0

    def part_bytes(rows, kv_tokens, pages):
        qo_b = rows * hq * d * 2 * 2 + rows * hq * 4          # Q + O (bf16) + LSE
        kv_b = kv_tokens * hkv * d * kv_elem * 2              # K + V
        return qo_b + kv_b + (pages * 4 if paged else 0.0)

    try:
        groups = get("prefix_groups") or ()
    except (AttributeError, KeyError):
        groups = ()
    shared = float(sum((len(m) - 1) * pl for m, pl in groups))   # tokens read once, not per member
    bp = part_bytes(rows_p, float(np.sum(pkv)), float(np.sum(np.ceil(pkv / ps))))
    bd_unshared = part_bytes(rows_d, float(np.sum(dkv)), float(np.sum(np.ceil(dkv / ps))))
    bd = bd_unshared - shared * hkv * d * kv_elem * 2
    if kv_elem == 1.0:
        bd += 2 * hkv * 4                                     # K and V scales
        bd_unshared += 2 * hkv * 4
    fp = 4.0 * d * hq * pairs_p
    fd = 4.0 * d * hq * pairs_d
    return {"flops": fp + fd, "bytes": bp + bd, "flops_prefill": fp, "flops_decode": fd,
            "bytes_prefill": bp, "bytes_decode": bd, "bytes_unshared": bp + bd_unshared}


def overlap_roofline_s(c: dict) -> float:
    return max(c["flops"] / PEAK_BF16_FLOPS, c["bytes"] / PEAK_HBM_BYTES)
