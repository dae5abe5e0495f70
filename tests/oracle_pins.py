"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle is wrong.  They
are collected as tests in ``test_oracle.py`` and re-run against planted
mistakes in ``test_oracle_mutations.py`` (every planted mistake must make at
least one pin fail).  Nothing here calls the GPU library.

What each pin rests on:
  bruteforce      the definition evaluated with pure-Python loops + fsum
  rows_sum_to_one softmax probabilities are a distribution over visible keys
  single_key      one visible key: softmax weight 1, O = v exactly, LSE = score
  decode_is_last_prefill_row   a decode token is the last row of a chunk over
                  the same KV (bottom-right causal alignment)
  split_merge     softmax over a union of disjoint key ranges = LSE merge
  identical_keys  closed form: uniform weights -> prefix mean, LSE = s + ln n
  boundary_probe  a dominant key at the row's own position (and a larger one
                  just after it, which must stay invisible)
  gqa_is_mha      grouped heads == multi-head with repeated KV heads
  sdpa            torch float64 scaled_dot_product_attention, explicit mask
  page_invariance the paged gather == the same tokens stored contiguously
  bf16_upcast     known bfloat16 bit patterns
  sample_rows_bruteforce  the row-sampling entry point against the loop
                  definition on tiny batches (every chunk's first and last
                  row, decodes in shuffled order)
  sample_rows_match_batch the row-sampling entry point against the whole-batch
                  oracle on a paged batch of several chunks and decodes
  fp8_codes       E4M3 bytes: values the format's table fixes, and torch's own
                  float8_e4m3fn decoding of all 256 codes
  fp8_batch_is_dequantized_bf16  an FP8 batch with power-of-two per-head
                  scales equals the bf16 batch holding the decoded values
                  (exact in bf16), different scales per head and for K and V
"""

import math

import numpy as np

import oracle
import oracle.attention as oa
from prefill_decode_amd import inputs
from tests.bruteforce import brute_attention


def _bits_to_float_torch(bits):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.double().numpy()


def _tiny_specs():
    S = inputs.custom_spec
    return [
        S("bf_a", 2, 1, [(3, 7), (1, 1), (5, 5)], [4, 9, 1], seed=11, head_dim=4,
          layout="contiguous", extra_pages=0),
        S("bf_b", 4, 2, [(5, 9), (2, 6)], [3, 8], seed=12, head_dim=8, page_size=2,
          extra_pages=2),
        S("bf_c", 1, 1, [(4, 6)], [5], seed=13, head_dim=1, page_size=3,
          random_pages=True, extra_pages=1),
        S("bf_d", 4, 1, [(3, 8)], [2, 6], seed=14, head_dim=4, causal=False,
          layout="contiguous", extra_pages=0, sm_scale=0.7),
        S("bf_e", 4, 4, [(2, 5)], [7], seed=15, head_dim=8, page_size=4,
          sm_scale=1.3),
    ]


def _request_lists(batch, r):
    """(q rows, k, v) of request r as Python lists via torch's bf16->f64."""
    n_p = len(batch["prefill_qo_len"])
    kv_lens = list(batch["prefill_kv_len"]) + list(batch["decode_kv_len"])
    L = int(kv_lens[r])
    if r < n_p:
        off = int(np.sum(batch["prefill_qo_len"][:r]))
        qo = int(batch["prefill_qo_len"][r])
        qb = batch["q_prefill"][off:off + qo]
    else:
        qo = 1
        qb = batch["q_decode"][r - n_p:r - n_p + 1]
    if batch["layout"] == "contiguous":
        s = int(batch["kv_indptr"][r])
        kb = batch["k_cache"][s:s + L]
        vb = batch["v_cache"][s:s + L]
    else:
        ps = batch["page_size"]
        pages = batch["page_indices"][batch["page_indptr"][r]:batch["page_indptr"][r + 1]]
        kb = np.concatenate([batch["k_cache"][p] for p in pages])[:L]
        vb = np.concatenate([batch["v_cache"][p] for p in pages])[:L]
    return (_bits_to_float_torch(qb).tolist(), _bits_to_float_torch(kb).tolist(),
            _bits_to_float_torch(vb).tolist(), qo, L)


def pin_bruteforce():
    for spec in _tiny_specs():
        b = inputs.make_batch_host(spec)
        out = oracle.batch_attention(b, workers=1)
        n_p = spec.num_prefill
        offs = np.concatenate([[0], np.cumsum(spec.prefill_qo_len)])
        for r in range(n_p + spec.num_decode):
            q, k, v, qo, L = _request_lists(b, r)
            bo, bl = brute_attention(q, k, v, L, qo, spec.num_qo_heads,
                                     spec.num_kv_heads, spec.causal, spec.sm_scale)
            if r < n_p:
                o = out["o_prefill"][offs[r]:offs[r] + qo]
                l = out["lse_prefill"][offs[r]:offs[r] + qo]
            else:
                o = out["o_decode"][r - n_p:r - n_p + 1]
                l = out["lse_decode"][r - n_p:r - n_p + 1]
            assert np.max(np.abs(o - np.array(bo))) <= 1e-12, (spec.name, r)
            assert np.max(np.abs(l - np.array(bl))) <= 1e-12, (spec.name, r)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def pin_rows_sum_to_one():
    rng = np.random.default_rng(21)
    for causal in (True, False):
        q = _rand(rng, 6, 4, 16)
        k = _rand(rng, 11, 2, 16)
        v = _rand(rng, 11, 2, 16)
        pos = np.arange(5, 11)
        o, l, p = oa.attention_rows(q, pos, k, v, causal, 0.4, return_probs=True)
        assert np.max(np.abs(p.sum(axis=2) - 1.0)) <= 1e-12
        assert np.all(p >= 0)
        if causal:
            for i, ps in enumerate(pos):
                assert np.all(p[i, :, ps + 1:] == 0.0)
                assert np.all(p[i, :, :ps + 1] > 0.0)
        # O is the probability-weighted mean of V of the head's KV head
        for h in range(4):
            ref = p[:, h, :] @ v[:, h // 2, :]
            assert np.max(np.abs(o[:, h, :] - ref)) <= 1e-12


def pin_single_key():
    rng = np.random.default_rng(22)
    q = _rand(rng, 1, 3, 8)
    k = _rand(rng, 1, 3, 8)
    v = _rand(rng, 1, 3, 8)
    for causal in (True, False):
        o, l = oa.attention_rows(q, [0], k, v, causal, 0.3)
        assert np.array_equal(o[0], v[0]), "single key must return V exactly"
        for h in range(3):
            s = 0.3 * math.fsum(q[0, h, c] * k[0, h, c] for c in range(8))
            assert abs(l[0, h] - s) <= 1e-15 * max(1.0, abs(s))
    # causal chunk with qo == kv: row 0 sees only key 0
    spec = inputs.custom_spec("sk", 2, 2, [(6, 6)], [], seed=23, head_dim=8,
                              layout="contiguous", extra_pages=0)
    b = inputs.make_batch_host(spec)
    out = oracle.batch_attention(b, workers=1)
    v0 = oa.bf16_bits_to_f64(b["v_cache"][0])
    assert np.array_equal(out["o_prefill"][0], v0)


def pin_decode_is_last_prefill_row():
    for layout in ("contiguous", "paged"):
        L, n = 37, 9
        spec = inputs.custom_spec("dl", 4, 2, [(n, L)], [L], seed=24, head_dim=16,
                                  layout=layout, page_size=4, extra_pages=0)
        b = inputs.make_batch_host(spec)
        b["q_decode"][0] = b["q_prefill"][n - 1]
        if layout == "contiguous":
            b["k_cache"][L:2 * L] = b["k_cache"][0:L]
            b["v_cache"][L:2 * L] = b["v_cache"][0:L]
        else:
            ip = b["page_indptr"]
            b["page_indices"][ip[1]:ip[2]] = b["page_indices"][ip[0]:ip[1]]
        out = oracle.batch_attention(b, workers=1)
        # equal up to BLAS rounding (a 1-row product may take another kernel)
        assert np.max(np.abs(out["o_decode"][0] - out["o_prefill"][n - 1])) <= 1e-13
        assert np.max(np.abs(out["lse_decode"][0] - out["lse_prefill"][n - 1])) <= 1e-13
        # and not equal to the first row (alignment matters)
        assert not np.allclose(out["o_decode"][0], out["o_prefill"][0])


def pin_split_merge():
    rng = np.random.default_rng(25)
    kv = 29
    q = _rand(rng, 7, 4, 8)
    k = _rand(rng, kv, 2, 8)
    v = _rand(rng, kv, 2, 8)
    pos = np.arange(kv - 7, kv)
    for causal in (True, False):
        o_ref, l_ref = oa.attention_rows(q, pos, k, v, causal, 0.5)
        cuts = [[0, kv], [0, 13, kv], [0, 10, 20, kv],
                [0, 4, 8, 12, 16, 20, 24, kv], list(range(kv + 1)),
                [0, 25, kv]]          # last split above the diagonal for early rows
        for c in cuts:
            parts = [oa.attention_partial(q, pos, k, v, causal, 0.5, a, e)
                     for a, e in zip(c[:-1], c[1:])]
            o, l = oa.merge_partials(parts)
            assert np.max(np.abs(o - o_ref)) <= 1e-12, c
            assert np.max(np.abs(l - l_ref)) <= 1e-12, c
    # an all-empty split is (0, -inf) and leaves a merge unchanged
    o_e, l_e = oa.attention_partial(q, pos, k, v, True, 0.5, kv, kv + 3)
    assert np.all(o_e == 0) and np.all(np.isneginf(l_e))
    o1, l1 = oa.attention_rows(q, pos, k, v, True, 0.5)
    o2, l2 = oa.merge_partials([(o1, l1), (o_e, l_e)])
    assert np.max(np.abs(o2 - o1)) <= 1e-15 and np.max(np.abs(l2 - l1)) <= 1e-15


def pin_identical_keys():
    rng = np.random.default_rng(26)
    kv, n, d = 12, 5, 8
    q = _rand(rng, n, 2, d)
    kvec = _rand(rng, d)
    k = np.tile(kvec, (kv, 1, 1))           # [kv, 1, d]
    v = _rand(rng, kv, 1, d)
    pos = np.arange(kv - n, kv)
    for causal in (True, False):
        o, l = oa.attention_rows(q, pos, k, v, causal, 0.9)
        for i in range(n):
            cnt = pos[i] + 1 if causal else kv
            mean = v[:cnt, 0, :].mean(axis=0)
            for h in range(2):
                assert np.max(np.abs(o[i, h] - mean)) <= 1e-12
                s = 0.9 * float(np.dot(q[i, h], kvec))
                assert abs(l[i, h] - (s + math.log(cnt))) <= 1e-12


def pin_boundary_probe():
    rng = np.random.default_rng(27)
    kv, n, d = 16, 6, 8
    pos = np.arange(kv - n, kv)
    q = _rand(rng, n, 1, d)
    for i in [0, 2, 4]:
        k = 0.1 * _rand(rng, kv, 1, d)
        v = _rand(rng, kv, 1, d)
        qn = q[i, 0] / np.linalg.norm(q[i, 0])
        k[pos[i], 0] = 60.0 * qn              # dominant visible key
        if pos[i] + 1 < kv:
            k[pos[i] + 1, 0] = 120.0 * qn     # even larger, but in the future
        o, l = oa.attention_rows(q, pos, k, v, True, 1.0 / math.sqrt(d))
        assert np.max(np.abs(o[i, 0] - v[pos[i], 0])) <= 1e-6, i


def pin_gqa_is_mha():
    rng = np.random.default_rng(28)
    kv, n, d, hq, hkv = 10, 4, 8, 6, 2
    g = hq // hkv
    q = _rand(rng, n, hq, d)
    k = _rand(rng, kv, hkv, d)
    v = _rand(rng, kv, hkv, d)
    pos = np.arange(kv - n, kv)
    o1, l1 = oa.attention_rows(q, pos, k, v, True, 0.6)
    krep = np.repeat(k, g, axis=1)            # head h -> kv head h // g
    vrep = np.repeat(v, g, axis=1)
    o2, l2 = oa.attention_rows(q, pos, krep, vrep, True, 0.6)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # and a different head->group map gives a different answer
    kalt = np.tile(k, (1, g, 1))              # head h -> kv head h % hkv
    valt = np.tile(v, (1, g, 1))
    o3, _ = oa.attention_rows(q, pos, kalt, valt, True, 0.6)
    assert not np.allclose(o1, o3)


def pin_sdpa():
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(29)
    for (n, kv, hq, hkv, d, causal) in [(5, 9, 4, 2, 16, True), (7, 7, 2, 1, 8, True),
                                         (1, 33, 4, 4, 32, True), (6, 20, 3, 1, 8, False),
                                         (64, 200, 4, 2, 128, True)]:
        q = _rand(rng, n, hq, d)
        k = _rand(rng, kv, hkv, d)
        v = _rand(rng, kv, hkv, d)
        pos = np.arange(kv - n, kv)
        scale = 1.0 / math.sqrt(d)
        o, l = oa.attention_rows(q, pos, k, v, causal, scale)
        g = hq // hkv
        qt = torch.from_numpy(q).permute(1, 0, 2)                      # [hq, n, d]
        kt = torch.from_numpy(np.repeat(k, g, axis=1)).permute(1, 0, 2)
        vt = torch.from_numpy(np.repeat(v, g, axis=1)).permute(1, 0, 2)
        mask = torch.ones(n, kv, dtype=torch.bool)
        if causal:
            mask = torch.arange(kv)[None, :] <= torch.from_numpy(pos)[:, None]
        ot = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
        st = (qt @ kt.transpose(1, 2)) * scale
        lt = torch.logsumexp(st.masked_fill(~mask, float("-inf")), dim=-1)  # [hq, n]
        assert np.max(np.abs(o - ot.permute(1, 0, 2).numpy())) <= 1e-10
        assert np.max(np.abs(l - lt.T.numpy())) <= 1e-10


def pin_page_invariance():
    base = inputs.custom_spec("pg", 4, 2, [(7, 40), (3, 21)], [17, 33, 1], seed=30,
                              head_dim=8, page_size=4, extra_pages=5)
    bp = inputs.make_batch_host(base)
    # the same logical tokens laid out contiguously
    bc = dict(bp)
    bc["layout"] = "contiguous"
    lens = list(base.prefill_kv_len) + list(base.decode_kv_len)
    ks, vs, ip = [], [], [0]
    for r, L in enumerate(lens):
        pages = bp["page_indices"][bp["page_indptr"][r]:bp["page_indptr"][r + 1]]
        ks.append(np.concatenate([bp["k_cache"][p] for p in pages])[:L])
        vs.append(np.concatenate([bp["v_cache"][p] for p in pages])[:L])
        ip.append(ip[-1] + L)
    bc["k_cache"] = np.concatenate(ks)
    bc["v_cache"] = np.concatenate(vs)
    bc["kv_indptr"] = np.array(ip, dtype=np.int32)
    o1 = oracle.batch_attention(bp, workers=1)
    o2 = oracle.batch_attention(bc, workers=1)
    for key in o1:
        assert np.array_equal(o1[key], o2[key]), key
        assert np.all(np.isfinite(o1[key])), key   # poison never read


def pin_bf16_upcast():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F80, 0x0000, 0x8000, 0x4049],
                    dtype=np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, math.inf, 0.0, -0.0,
            3.140625]
    got = oa.bf16_bits_to_f64(bits)
    for g_, w in zip(got, want):
        assert g_ == w, (g_, w)


def _chunk_edge_rows(qo_lens, rng, extra=2):
    """Every chunk's first, second, last and second-to-last rows plus a few
    random rows (global row indices), shuffled."""
    offs = np.concatenate([[0], np.cumsum(qo_lens)]).astype(int)
    rows = set()
    for r in range(len(qo_lens)):
        a, b = int(offs[r]), int(offs[r + 1])
        rows.update([a, min(a + 1, b - 1), b - 1, max(a, b - 2)])
        rows.update(int(x) for x in rng.integers(a, b, size=min(extra, b - a)))
    rows = sorted(rows)
    rng.shuffle(rows)
    return rows


def pin_sample_rows_bruteforce():
    rng = np.random.default_rng(31)
    for spec in _tiny_specs():
        b = inputs.make_batch_host(spec)
        n_p = spec.num_prefill
        offs = np.concatenate([[0], np.cumsum(spec.prefill_qo_len)]).astype(int)
        rows = _chunk_edge_rows(spec.prefill_qo_len, rng)
        dec = list(rng.permutation(spec.num_decode))
        out = oracle.sample_batch_attention(b, rows, dec, workers=1)
        assert list(out["prefill_rows"]) == rows and list(out["decode_ids"]) == dec
        brute = {}
        for r in range(n_p + spec.num_decode):
            q, k, v, qo, L = _request_lists(b, r)
            brute[r] = brute_attention(q, k, v, L, qo, spec.num_qo_heads,
                                       spec.num_kv_heads, spec.causal, spec.sm_scale)
        for t, g in enumerate(rows):
            r = int(np.nonzero(offs[1:] > g)[0][0])           # offs[r] <= g < offs[r+1]
            bo, bl = brute[r]
            assert np.max(np.abs(out["o_prefill"][t] - np.array(bo[g - offs[r]]))) <= 1e-12, \
                (spec.name, g)
            assert np.max(np.abs(out["lse_prefill"][t] - np.array(bl[g - offs[r]]))) <= 1e-12
        for t, i in enumerate(dec):
            bo, bl = brute[n_p + int(i)]
            assert np.max(np.abs(out["o_decode"][t] - np.array(bo[0]))) <= 1e-12, (spec.name, i)
            assert np.max(np.abs(out["lse_decode"][t] - np.array(bl[0]))) <= 1e-12


def pin_sample_rows_match_batch():
    rng = np.random.default_rng(32)
    spec = inputs.custom_spec("samp", 8, 2, [(37, 200), (1, 64), (90, 90), (64, 300)],
                              [1, 17, 300, 64, 129], seed=33, head_dim=16, page_size=8,
                              extra_pages=3)
    b = inputs.make_batch_host(spec)
    full = oracle.batch_attention(b, workers=1)
    rows = _chunk_edge_rows(spec.prefill_qo_len, rng, extra=4)
    dec = [4, 0, 2, 3, 1]
    out = oracle.sample_batch_attention(b, rows, dec, workers=2)
    for key, idx in (("o_prefill", rows), ("lse_prefill", rows), ("o_decode", dec),
                     ("lse_decode", dec)):
        assert np.all(np.isfinite(out[key])), key
        assert np.max(np.abs(out[key] - full[key][idx])) <= 1e-13, key


def pin_fp8_codes():
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x3C: 1.5, 0x40: 2.0, 0x77: 240.0, 0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0,
             0xFE: -448.0}
    got = oa.fp8_e4m3_bits_to_f64(np.array(list(table), dtype=np.uint8))
    for g_, w in zip(got, table.values()):
        assert g_ == w and np.signbit(g_) == np.signbit(w), (g_, w)
    nan = oa.fp8_e4m3_bits_to_f64(np.array([0x7F, 0xFF], dtype=np.uint8))
    assert np.all(np.isnan(nan))
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    mine = oa.fp8_e4m3_bits_to_f64(codes)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.all(np.diff(mine[:0x7F]) > 0)                   # codes 0..0x7E increase


def pin_fp8_batch_is_dequantized_bf16():
    spec = inputs.custom_spec("f8", 4, 2, [], [5, 13, 1], seed=34, head_dim=8, page_size=4,
                              extra_pages=1, kv_dtype="fp8_e4m3")
    b8 = inputs.make_batch_host(spec, poison=False)
    b8["k_scale"] = np.array([2.0 ** -3, 2.0 ** -1], dtype=np.float32)
    b8["v_scale"] = np.array([2.0 ** -2, 2.0], dtype=np.float32)
    out8 = oracle.batch_attention(b8, workers=1)
    # the same batch in bf16: the decoded values, exact in bf16 (3 mantissa
    # bits times a power of two), computed without the oracle's decoder
    import torch
    bb = dict(b8)
    bb["kv_dtype"] = "bf16"
    for key, sc in (("k_cache", "k_scale"), ("v_cache", "v_scale")):
        x = torch.from_numpy(b8[key]).view(torch.float8_e4m3fn).float().numpy()
        x = x * b8[sc][None, None, :, None]
        bb[key] = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        assert np.array_equal(bb[key].astype(np.uint32) << 16, x.astype(np.float32).view(np.uint32))
    outb = oracle.batch_attention(bb, workers=1)
    for k in ("o_decode", "lse_decode"):
        assert np.all(np.isfinite(out8[k])), k
        assert np.max(np.abs(out8[k] - outb[k])) <= 1e-13, k


ALL_PINS = [pin_bruteforce, pin_rows_sum_to_one, pin_single_key,
            pin_decode_is_last_prefill_row, pin_split_merge, pin_identical_keys,
            pin_boundary_probe, pin_gqa_is_mha, pin_sdpa, pin_page_invariance,
            pin_bf16_upcast, pin_sample_rows_bruteforce, pin_sample_rows_match_batch,
            pin_fp8_codes, pin_fp8_batch_is_dequantized_bf16]
