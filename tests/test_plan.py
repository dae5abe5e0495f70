"""Host planner invariants (CPU, through pod_attn_plan_host).

Every (row, head) is covered by exactly one prefill tile or decode unit group,
whose KV splits partition the visible keys; partial slots are disjoint and the
merge tasks reference exactly them; XCD pools partition the prefill list; the
split caps and the proportional mix follow the planner's rules."""

import numpy as np
import pytest

from prefill_decode_amd import binding as B
from prefill_decode_amd import inputs

# item layouts (include/pod_attn.h, pod_attn_plan_export)
P_F, D_F, M_F = 8, 8, 4


def _spec_lists(spec, **tun):
    p = B.make_params(spec.num_qo_heads, spec.num_kv_heads, spec.layout, spec.page_size,
                      spec.causal, spec.sm_scale)
    t = B.make_tuning(**tun) if tun else None
    pl = B.plan_host(p, spec.prefill_qo_len, spec.prefill_kv_len, spec.decode_kv_len, t)
    return pl


def _check_lists(spec, pitems, ditems, mtasks, pool_off, n_partials):
    hq, hkv = spec.num_qo_heads, spec.num_kv_heads
    g = hq // hkv
    qo = np.array(spec.prefill_qo_len, dtype=np.int64)
    kv = np.array(spec.prefill_kv_len, dtype=np.int64)
    offs = np.concatenate([[0], np.cumsum(qo)])
    P = pitems.reshape(-1, P_F)
    D = ditems.reshape(-1, D_F)
    M = mtasks.reshape(-1, M_F)
    used = np.zeros(max(n_partials, 1), dtype=np.int32)

    # ---- prefill: group items by tile (qrow0, first head); a tile covers
    # nh heads (4, 2 or 1: the largest dividing g) x up to 256 / nh positions
    nh = 4 if g % 4 == 0 else 2 if g % 2 == 0 else 1
    npos = 256 // nh
    tiles = {}
    for it in P:
        tiles.setdefault((int(it[0]), int(it[1])), []).append(it)
    covered = np.zeros((int(offs[-1]), hq), dtype=np.int32)
    for (qrow0, h), its in tiles.items():
        assert h % nh == 0 and h + nh <= hq
        its = sorted(its, key=lambda x: x[4])
        r = int(its[0][6])
        nrows, pos0 = int(its[0][2]), int(its[0][3])
        assert all(int(x[2]) == nrows and int(x[3]) == pos0 and int(x[6]) == r for x in its)
        assert 1 <= nrows <= npos
        assert offs[r] <= qrow0 and qrow0 + nrows <= offs[r + 1]
        row_in_req = qrow0 - offs[r]
        assert pos0 == kv[r] - qo[r] + row_in_req            # bottom-right alignment
        end = min(kv[r], pos0 + nrows) if spec.causal else kv[r]
        # splits partition [0, end) on 64-key boundaries
        assert int(its[0][4]) == 0 and int(its[-1][5]) == end
        for a, b in zip(its[:-1], its[1:]):
            assert int(a[5]) == int(b[4]) and int(b[4]) % 64 == 0
        assert all(int(x[4]) < int(x[5]) for x in its)
        covered[qrow0:qrow0 + nrows, h:h + nh] += 1
        parts = [int(x[7]) for x in its]
        if len(its) == 1:
            assert parts == [-1]
        else:
            assert all(p >= 0 for p in parts)
            for p in parts:
                for j in range(nh):           # head slot j: rows p + j * npos + i
                    assert np.all(used[p + j * npos:p + j * npos + nrows] == 0)
                    used[p + j * npos:p + j * npos + nrows] += 1
    assert np.all(covered == 1)

    # ---- decode: units partition heads x keys ----
    dkv = np.array(spec.decode_kv_len, dtype=np.int64)
    n_p = len(qo)
    per_req = {}
    for it in D:
        per_req.setdefault(int(it[0]), []).append(it)
    assert sorted(per_req) == list(range(len(dkv)))
    for i, its in per_req.items():
        heads = {}
        for it in its:
            h0, nq = int(it[1]), int(it[2])
            assert 1 <= nq <= 16 and h0 // g == (h0 + nq - 1) // g    # one KV head
            assert int(it[5]) == n_p + i
            heads.setdefault((h0, nq), []).append(it)
        hcov = np.zeros(hq, dtype=np.int32)
        nsplit = None
        for (h0, nq), sp in heads.items():
            hcov[h0:h0 + nq] += 1
            sp = sorted(sp, key=lambda x: x[3])
            assert int(sp[0][3]) == 0 and int(sp[-1][4]) == dkv[i]
            for a, b in zip(sp[:-1], sp[1:]):
                assert int(a[4]) == int(b[3]) and int(b[3]) % 32 == 0
            nsplit = len(sp) if nsplit is None else nsplit
            assert len(sp) == nsplit
            for it in sp:
                if nsplit == 1:
                    assert int(it[6]) == -1
                else:
                    for jj in range(nq):
                        p = int(it[6]) + jj * int(it[7])
                        assert used[p] == 0
                        used[p] += 1
        assert np.all(hcov == 1)
    # ---- merge tasks cover exactly the split rows ----
    seen = set()
    for t in M:
        out, base, stride, nf = (int(x) for x in t)
        n, dec = nf & 0xFFFF, nf >> 16
        assert n >= 2
        assert (out, dec) not in seen
        seen.add((out, dec))
        for s in range(n):
            assert used[base + s * stride] == 1
            used[base + s * stride] = 2
    assert np.all(used[:n_partials] != 1), "a partial slot is written but never merged"
    # ---- pools ----
    po = np.asarray(pool_off)
    assert po[0] == 0 and po[-1] == len(P) and np.all(np.diff(po) >= 0)


def _specs():
    S = inputs.custom_spec
    out = [inputs.config_spec(n) for n in inputs.CONFIG_NAMES]
    out += [inputs.config_spec("batched", n_dec=n) for n in (32, 64, 128, 256)]
    out += [
        S("ragged", 12, 4, [(1, 1), (129, 300), (7, 7), (300, 1000)], [1, 31, 33, 500], seed=1),
        S("gqa32", 64, 2, [(200, 200)], [4000, 17], seed=2),        # 32 q heads per kv head
        S("only_prefill", 8, 8, [(513, 2000)], [], seed=3),
        S("only_decode", 32, 8, [], [1, 2, 3, 40000], seed=4),
        S("noncausal", 4, 2, [(100, 250)], [9], seed=5, causal=False),
        S("page1", 4, 1, [(5, 70)], [65], seed=6, page_size=1),
        S("page64", 8, 2, [(70, 140)], [1000], seed=7, page_size=64),
        S("empty", 4, 2, [], [], seed=8),
    ]
    return out


@pytest.mark.parametrize("spec", _specs(), ids=lambda s: s.name)
@pytest.mark.parametrize("tun", [{}, dict(prefill_kv_splits=3, decode_kv_splits=5),
                                 dict(match_sequential=1), dict(prefill_quarters_per_cu=1)],
                         ids=["auto", "forced", "matched", "q1"])
def test_lists_cover_and_partition(spec, tun):
    pl = _spec_lists(spec, **tun)
    info = pl.info()
    for which_p, which_d, which_m, which_pool in ((0, 1, 2, 6), (3, 4, 5, 7)):
        _check_lists(spec, pl.export(which_p), pl.export(which_d), pl.export(which_m),
                     pl.export(which_pool), info["num_partials"])
    if tun.get("match_sequential"):
        for a, b in ((0, 3), (1, 4), (2, 5)):
            assert np.array_equal(pl.export(a), pl.export(b))


def test_forced_splits_are_honoured():
    spec = inputs.custom_spec("f", 8, 2, [(128, 4096)], [4096, 100], seed=9)
    pl = _spec_lists(spec, prefill_kv_splits=4, decode_kv_splits=8)
    P = pl.export(0).reshape(-1, P_F)
    D = pl.export(1).reshape(-1, D_F)
    assert len(P) == 2 * 2 * 4                  # 2 groups of 4 heads x 2 blocks of 64 x 4 splits
    d0 = D[D[:, 0] == 0]
    assert len(d0) == 2 * 8                     # 2 kv heads x 8 splits
    d1 = D[D[:, 0] == 1]
    assert len(d1) == 2 * 4                     # 100 keys: at most ceil(100/32) splits


def test_split_cap_two_waves():
    # [POD] "Cap prefill splitting": tiles x splits <= 2 x slots.  The
    # sequential list keeps that cap (it aims at one item per slot).  The
    # fused list departs from it for large prefills (> 1536 tokens): 3 items
    # per slot of the whole GPU, three waves, which measured 0.8% faster on
    # the 70B-shaped layer than two (more waves were slower); small prefills
    # aim at 1.5 items per slot of the prefill CUs.
    slots = 256 * 2
    for spec in _specs():
        pl = _spec_lists(spec, match_sequential=0)
        P = pl.export(3).reshape(-1, P_F)
        tiles = {(int(r[0]), int(r[1])) for r in P}
        if len(tiles):
            assert len(P) <= max(len(tiles), 2 * slots), spec.name
        D = pl.export(4).reshape(-1, D_F)
        per = {}
        for r in D:
            per.setdefault((int(r[0]), int(r[1])), 0)
            per[(int(r[0]), int(r[1]))] += 1
        assert max(per.values(), default=1) <= 64
        # fused list
        F = pl.export(0).reshape(-1, P_F)
        tiles = {(int(r[0]), int(r[1])) for r in F}
        if len(tiles):
            q = pl.info()["prefill_quarters_per_cu"]
            if sum(spec.prefill_qo_len) > 1536:
                cap = 3 * slots
            else:
                cap = (3 * max(1, 256 * q // 4)) // 2
            assert len(F) <= max(len(tiles), cap), (spec.name, len(F), cap)


def test_small_prefill_regime_accounts_for_colocated_decode():
    # [PR] "Limit kv split when prefill tokens <= 1536": the fused plan's
    # prefill splits fill only the slots beside the co-located decode WGs;
    # above 1536 tokens every slot.  Fused plans aim at up to 1.5 items per
    # slot in the small regime and 3 in the large one, sequential plans at 1.
    def per_tile_max(P):
        per = {}
        for r in P:
            per[(int(r[0]), int(r[1]))] = per.get((int(r[0]), int(r[1])), 0) + 1
        return len(per), max(per.values())

    spec = inputs.config_spec("batched")          # exactly 1536 prefill tokens
    pl = _spec_lists(spec)
    q = pl.info()["prefill_quarters_per_cu"]
    fused = pl.export(0).reshape(-1, P_F)
    seq = pl.export(3).reshape(-1, P_F)
    tiles, fmax = per_tile_max(fused)
    coloc_slots = max(1, 256 * q // 4)
    assert fmax <= max(1, 3 * coloc_slots // (2 * tiles))
    _, smax = per_tile_max(seq)
    assert smax <= max(1, 1 * 512 // tiles)
    big = inputs.custom_spec("big", 32, 8, [(1600, 4096)], [2000] * 64, seed=3)
    pb = _spec_lists(big)
    tiles_b, fmax_b = per_tile_max(pb.export(0).reshape(-1, P_F))
    assert fmax_b == min(16, max(1, 3 * 512 // tiles_b))   # every slot counts


def test_proportional_mix():
    info = {n: _spec_lists(inputs.config_spec(n)).info() for n in inputs.CONFIG_NAMES}
    q = {n: i["prefill_quarters_per_cu"] for n, i in info.items()}
    for n, i in info.items():
        # automatic launch shape: one workgroup per unit for at most two
        # fused units per workgroup slot (co-located roles with one prefill
        # request, CU-partition roles with several), else persistent CU
        # partition
        small = i["prefill_items"] + i["decode_groups"] <= 2 * 512
        assert i["one_unit_per_wg"] == int(small), n
        several = len(inputs.config_spec(n).prefill_qo_len) > 1
        if small and not several:
            assert i["sched_mode"] == B.SCHED_COLOCATE and 1 <= q[n] <= 7, n
        elif small:
            assert i["sched_mode"] == B.SCHED_SPLIT and 3 <= q[n] <= 6, n
        else:
            # CU partition: 3..6 eighths of the CUs start on prefill
            assert i["sched_mode"] == B.SCHED_SPLIT and 3 <= q[n] <= 6, n
    assert info["llama3_8b"]["one_unit_per_wg"] == 1 and info["tiny"]["one_unit_per_wg"] == 1
    assert q["llama2_7b"] == 3              # decode-heavy MHA: smallest prefill share
    assert q["l70b_tp1"] >= 3               # large prefill: about half or more
    assert _spec_lists(inputs.config_spec("l70b_tp1"), sched_mode=B.SCHED_SPLIT).info()[
        "sched_mode"] == B.SCHED_SPLIT
    assert _spec_lists(inputs.config_spec("l70b_tp1")).info()["sched_mode"] == B.SCHED_SPLIT
    qc = _spec_lists(inputs.config_spec("llama2_7b"), sched_mode=B.SCHED_COLOCATE).info()
    assert 1 <= qc["prefill_quarters_per_cu"] <= 7
    only_p = inputs.custom_spec("p", 8, 8, [(256, 512)], [], seed=1)
    only_d = inputs.custom_spec("d", 8, 8, [], [512], seed=1)
    assert _spec_lists(only_p).info()["prefill_quarters_per_cu"] == 8
    assert _spec_lists(only_d).info()["prefill_quarters_per_cu"] == 0
    assert _spec_lists(only_p, prefill_quarters_per_cu=3).info()["prefill_quarters_per_cu"] == 3


def test_prefill_items_longest_first_within_pools():
    for name in ("llama3_8b", "batched"):
        pl = _spec_lists(inputs.config_spec(name))
        P = pl.export(0).reshape(-1, P_F)
        po = pl.export(6)
        work = P[:, 2].astype(np.int64) * (P[:, 5] - P[:, 4])
        for x in range(len(po) - 1):
            w = work[po[x]:po[x + 1]]
            assert np.all(np.diff(w) <= 0), (name, x)


def test_decode_items_longest_first_and_pools_by_kv_head():
    spec = inputs.config_spec("l70b_tp1")
    pl = _spec_lists(spec)
    D = pl.export(1).reshape(-1, D_F)
    work = D[:, 4] - D[:, 3]
    assert np.all(np.diff(work) <= 0)
    P = pl.export(0).reshape(-1, P_F)
    po = pl.export(6)
    g = spec.num_qo_heads // spec.num_kv_heads
    for x in range(len(po) - 1):
        kvh = set((P[po[x]:po[x + 1], 1] // g).tolist())
        assert kvh == {x}, (x, kvh)           # 8 KV heads -> one per XCD pool


def test_forced_splits_are_capped_at_64():
    spec = inputs.custom_spec("cap", 8, 2, [(64, 16384)], [16384], seed=5)
    pl = _spec_lists(spec, prefill_kv_splits=100, decode_kv_splits=100)
    P = pl.export(0).reshape(-1, P_F)
    D = pl.export(1).reshape(-1, D_F)
    assert len(P) == 2 * 64                     # 2 head groups x 1 block x 64 splits
    assert len(D) == 2 * 64                     # 2 kv heads x 64 splits
    M = pl.export(2).reshape(-1, M_F)
    assert int((M[:, 3] & 0xFFFF).max()) == 64


def test_decode_chunk_floor_follows_batch_size():
    # enough decode keys for every decode wavefront: chunks of >= 512 keys
    # (only a request's remainder is shorter); too few: chunks down to 128
    tiny = inputs.config_spec("tiny")
    D = _spec_lists(tiny).export(1).reshape(-1, D_F)
    assert (D[:, 4] - D[:, 3]).max() <= 128
    spec = inputs.config_spec("llama3_8b")
    D = _spec_lists(spec).export(1).reshape(-1, D_F)
    for i, kv in enumerate(spec.decode_kv_len):
        d = D[D[:, 0] == i]
        n_split = len(d) // spec.num_kv_heads
        assert n_split <= -(-kv // 512), (i, kv, n_split)


@pytest.mark.parametrize("spec", [s for s in _specs() if s.name != "empty"], ids=lambda s: s.name)
def test_batched_prefill_lists_cover_every_row(spec):
    # the batched-prefill comparator's list: prefill tiles as in the other
    # lists, plus one one-row tile per (decode, packed head group) whose KV
    # splits partition the decode's keys; merge tasks write the decode rows
    import dataclasses
    pl = _spec_lists(spec, flags=B.FLAG_BATCHED_PREFILL)
    n_p = spec.num_prefill
    hq, g = spec.num_qo_heads, spec.num_qo_heads // spec.num_kv_heads
    nh = 4 if g % 4 == 0 else 2 if g % 2 == 0 else 1
    P = pl.export(8).reshape(-1, P_F)
    M = pl.export(9).reshape(-1, M_F)
    po = pl.export(10)
    assert po[0] == 0 and po[-1] == len(P) and np.all(np.diff(po) >= 0)
    is_dec = P[:, 6] >= n_p
    m_dec = (M[:, 3] >> 16) == 1
    # the prefill tiles (and their merge tasks) pass the tuned lists' checks
    _check_lists(dataclasses.replace(spec, decode_kv_len=()), P[~is_dec].ravel(),
                 np.zeros(0, np.int32), M[~m_dec].ravel(), [0, int((~is_dec).sum())],
                 pl.info()["num_partials"])
    cov = np.zeros((spec.num_decode, hq), np.int32)
    tiles = {}
    for it in P[is_dec]:
        i, h = int(it[0]), int(it[1])
        assert int(it[6]) == n_p + i and int(it[2]) == 1
        assert int(it[3]) == spec.decode_kv_len[i] - 1     # the decode row's position
        tiles.setdefault((i, h), []).append(it)
    used = set()
    for (i, h), its in tiles.items():
        assert h % nh == 0
        cov[i, h:h + nh] += 1
        its = sorted(its, key=lambda x: x[4])
        assert int(its[0][4]) == 0 and int(its[-1][5]) == spec.decode_kv_len[i]
        for a, b in zip(its[:-1], its[1:]):
            assert int(a[5]) == int(b[4])
        if len(its) == 1:
            assert int(its[0][7]) == -1
        else:
            for t in its:
                for j in range(nh):
                    slot = int(t[7]) + j * (256 // nh)
                    assert slot not in used
                    used.add(slot)
    assert np.all(cov == 1)
    # decode merge tasks: one per split (decode, head), reading exactly the
    # slots the decode tiles write, and writing decode rows
    outs = set()
    for t in M[m_dec]:
        out, base, stride, n = int(t[0]), int(t[1]), int(t[2]), int(t[3]) & 0xFFFF
        assert 0 <= out < spec.num_decode * hq and out not in outs
        outs.add(out)
        for k in range(n):
            used.remove(base + k * stride)
    assert not used


def test_ordered_mode_takes_the_sequential_lists():
    # the ordered scheduler runs prefill units on every slot, then decode
    # units: its lists are sized as the sequential kernels' are
    for name in inputs.CONFIG_NAMES:
        spec = inputs.config_spec(name)
        po = _spec_lists(spec, sched_mode=B.SCHED_ORDERED)
        ps = _spec_lists(spec)
        for a, b in ((0, 3), (1, 4), (2, 5)):
            assert np.array_equal(po.export(a), ps.export(b)), (name, a)


def test_mha_small_prefill_share_runs_sequentially():
    # automatic scheduling routes an MHA batch with a small prefill share and
    # too many units for the one-unit launch to the two kernels back to back
    def routed(spec, **tun):
        p = B.make_params(spec.num_qo_heads, spec.num_kv_heads, spec.layout, spec.page_size,
                          spec.causal, spec.sm_scale, kv_dtype=spec.kv_dtype)
        t = B.make_tuning(**tun) if tun else None
        return B.plan_host(p, spec.prefill_qo_len, spec.prefill_kv_len, spec.decode_kv_len,
                           t).info()["runs_sequential"]
    assert routed(inputs.config_spec("llama2_7b")) == 1
    assert routed(inputs.config_spec("llama2_7b_fp8")) == 1
    assert routed(inputs.config_spec("llama2_7b"), sched_mode=B.SCHED_SPLIT) == 0
    for name in ("tiny", "llama3_8b", "l70b_tp1"):       # GQA with one request, or one-unit
        assert routed(inputs.config_spec(name)) == 0, name
    big = inputs.custom_spec("mha_big_prefill", 32, 32, [(4096, 12288)], [8192] * 128, seed=1)
    assert routed(big) == 0                                          # share ~0.24


def _random_spec(rng, i):
    """A random small batch: head layout, page size, causal flag, prefill
    chunks (qo <= kv) and decode lengths drawn from a seeded generator."""
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 16, 24, 32]))
    np_ = int(rng.integers(0, 5))
    nd = int(rng.integers(0, 12))
    if np_ + nd == 0:
        nd = 1
    pre = []
    for _ in range(np_):
        qo = int(rng.integers(1, 700))
        pre.append((qo, qo + int(rng.integers(0, 3000))))
    dec = [int(x) for x in rng.integers(1, 9000, size=nd)]
    return inputs.custom_spec(f"rand{i}", g * hkv, hkv, pre, dec, seed=9000 + i,
                              causal=bool(rng.integers(0, 4)),
                              page_size=int(rng.choice([1, 8, 16, 64])))


def test_random_batches_cover_and_partition():
    """Seeded random batches (head groups 1-32, 0-4 prefill chunks, 0-11
    decodes, causal or not, page sizes 1-64) under random tunings: every
    list the planner builds (fused and sequential) covers each (row, head)
    once, splits partition the visible keys, and every partial slot is
    merged exactly once."""
    rng = np.random.default_rng(20261204)
    for i in range(60):
        spec = _random_spec(rng, i)
        tun = {}
        if rng.integers(0, 2):
            tun["prefill_kv_splits"] = int(rng.integers(0, 70))
        if rng.integers(0, 2):
            tun["decode_kv_splits"] = int(rng.integers(0, 70))
        if rng.integers(0, 3) == 0:
            tun["prefill_quarters_per_cu"] = int(rng.integers(0, 9))
        if rng.integers(0, 3) == 0:
            tun["sched_mode"] = int(rng.integers(0, 4))
        pl = _spec_lists(spec, **tun)
        info = pl.info()
        for which in ((0, 1, 2, 6), (3, 4, 5, 7)):
            _check_lists(spec, *(pl.export(w) for w in which), info["num_partials"])
        pl.destroy()


def test_one_unit_roles_follow_prefill_request_count():
    """Small batches run one workgroup per unit: with co-located roles for one
    prefill request, with the CU partition's roles (and its lists) for
    several; an explicit mode keeps the persistent launch."""
    for nd in (32, 64, 96):
        spec = inputs.config_spec("batched", n_dec=nd)
        i = _spec_lists(spec).info()
        f = _spec_lists(spec, sched_mode=B.SCHED_SPLIT)
        assert i["one_unit_per_wg"] == 1 and i["sched_mode"] == B.SCHED_SPLIT, nd
        assert np.array_equal(_spec_lists(spec).export(0), f.export(0))
        assert f.info()["one_unit_per_wg"] == 0
    i = _spec_lists(inputs.config_spec("llama3_8b")).info()
    assert i["one_unit_per_wg"] == 1 and i["sched_mode"] == B.SCHED_COLOCATE


def test_gqa_small_prefill_share_runs_on_two_streams():
    """Automatic scheduling runs a GQA batch with several prefill requests,
    too many units for the one-unit launch and a prefill under 0.15 of the
    estimated work on two streams (runs_sequential 2); one prefill request,
    a larger share, MHA or an explicit mode keep their launch."""
    def routed(spec, **tun):
        p = B.make_params(spec.num_qo_heads, spec.num_kv_heads, spec.layout, spec.page_size,
                          spec.causal, spec.sm_scale, kv_dtype=spec.kv_dtype)
        t = B.make_tuning(**tun) if tun else None
        return B.plan_host(p, spec.prefill_qo_len, spec.prefill_kv_len, spec.decode_kv_len,
                           t).info()["runs_sequential"]
    assert routed(inputs.config_spec("batched")) == 2                    # share 0.09
    assert routed(inputs.config_spec("batched", n_dec=256)) == 2         # 0.11
    assert routed(inputs.config_spec("batched", n_dec=128)) == 0         # 0.17
    assert routed(inputs.config_spec("batched_fp8")) == 0                # 0.16
    assert routed(inputs.config_spec("batched", n_dec=64)) == 0          # one-unit launch
    assert routed(inputs.config_spec("batched"), sched_mode=B.SCHED_SPLIT) == 0
    rng = np.random.default_rng(13)
    one = inputs.custom_spec("one_chunk", 32, 8, [(512, 8192)],
                             list(rng.integers(512, 16384, 256)), seed=13)
    assert routed(one) == 0                                              # one request
