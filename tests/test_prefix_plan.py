"""Shared-prefix (PAT-style) decode plans, on the CPU.

The packed lists come from pod_attn_plan_shared_prefix_host.  Their meaning
(include/pod_attn.h): a unit's row j is query head h0 + j % rpr of decode
request members[D_QROW + j / rpr], rpr = min(Hq/Hkv, 16); it reads keys
[kb, ke) through request D_KVREQ's page table and writes partial slot
D_PART + (j / rpr) Hq D_PSTRIDE + (j % rpr) D_PSTRIDE; merge tasks combine
each (request, head)'s slots.  The tests check that every (request, head)'s
keys are covered once, that prefix units are shared by the members ([PAT]
abstract: the prefix's KV is loaded once per pack of queries), and -- on a
small batch -- that running the lists with the oracle's partial and merge
arithmetic reproduces the oracle's attention (the lists decide which pages
each unit reads, so a wrong page table or a wrong slot shows up here).
"""

import numpy as np
import pytest

import oracle
from oracle import attention as OA
from prefill_decode_amd import binding as B
from prefill_decode_amd import inputs

D_F, M_F = 8, 4


def _params(spec):
    return B.make_params(spec.num_qo_heads, spec.num_kv_heads, spec.layout, spec.page_size,
                         spec.causal, spec.sm_scale)


def _groups(spec):
    nd = len(spec.decode_kv_len)
    grp = np.full(nd, -1, dtype=np.int32)
    plen = []
    for gi, (members, pl) in enumerate(spec.prefix_groups):
        grp[list(members)] = gi
        plen.append(pl)
    return grp, plen


def _host_plan(spec, **tun):
    grp, plen = _groups(spec)
    t = B.make_tuning(**tun) if tun else None
    return B.plan_shared_prefix_host(_params(spec), spec.decode_kv_len, grp, plen, t)


def _spec(name, hq, hkv, dkv, groups, seed=5, page_size=16, **kw):
    return inputs.custom_spec(name, hq, hkv, [], dkv, seed=seed, page_size=page_size,
                              prefix_groups=tuple((tuple(m), p) for m, p in groups), **kw)


def _units(spec, pl):
    """Per (request, head): list of (kb, ke, kvreq, slot) from the packed lists."""
    hq, hkv = spec.num_qo_heads, spec.num_kv_heads
    rpr = min(hq // hkv, 16)
    T = pl.export(0).reshape(-1, D_F)          # prefix tiles (<= 64 rows)
    D = pl.export(1).reshape(-1, D_F)          # suffix units (<= 16 rows)
    mem = pl.export(11)
    per = {}
    for it, cap in [(t, 64) for t in T] + [(d, 16) for d in D]:
        q0, h0, nq, kb, ke, kvreq, part, ps = (int(x) for x in it)
        assert 1 <= nq <= cap and 0 <= kb < ke
        for j in range(nq):
            r = int(mem[q0 + j // rpr])
            h = h0 + j % rpr
            assert h // (hq // hkv) == h0 // (hq // hkv)        # one KV head per unit
            slot = part + (j // rpr) * hq * ps + (j % rpr) * ps
            per.setdefault((r, h), []).append((kb, ke, kvreq, slot))
    return per, np.concatenate([T, D]), mem


CASES = [
    # (name, hq, hkv, decode kv lens, groups [(members, prefix)])
    ("g8_two_groups", 32, 4, [100, 130, 97, 260, 64, 200, 33],
     [((0, 1, 2), 96), ((3, 5), 192)]),
    ("g4_one_big_group", 16, 4, [80 + 7 * i for i in range(9)], [(tuple(range(9)), 80)]),
    ("g1_mha", 8, 8, [48, 49, 50, 200], [((0, 1, 2), 48)]),
    ("g16", 32, 2, [300, 301, 40], [((0, 1), 288)]),
    ("g32_two_chunks", 64, 2, [70, 90], [((0, 1), 64)]),
    ("g24_partial_chunk", 48, 2, [64, 70, 80, 96, 65], [((0, 1, 2, 3, 4), 64)]),
    ("g8_big_group", 32, 4, [100 + i for i in range(20)], [(tuple(range(20)), 96)]),
    ("g6_ragged_pack", 12, 2, [64, 65, 66, 67, 68], [((0, 1, 2, 3, 4), 64)]),
    ("prefix_is_all", 16, 2, [64, 64, 64], [((0, 1, 2), 64)]),
    ("ungrouped_only", 16, 2, [64, 65], []),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("splits", [0, 3])
def test_prefix_lists_cover_keys_once(case, splits):
    name, hq, hkv, dkv, groups = case
    spec = _spec(name, hq, hkv, dkv, groups)
    pl = _host_plan(spec, decode_kv_splits=splits) if splits else _host_plan(spec)
    per, D, mem = _units(spec, pl)
    n_partials = pl.info()["num_partials"]
    grp, plen = _groups(spec)
    used = np.zeros(max(n_partials, 1), dtype=np.int32)
    nd = len(dkv)
    assert sorted(per) == [(r, h) for r in range(nd) for h in range(hq)]
    for (r, h), us in per.items():
        us = sorted(us)
        assert us[0][0] == 0 and us[-1][1] == dkv[r]
        for a, b in zip(us[:-1], us[1:]):
            assert a[1] == b[0]
        P = plen[grp[r]] if grp[r] >= 0 else 0
        for kb, ke, kvreq, slot in us:
            # a unit lies wholly in the prefix or wholly in the own keys
            assert ke <= P or kb >= P
            if ke <= P:
                # the prefix is read through a member of the same group
                assert grp[kvreq] == grp[r]
            else:
                assert kvreq == r
            assert 0 <= slot < n_partials and used[slot] == 0
            used[slot] = 1
    # merge tasks: one per (request, head), exactly its slots
    M = pl.export(2).reshape(-1, M_F)
    assert len(M) == nd * hq
    for out, base, stride, nf in (tuple(int(x) for x in t) for t in M):
        n, dec = nf & 0xFFFF, nf >> 16
        assert dec == 1 and 1 <= n <= 64
        r, h = divmod(out, hq)
        slots = sorted(base + s * stride for s in range(n))
        assert slots == sorted(u[3] for u in per[(r, h)])
        for s_ in slots:
            assert used[s_] == 1
            used[s_] = 2
    assert np.all(used[:n_partials] != 1)


def test_prefix_units_are_shared_by_the_pack():
    # g = 4: rpr 4, sixteen members per 64-row workgroup tile; a group of 9
    # members over a 160-token prefix is one tile (36 rows) per KV head and
    # split, so each prefix key is read once per KV head, not once per member
    spec = _spec("pack", 16, 4, [200] * 9 + [150], [(tuple(range(9)), 160)])
    pl = _host_plan(spec, decode_kv_splits=2)
    T = pl.export(0).reshape(-1, D_F)
    assert len(T) == 4 * 2
    assert all(int(x) == 36 for x in T[:, 2])
    assert int((T[:, 4] - T[:, 3]).sum()) == 4 * 160
    D = pl.export(1).reshape(-1, D_F)
    assert np.all(D[:, 2] <= 4) and not np.any((D[:, 5] < 9) & (D[:, 3] < 160))
    # g = 24 (a partial block of 8 heads per KV head): full blocks pack four
    # members, the partial block one member per tile
    spec = _spec("g24", 48, 2, [64] * 5, [(tuple(range(5)), 64)])
    T = _host_plan(spec, decode_kv_splits=1).export(0).reshape(-1, D_F)
    rows = sorted(int(x) for x in T[:, 2])
    assert rows == [8] * 10 + [16, 16, 64, 64]


def test_prefix_plan_rejects_bad_groups():
    spec = _spec("bad", 16, 2, [64, 80], [((0, 1), 64)])
    p = _params(spec)
    bad = [([0, 2], [64]),          # group id out of range
           ([0, -2], [64]),         # below -1
           ([0, 0], [80]),          # longer than member 0
           ([0, 0], [0]),           # empty prefix
           ([0, 0], [24])]          # not whole pages
    for grp, plen in bad:
        with pytest.raises(B.PodError, match=B.STATUS[1]):
            B.plan_shared_prefix_host(p, [64, 80], grp, plen)
    pc = B.make_params(16, 2, "contiguous", 16, True, spec.sm_scale)
    with pytest.raises(B.PodError, match=B.STATUS[2]):
        B.plan_shared_prefix_host(pc, [64, 80], [0, 0], [64])
    with pytest.raises(B.PodError, match=B.STATUS[2]):
        B.plan_shared_prefix_host(p, [64, 80], [0, 0], [64],
                                  B.make_tuning(flags=B.FLAG_BATCHED_PREFILL))


def test_tile_splits_follow_the_work_share():
    # 128 base tiles (16 groups x 8 KV heads); 512 workgroup slots.  Tiles take
    # the slots' share that their work has (a tile wave-key at half a suffix
    # unit's): a long prefix with short suffixes fills every slot, a short
    # prefix with long suffixes keeps one tile per pack
    def count(plen, own):
        groups = [(tuple(range(8 * g, 8 * g + 8)), plen) for g in range(16)]
        spec = _spec("w", 64, 8, [plen + own] * 128, groups)
        return _host_plan(spec).info()["prefill_items"]
    assert count(4096, 64) == 512
    assert count(2048, 544) == 256
    assert count(512, 2560) == 128


def test_page_table_shares_prefix_pages():
    spec = _spec("pages", 16, 2, [64, 80, 100, 40], [((0, 1, 2), 48)], page_size=16)
    ind, idx, pool = inputs.page_table(spec)
    pages = [idx[ind[r]:ind[r + 1]] for r in range(4)]
    assert np.array_equal(pages[0][:3], pages[1][:3]) and np.array_equal(pages[0][:3], pages[2][:3])
    # every other page belongs to one request only
    own = np.concatenate([pages[0], pages[1][3:], pages[2][3:], pages[3]])
    assert len(np.unique(own)) == len(own)
    assert pool == len(own) + spec.extra_pages
    with pytest.raises(ValueError):
        inputs.page_table(_spec("p2", 16, 2, [64, 80], [((0, 1), 40)]))
    with pytest.raises(ValueError):
        inputs.page_table(_spec("p3", 16, 2, [32, 80], [((0, 1), 48)]))


@pytest.mark.parametrize("case", [CASES[0], CASES[2], CASES[5], CASES[6]], ids=lambda c: c[0])
def test_lists_reproduce_the_oracle(case):
    """Execute the packed lists with the oracle's split and merge arithmetic."""
    name, hq, hkv, dkv, groups = case
    spec = _spec(name, hq, hkv, dkv, groups, seed=11)
    batch = inputs.make_batch_host(spec)
    ref = oracle.batch_attention(batch, workers=1)
    pl = _host_plan(spec, decode_kv_splits=2)
    per, _, _ = _units(spec, pl)
    scale = float(batch["sm_scale"])
    for (r, h), us in per.items():
        q = OA.bf16_bits_to_f64(batch["q_decode"][r:r + 1, h:h + 1])      # [1, 1, d]
        kvh = h // (hq // hkv)
        parts = []
        for kb, ke, kvreq, _ in us:
            k, v = OA.gather_request_kv(batch, kvreq, ke)
            parts.append(OA.attention_partial(q, [dkv[r] - 1], k[:, kvh:kvh + 1],
                                              v[:, kvh:kvh + 1], True, scale, kb, ke))
        o, lse = OA.merge_partials(parts)
        np.testing.assert_allclose(o[0, 0], ref["o_decode"][r, h], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, 0], ref["lse_decode"][r, h], rtol=0, atol=1e-12)
