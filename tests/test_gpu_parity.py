"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Reduced-size batches of each workload shape (the oracle checks every row),
edge cases, split counts, page sizes, scheduler modes and bitwise scheduler
invariants.  Full-size workloads are checked on sampled rows in
test_gpu_fullsize.py."""

import math

import numpy as np
import pytest

import oracle
from prefill_decode_amd import binding as B
from prefill_decode_amd import inputs
from tests.gpu_util import bits, compare, run_path, say

pytestmark = pytest.mark.gpu

S = inputs.custom_spec


def reduced_specs():
    rng = np.random.default_rng(77)
    ln = np.clip(np.rint(300 * np.exp(rng.standard_normal(12))), 1, 2400).astype(int)
    return [
        inputs.config_spec("tiny"),
        S("llama3_8b_r", 32, 8, [(300, 1100)], list(rng.integers(1, 1500, 9, endpoint=True)),
          seed=101),
        S("llama2_7b_r", 32, 32, [(200, 900)], [700] * 6, seed=102),
        S("l70b_r", 64, 8, [(260, 1300)], list(ln), seed=103),
        S("batched_r", 32, 8, [(17, 40), (64, 300), (129, 129), (200, 777)],
          list(rng.integers(1, 2000, 20, endpoint=True)), seed=104),
    ]


def edge_specs():
    return [
        S("one_key", 4, 4, [(1, 1)], [1], seed=201, layout="contiguous", extra_pages=0),
        S("qo_eq_kv", 8, 2, [(190, 190)], [33], seed=202),
        S("only_prefill", 8, 8, [(257, 600)], [], seed=203),
        S("only_decode", 16, 4, [], [1, 2, 31, 32, 33, 1000], seed=204),
        S("gqa32", 64, 2, [(70, 150)], [300, 5], seed=205),         # 32 q heads / kv head
        S("mqa", 8, 1, [(40, 90)], [77], seed=206),
        S("noncausal", 8, 2, [(100, 333)], [64], seed=207, causal=False),
        S("many_req", 8, 2, [(3, 5)] * 7 + [(128, 128)], list(range(1, 41)), seed=208),
        S("page1", 8, 2, [(33, 70)], [65, 3], seed=209, page_size=1),
        S("page8", 8, 2, [(33, 70)], [65, 3], seed=210, page_size=8),
        S("page32", 8, 2, [(150, 300)], [65, 200], seed=211, page_size=32),
        S("page128", 8, 2, [(150, 300)], [65, 700], seed=212, page_size=128),
        S("contig", 16, 4, [(150, 400), (5, 9)], [100, 1, 513], seed=213,
          layout="contiguous", extra_pages=0),
    ]


def _check(spec, tuning=None, paths=("fused", "seq")):
    say(f"[parity] {spec.name} tuning={tuning}")
    b = inputs.make_batch_host(spec, poison=True)
    ref = oracle.batch_attention(b)
    runner = B.BatchRunner(b, tuning)
    outs = {}
    for path in paths:
        say(f"  path {path}")
        got = run_path(runner, path)
        compare(got, ref, f"{spec.name}/{path}")
        outs[path] = got
    return runner, outs


@pytest.mark.parametrize("spec", reduced_specs(), ids=lambda s: s.name)
def test_reduced_configs(spec):
    _check(spec)


@pytest.mark.parametrize("spec", edge_specs(), ids=lambda s: s.name)
def test_edge_cases(spec):
    _check(spec)


@pytest.mark.parametrize("spec", reduced_specs() + edge_specs()[:4], ids=lambda s: s.name)
def test_one_unit_per_workgroup(spec):
    # the fused launch of one workgroup per unit (split and co-located roles)
    for mode in (B.SCHED_SPLIT, B.SCHED_COLOCATE):
        _check(spec, B.make_tuning(sched_mode=mode, flags=B.FLAG_ONE_UNIT_PER_WG),
               paths=("fused",))


@pytest.mark.parametrize("spec", [inputs.config_spec("tiny"), reduced_specs()[1]],
                         ids=lambda s: s.name)
def test_sharp_scale(spec):
    # sm_scale = 1: peaked softmax, O = O(1); catches a dropped or extra key
    _check(inputs.with_scale(spec, 1.0))


@pytest.mark.parametrize("ps,ds", [(1, 1), (2, 2), (4, 4), (16, 64)])
def test_forced_splits(ps, ds):
    spec = reduced_specs()[1]
    _check(spec, B.make_tuning(prefill_kv_splits=ps, decode_kv_splits=ds))


_SHARP_REF = {}


@pytest.mark.parametrize("splits", [1, 2, 3, 4, 8, 16, 64])
@pytest.mark.parametrize("which", [0, 1, 4], ids=["tiny", "llama3_8b_r", "batched_r"])
def test_sharp_scale_forced_splits(which, splits):
    # sm_scale = 1 (a peaked softmax, O = O(1)) with every split count the
    # tuning accepts up to its cap, for prefill and decode at once: where a
    # row's splits nearly cancel, the partials' precision shows
    spec = inputs.with_scale(reduced_specs()[which], 1.0)
    say(f"[sharp-splits] {spec.name} splits {splits}")
    if spec.name not in _SHARP_REF:
        b = inputs.make_batch_host(spec, poison=True)
        _SHARP_REF[spec.name] = (b, oracle.batch_attention(b))
    b, ref = _SHARP_REF[spec.name]
    runner = B.BatchRunner(b, B.make_tuning(prefill_kv_splits=splits, decode_kv_splits=splits))
    for path in ("fused", "seq"):
        compare(run_path(runner, path), ref, f"{spec.name}/splits{splits}/{path}")


def test_fused_equals_matched_sequential_bitwise_and_sched_modes():
    spec = reduced_specs()[4]
    b = inputs.make_batch_host(spec)
    ref = oracle.batch_attention(b)
    results = []
    for mode, flags in ((B.SCHED_AUTO, 0), (B.SCHED_COLOCATE, 0), (B.SCHED_ORDERED, 0),
                        (B.SCHED_SPLIT, 0), (B.SCHED_SPLIT, B.FLAG_ONE_UNIT_PER_WG),
                        (B.SCHED_COLOCATE, B.FLAG_ONE_UNIT_PER_WG),
                        (B.SCHED_ORDERED, B.FLAG_ONE_UNIT_PER_WG)):
        for q in (1, 4, 7):
            say(f"[bitwise] mode={mode} flags={flags} quarters={q}")
            t = B.make_tuning(match_sequential=1, sched_mode=mode, prefill_quarters_per_cu=q,
                              prefill_kv_splits=2, decode_kv_splits=3, flags=flags)
            r = B.BatchRunner(b, t)
            f1 = run_path(r, "fused")
            f2 = run_path(r, "fused")
            s1 = run_path(r, "seq")
            compare(f1, ref, "bitwise-case")
            for k in f1:
                assert np.array_equal(f1[k], f2[k]), ("rerun", k)
                assert np.array_equal(f1[k], s1[k]), ("fused vs sequential", k)
            results.append(f1)
    for other in results[1:]:
        for k in results[0]:
            assert np.array_equal(results[0][k], other[k]), k


def test_page_order_invariance():
    # same tokens, identity vs random page order: bitwise equal outputs
    base = S("perm", 8, 2, [(100, 500)], [300, 17], seed=301, random_pages=True)
    ident = S("perm", 8, 2, [(100, 500)], [300, 17], seed=301, random_pages=False)
    bp, bi = inputs.make_batch_host(base), inputs.make_batch_host(ident)
    # rebuild the identity batch's pool from the permuted one so tokens agree
    for r in range(3):
        a0, a1 = bp["page_indptr"][r], bp["page_indptr"][r + 1]
        bi["k_cache"][bi["page_indices"][a0:a1]] = bp["k_cache"][bp["page_indices"][a0:a1]]
        bi["v_cache"][bi["page_indices"][a0:a1]] = bp["v_cache"][bp["page_indices"][a0:a1]]
    outs = []
    for b in (bp, bi):
        outs.append(run_path(B.BatchRunner(b), "fused"))
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[1][k]), k


def test_decode_row_equals_last_prefill_row():
    L, n = 1000, 77
    spec = S("dl", 16, 4, [(n, L)], [L], seed=302, layout="contiguous", extra_pages=0)
    b = inputs.make_batch_host(spec)
    b["q_decode"][0] = b["q_prefill"][n - 1]
    b["k_cache"][L:2 * L] = b["k_cache"][0:L]
    b["v_cache"][L:2 * L] = b["v_cache"][0:L]
    got = run_path(B.BatchRunner(b), "fused")
    d = np.abs(got["o_decode"][0] - got["o_prefill"][n - 1])
    assert np.all(d <= 5e-3 + 1e-2 * np.abs(got["o_prefill"][n - 1]))
    assert np.all(np.abs(got["lse_decode"][0] - got["lse_prefill"][n - 1]) <= 1e-3)


def test_boundary_probe():
    # key at each probed row's own position dominates; a larger key one step
    # in the future must stay invisible (off-by-one masks fail by O(1))
    spec = S("probe", 4, 4, [(128, 400)], [], seed=303, layout="contiguous", extra_pages=0,
             sm_scale=1.0 / math.sqrt(128))
    b = inputs.make_batch_host(spec)
    q = (b["q_prefill"].astype(np.uint32) << 16).view(np.float32)
    rows = [0, 31, 32, 63, 64, 100, 127]
    kf = (b["k_cache"].astype(np.uint32) << 16).view(np.float32) * 0.05
    for i in rows:
        pos = 400 - 128 + i
        for h in range(4):
            u = q[i, h] / np.linalg.norm(q[i, h])
            kf[pos, h] = 40.0 * u
            if pos + 1 < 400:
                kf[pos + 1, h] = 80.0 * u
    b["k_cache"] = inputs.f32_to_bf16_bits(kf)
    # other rows see the planted keys too; compare only probed rows to V
    got = run_path(B.BatchRunner(b), "fused")
    v = (b["v_cache"].astype(np.uint32) << 16).view(np.float32)
    ref = oracle.batch_attention(b)
    compare(got, ref, "probe")
    for i in rows:
        pos = 400 - 128 + i
        for h in range(4):
            assert np.max(np.abs(got["o_prefill"][i, h] - v[pos, h])) < 0.05, (i, h)


def test_hwid_probe_and_workspace_error():
    import torch
    ids = B.probe_hwid(4096)
    hw, xcc = ids[:, 0].astype(np.int64), ids[:, 1].astype(np.int64)
    slots = ((xcc & 7) << 8) | (((hw >> 13) & 7) << 5) | (((hw >> 12) & 1) << 4) | ((hw >> 8) & 0xF)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    say(f"[probe] distinct slots {len(set(slots.tolist()))}, CUs {n_cu}, "
        f"xcc ids {sorted(set((xcc & 15).tolist()))}")
    assert len(set(slots.tolist())) == n_cu
    assert len(set((xcc & 15).tolist())) == 8
    # too small a workspace is an error, not a fault
    import ctypes as C
    p = B.make_params(8, 2)
    qo = np.array([64], np.int32)
    kv = np.array([200], np.int32)
    dk = np.array([50], np.int32)
    need = C.c_size_t(0)
    lib = B.lib()
    st = lib.pod_attn_plan(C.byref(p), 1, B._ptr(qo), B._ptr(kv), 1, B._ptr(dk), None, None, 0,
                           C.byref(need), None, None)
    assert st == 0 and need.value > 0
    ws = torch.empty(need.value, dtype=torch.uint8, device="cuda")
    h = C.c_void_p(0)
    st = lib.pod_attn_plan(C.byref(p), 1, B._ptr(qo), B._ptr(kv), 1, B._ptr(dk), None,
                           C.c_void_p(ws.data_ptr()), need.value - 256, C.byref(need), None,
                           C.byref(h))
    assert st == 3 and not h.value


def test_graph_replays_match_eager():
    # A run recorded into a HIP graph uses the self-resetting counter block;
    # every replay (with eager runs in between) must equal the eager result.
    import torch
    spec = reduced_specs()[4]
    b = inputs.make_batch_host(spec)
    r = B.BatchRunner(b)
    ref = run_path(r, "fused")
    compare(ref, oracle.batch_attention(b), "graph-eager")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        r.run()
    torch.cuda.synchronize()
    for i in range(3):
        say(f"[graph] replay {i}")
        for t in (r.o_prefill, r.o_decode, r.lse_prefill, r.lse_decode):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = r.outputs()
        for k in ref:
            assert np.array_equal(got[k], ref[k]), ("replay", i, k)
        eager = run_path(r, "fused")
        for k in ref:
            assert np.array_equal(eager[k], ref[k]), ("eager after replay", i, k)


@pytest.mark.parametrize("which", [2, 3], ids=["only_prefill", "only_decode"])
def test_single_kind_batch(which):
    """A batch of one kind has nothing to overlap: pod_attn_run runs the one
    kernel it needs with the sequential plan's lists (bitwise the sequential
    result); a traced plan keeps the fused launch (its trace covers every
    unit), and both match the oracle."""
    spec = edge_specs()[which]
    say(f"[single kind] {spec.name}")
    b = inputs.make_batch_host(spec, poison=True)
    ref = oracle.batch_attention(b)
    r = B.BatchRunner(b)
    f, s = run_path(r, "fused"), run_path(r, "seq")
    compare(f, ref, f"{spec.name}/fused")
    for k in f:
        assert np.array_equal(f[k], s[k]), k
    rt = B.BatchRunner(b, B.make_tuning(flags=B.FLAG_TRACE))
    ft = run_path(rt, "fused")
    compare(ft, ref, f"{spec.name}/fused traced")
    tr = rt.plan.read_trace()
    info = rt.plan.info()
    assert len(tr) == info["trace_records"] == info["prefill_items"] + info["decode_items"] > 0
    assert np.all(tr[:, 5] >= tr[:, 4]) and np.all(tr[:, 4] > 0)     # t_end >= t_start > 0


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_mha_small_prefill_runs_sequentially(kv_dtype):
    """An MHA batch with a small prefill share: pod_attn_run runs the two
    kernels back to back (bitwise the sequential result); an explicit
    scheduler mode keeps the fused launch; both match the oracle."""
    spec = S(f"mha_routed_{kv_dtype}", 32, 32, [(64, 2048)], [1024] * 128, seed=231,
             kv_dtype=kv_dtype)
    say(f"[routed] {spec.name}")
    b = inputs.make_batch_host(spec, poison=True)
    ref = oracle.batch_attention(b)
    r = B.BatchRunner(b)
    assert r.plan.info()["runs_sequential"] == 1
    f, s_ = run_path(r, "fused"), run_path(r, "seq")
    compare(f, ref, f"{spec.name}/fused (routed)")
    for k in f:
        assert np.array_equal(f[k], s_[k]), k
    rf = B.BatchRunner(b, B.make_tuning(sched_mode=B.SCHED_SPLIT))
    assert rf.plan.info()["runs_sequential"] == 0
    compare(run_path(rf, "fused"), ref, f"{spec.name}/fused launch")


def test_empty_batch_every_entry_point():
    """A batch with no request plans and runs on every path as a no-op: no
    launch, status OK, and an unrelated canary on the stream is untouched."""
    import torch
    spec = S("empty", 8, 2, [], [], seed=301)
    say("[empty] plan and run an empty batch on every path")
    b = inputs.make_batch_host(spec)
    r = B.BatchRunner(b, B.make_tuning(flags=B.FLAG_BATCHED_PREFILL))
    info = r.plan.info()
    assert info["prefill_items"] == info["decode_items"] == info["merge_tasks"] == 0
    canary = torch.full((1024,), 7.0, device="cuda")
    for path in ("fused", "seq", "streams", "batched"):
        got = run_path(r, path)
        assert all(v.size == 0 for v in got.values()), path
    torch.cuda.synchronize()
    assert bool((canary == 7.0).all())
