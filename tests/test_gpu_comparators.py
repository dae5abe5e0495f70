"""GPU parity of the merge kernel on its own and of the pages' comparators.

* pod_attn_merge against the oracle's log-sum-exp merge on injected partials:
  empty (-inf) splits, rows with every split empty, a single split, split
  counts up to the 64 the kernel takes, partials of very different weight.
* The two-stream comparator (prefill and decode kernels on two streams) and
  the batched-prefill comparator (decodes as one-row chunks through the
  prefill kernel) against the fp64 oracle on reduced workloads; the
  two-stream run is bitwise equal to the sequential run (same kernels, same
  work lists)."""

import numpy as np
import pytest

import oracle
from prefill_decode_amd import binding as B
from prefill_decode_amd import inputs
from tests.gpu_util import compare, run_path, say
from tests.test_gpu_parity import edge_specs, reduced_specs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16, 33, 64])
def test_merge_kernel_against_oracle(splits):
    import torch
    say(f"[merge] splits {splits}")
    rng = np.random.default_rng(400 + splits)
    rows = 301                                   # ragged against the 16-row workgroup
    part_o = rng.standard_normal((rows, splits, 128))
    lse = rng.normal(0.0, 4.0, (rows, splits))   # weights spanning many orders
    # empty splits: random ones, a whole split column, and every split of some rows
    lse[rng.random((rows, splits)) < 0.2] = -np.inf
    if splits > 1:
        lse[:, splits // 2] = -np.inf
    lse[[0, 17, rows - 1]] = -np.inf
    po = torch.from_numpy(part_o.astype(np.float32)).cuda()
    pl = torch.from_numpy(lse.astype(np.float32)).cuda()
    o = torch.full((rows, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    lo = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    B.merge(po, pl, o, lo)
    torch.cuda.synchronize()
    # the oracle merges the same fp32 values (exact in fp64)
    ref_o, ref_l = oracle.merge_partials(
        [(part_o.astype(np.float32).astype(np.float64)[:, s],
          lse.astype(np.float32).astype(np.float64)[:, s]) for s in range(splits)])
    got_o = o.float().cpu().double().numpy()
    got_l = lo.cpu().double().numpy()
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(got_l), empty)
    assert np.all(got_o[empty] == 0.0)
    fin = ~empty
    assert np.all(np.abs(got_o[fin] - ref_o[fin]) <= 5e-3 + 1e-2 * np.abs(ref_o[fin]))
    # a bf16 output rounds at 2^-9 relative; the LSE is fp32 throughout
    assert np.all(np.abs(got_o[fin] - ref_o[fin]) <= 2.0 ** -8 * np.abs(ref_o[fin]) + 1e-6)
    assert np.all(np.abs(got_l[fin] - ref_l[fin]) <= 1e-5 * np.maximum(1.0, np.abs(ref_l[fin])))


def test_merge_rejects_bad_arguments():
    import ctypes as C
    import torch
    lib = B.lib()
    x = torch.zeros(16, dtype=torch.float32, device="cuda")
    assert lib.pod_attn_merge(C.c_void_p(x.data_ptr()), C.c_void_p(x.data_ptr()), 1, 65,
                              C.c_void_p(x.data_ptr()), None, None) == 1
    assert lib.pod_attn_merge(C.c_void_p(x.data_ptr()), C.c_void_p(x.data_ptr()), 1, 0,
                              C.c_void_p(x.data_ptr()), None, None) == 1
    assert lib.pod_attn_merge(None, C.c_void_p(x.data_ptr()), 1, 2,
                              C.c_void_p(x.data_ptr()), None, None) == 1
    assert lib.pod_attn_merge(C.c_void_p(x.data_ptr() + 4), C.c_void_p(x.data_ptr()), 1, 2,
                              C.c_void_p(x.data_ptr()), None, None) == 1
    # zero rows: nothing to do
    assert lib.pod_attn_merge(None, None, 0, 2, None, None, None) == 0


def _cases():
    return reduced_specs() + [s for s in edge_specs()
                              if s.name in ("only_decode", "only_prefill", "gqa32", "mqa",
                                            "noncausal", "many_req", "page1", "contig")]


@pytest.mark.parametrize("spec", _cases(), ids=lambda s: s.name)
def test_comparators_against_oracle(spec):
    say(f"[comparators] {spec.name}")
    b = inputs.make_batch_host(spec, poison=True)
    ref = oracle.batch_attention(b)
    runner = B.BatchRunner(b, B.make_tuning(flags=B.FLAG_BATCHED_PREFILL))
    seq = run_path(runner, "seq")
    compare(seq, ref, f"{spec.name}/seq")
    for path in ("streams", "batched"):
        say(f"  path {path}")
        got = run_path(runner, path)
        compare(got, ref, f"{spec.name}/{path}")
        if path == "streams":
            for k in got:
                assert np.array_equal(got[k], seq[k]), ("streams vs sequential", k)


@pytest.mark.parametrize("ps", [1, 3, 64])
def test_batched_prefill_forced_splits(ps):
    spec = reduced_specs()[1]
    say(f"[batched-prefill] splits {ps}")
    b = inputs.make_batch_host(inputs.with_scale(spec, 1.0), poison=True)
    ref = oracle.batch_attention(b)
    runner = B.BatchRunner(b, B.make_tuning(flags=B.FLAG_BATCHED_PREFILL, prefill_kv_splits=ps))
    compare(run_path(runner, "batched"), ref, f"batched-prefill splits {ps}")


def test_batched_prefill_needs_its_flag():
    spec = reduced_specs()[0]
    runner = B.BatchRunner(inputs.make_batch_host(spec))
    with pytest.raises(B.PodError) as e:
        runner.batched_prefill_run()
    assert e.value.status == 1


def test_gqa_small_prefill_runs_on_two_streams():
    """The batched mix at full size (four prefill requests, a prefill share
    of 0.09): pod_attn_run runs the prefill and decode kernels at once on two
    streams.  Its outputs equal pod_attn_streams_run's and the sequential
    run's bitwise (same kernels, same lists), match the fp64 oracle on
    sampled rows, and a graph capture of it (the fork onto the library's
    second stream and the join inside the capture) replays to the same bits,
    with eager runs between the replays."""
    import torch
    spec = inputs.config_spec("batched")
    say("[two-stream route] batched: generating on device")
    bd = inputs.make_batch_device(spec, poison=True)
    r = B.BatchRunner(bd)
    assert r.plan.info()["runs_sequential"] == 2
    fused = run_path(r, "fused")
    for path in ("streams", "seq"):
        other = run_path(r, path)
        for k in fused:
            assert np.array_equal(fused[k], other[k]), (path, k)
    rows = [0, 127, 128, 383, 384, 895, 896, 1535]
    dec = [0, 1, 95, 191]
    sub = inputs.host_subset(bd, list(range(spec.num_prefill)), dec)
    ref = oracle.sample_batch_attention(sub, rows, list(range(len(dec))))
    compare({"o_prefill": fused["o_prefill"][rows], "lse_prefill": fused["lse_prefill"][rows],
             "o_decode": fused["o_decode"][dec], "lse_decode": fused["lse_decode"][dec]},
            ref, "batched/two-stream route")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        r.run()
    torch.cuda.synchronize()
    for i in range(3):
        say(f"  graph replay {i}")
        for t in (r.o_prefill, r.o_decode, r.lse_prefill, r.lse_decode):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = r.outputs()
        for k in fused:
            assert np.array_equal(got[k], fused[k]), ("replay", i, k)
        eager = run_path(r, "fused")
        for k in fused:
            assert np.array_equal(eager[k], fused[k]), ("eager after replay", i, k)
    f = B.BatchRunner(bd, B.make_tuning(sched_mode=B.SCHED_SPLIT))
    assert f.plan.info()["runs_sequential"] == 0
    del r, f, bd
    torch.cuda.empty_cache()


def test_paths_interleaved_keep_their_counters():
    """Runs of every path of one plan, interleaved (fused, two streams, fused,
    sequential, batched prefill, fused): each fused run finds its counter
    block zeroed whatever ran before it, so every fused output is the same
    and matches the oracle (a counter block left dirty by another path would
    make the fused kernel skip its work)."""
    spec = reduced_specs()[1]
    say(f"[interleaved paths] {spec.name}")
    b = inputs.make_batch_host(spec, poison=True)
    ref = oracle.batch_attention(b)
    r = B.BatchRunner(b, B.make_tuning(flags=B.FLAG_BATCHED_PREFILL, sched_mode=B.SCHED_SPLIT))
    first = run_path(r, "fused")
    compare(first, ref, f"{spec.name}/fused")
    for path in ("streams", "fused", "seq", "batched", "fused", "fused"):
        got = run_path(r, path)
        compare(got, ref, f"{spec.name}/{path}")
        if path == "fused":
            for k in first:
                assert np.array_equal(got[k], first[k]), (path, k)
