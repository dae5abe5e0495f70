"""pod_attn_plan_scratch: the plan whose workspace is the library's static
device scratch (for callers that cannot allocate device memory), against
pod_attn_plan with a caller-allocated workspace.

Two scratch plans in a row on one device, the second smaller than the first
(so stale counters, lists or partials of the first would show), each run on
the fused and the sequential path: outputs bitwise equal to the workspace
plan's and within the parity bar of the fp64 oracle.  A plan larger than the
scratch is refused with the size it needs."""

import math

import numpy as np
import pytest

import oracle
from prefill_decode_amd import binding as B
from prefill_decode_amd import inputs
from tests.gpu_util import compare, run_path, say

pytestmark = pytest.mark.gpu

S = inputs.custom_spec


def _run_plan(runner, plan, path):
    import torch
    for t in (runner.o_prefill, runner.o_decode, runner.lse_prefill, runner.lse_decode):
        t.fill_(float("nan"))
    if path == "fused":
        B.run(plan, runner.tensors)
    else:
        B.sequential_run(plan, runner.tensors)
    torch.cuda.synchronize()
    return runner.outputs()


def test_scratch_plan_matches_workspace_plan_twice():
    specs = [S("scratch_big", 32, 8, [(300, 1100), (64, 300)], [1, 17, 700, 1500, 33], seed=501),
             S("scratch_small", 8, 2, [(40, 90)], [5, 64], seed=502)]
    for spec in specs:
        say(f"[scratch] {spec.name}")
        b = inputs.make_batch_host(spec, poison=True)
        ref = oracle.batch_attention(b)
        runner = B.BatchRunner(b)                      # workspace plan (caller memory)
        plan = B.plan_scratch(runner.params, spec.prefill_qo_len, spec.prefill_kv_len,
                              spec.decode_kv_len)
        assert plan.info()["workspace_bytes"] == runner.plan.info()["workspace_bytes"]
        for path in ("fused", "seq"):
            want = run_path(runner, path)
            got = _run_plan(runner, plan, path)
            compare(got, ref, f"{spec.name}/scratch/{path}")
            for k in want:
                assert np.array_equal(got[k], want[k]), (spec.name, path, k)
        # a second run of the same scratch plan (counters of the next parity)
        got = _run_plan(runner, plan, "fused")
        compare(got, ref, f"{spec.name}/scratch/fused-again")
        plan.destroy()


def test_scratch_plan_too_large_is_refused():
    spec = inputs.config_spec("l70b_tp1")
    p = B.make_params(spec.num_qo_heads, spec.num_kv_heads, spec.layout, spec.page_size,
                      spec.causal, 1.0 / math.sqrt(128))
    with pytest.raises(B.PodError) as e:
        B.plan_scratch(p, spec.prefill_qo_len, spec.prefill_kv_len, spec.decode_kv_len)
    assert e.value.status == 3 and "static scratch" in str(e.value)


def test_scratch_plan_keeps_the_fused_launch_for_two_stream_batches():
    """A batch pod_attn_plan runs on two streams (the batched mix) runs the
    fused launch from a scratch plan (which creates no stream), with the same
    results as the workspace plan's two-stream run within the parity bar."""
    import torch
    spec = inputs.config_spec("batched")
    say("[scratch] batched: generating on device")
    bd = inputs.make_batch_device(spec, poison=True)
    runner = B.BatchRunner(bd)
    assert runner.plan.info()["runs_sequential"] == 2
    plan = B.plan_scratch(runner.params, spec.prefill_qo_len, spec.prefill_kv_len,
                          spec.decode_kv_len)
    assert plan.info()["runs_sequential"] == 0
    want = run_path(runner, "fused")
    got = _run_plan(runner, plan, "fused")
    rows = [0, 127, 128, 383, 384, 895, 896, 1535]
    dec = [0, 1, 95, 191]
    sub = inputs.host_subset(bd, list(range(spec.num_prefill)), dec)
    ref = oracle.sample_batch_attention(sub, rows, list(range(len(dec))))
    for g in (want, got):
        compare({"o_prefill": g["o_prefill"][rows], "lse_prefill": g["lse_prefill"][rows],
                 "o_decode": g["o_decode"][dec], "lse_decode": g["lse_decode"][dec]},
                ref, "batched/scratch")
        for k in g:
            assert np.all(np.isfinite(g[k])), k
    plan.destroy()
    del runner, bd
    torch.cuda.empty_cache()
