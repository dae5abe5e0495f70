"""GPU parity of the FP8 E4M3 KV-cache decode path (per-KV-head scales)
against the fp64 oracle on the decoded values.

Decode-only batches (the path's scope): MHA and GQA packings of 1 to 32
query heads per KV head, contiguous and paged caches, lengths around the
32-key step and the 16-key block, forced KV splits, a sharp softmax, NaN in
every cache slot no token owns; every run entry point; and the decodes of
the llama2-7b and 70B-shaped layers at full size, every row."""

import numpy as np
import pytest

import oracle
from prefill_decode_amd import binding as B
from prefill_decode_amd import inputs
from tests.gpu_util import compare, run_path, say

pytestmark = pytest.mark.gpu

S = inputs.custom_spec
F8 = dict(kv_dtype="fp8_e4m3")


def fp8_specs():
    rng = np.random.default_rng(91)
    return [
        S("f8_mha", 8, 8, [], [1, 31, 32, 33, 512, 700], seed=601, **F8),
        S("f8_gqa4", 32, 8, [], list(rng.integers(1, 3000, 12, endpoint=True)), seed=602, **F8),
        S("f8_gqa8", 64, 8, [], [17, 4096, 1500, 63], seed=603, **F8),
        S("f8_gqa32", 64, 2, [], [300, 5, 2048], seed=604, **F8),
        S("f8_mqa", 8, 1, [], [77, 1000], seed=605, **F8),
        S("f8_contig", 16, 4, [], [100, 1, 513], seed=606, layout="contiguous", extra_pages=0, **F8),
        S("f8_page64", 16, 4, [], [65, 200, 1000], seed=607, page_size=64, **F8),
    ]


@pytest.mark.parametrize("spec", fp8_specs(), ids=lambda s: s.name)
def test_fp8_decode_against_oracle(spec):
    say(f"[fp8] {spec.name}")
    b = inputs.make_batch_host(spec, poison=True)
    ref = oracle.batch_attention(b)
    runner = B.BatchRunner(b)
    outs = {}
    for path in ("fused", "seq", "streams"):
        outs[path] = run_path(runner, path)
        compare(outs[path], ref, f"{spec.name}/{path}")
    # one kernel serves every path: the fused-plan and sequential-plan lists
    # may split differently, but with the plans matched the outputs agree bitwise
    rm = B.BatchRunner(b, B.make_tuning(match_sequential=1))
    f, s = run_path(rm, "fused"), run_path(rm, "seq")
    for k in f:
        assert np.array_equal(f[k], s[k]), k


@pytest.mark.parametrize("splits", [1, 3, 16])
def test_fp8_forced_splits_sharp(splits):
    spec = inputs.with_scale(fp8_specs()[1], 1.0)
    say(f"[fp8] sharp, splits {splits}")
    b = inputs.make_batch_host(spec, poison=True)
    ref = oracle.batch_attention(b)
    runner = B.BatchRunner(b, B.make_tuning(decode_kv_splits=splits))
    for path in ("fused", "seq"):
        compare(run_path(runner, path), ref, f"fp8 sharp splits {splits}/{path}")


def test_fp8_plan_rejections():
    p = B.make_params(8, 2, kv_dtype="fp8_e4m3")
    with pytest.raises(B.PodError) as e:                      # prefill on an FP8 cache
        B.plan(p, [4], [9], [5])
    assert e.value.status == 2
    with pytest.raises(B.PodError) as e:                      # pages of 8 tokens
        B.plan(B.make_params(8, 2, page_size=8, kv_dtype="fp8_e4m3"), [], [], [5])
    assert e.value.status == 2
    with pytest.raises(B.PodError) as e:                      # batched prefill comparator
        B.plan(p, [], [], [5], B.make_tuning(flags=B.FLAG_BATCHED_PREFILL))
    assert e.value.status == 2


@pytest.mark.parametrize("name", ["llama2_7b", "l70b_tp1"])
def test_fp8_fullsize_decodes_every_row(name):
    import dataclasses
    import torch
    base = inputs.config_spec(name)
    spec = dataclasses.replace(base, name=base.name + "_fp8dec", prefill_qo_len=(),
                               prefill_kv_len=(), kv_dtype="fp8_e4m3")
    say(f"[fp8-fullsize] {spec.name}: generating on device")
    bd = inputs.make_batch_device(spec, poison=True)
    runner = B.BatchRunner(bd)
    host = inputs.host_subset(bd, [], list(range(spec.num_decode)))
    say("  oracle on every decode")
    ref = oracle.batch_attention(host)
    del host
    for path in ("fused", "seq"):
        say(f"  path {path}")
        compare(run_path(runner, path), ref, f"{spec.name}/{path}")
    del runner, bd
    torch.cuda.empty_cache()
