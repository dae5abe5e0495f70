"""GPU parity of the FP8 E4M3 KV-cache paths (per-KV-head scales) against
the fp64 oracle on the decoded values.

Decode-only batches: MHA and GQA packings of 1 to 32 query heads per KV
head, contiguous and paged caches, lengths around the 32-key step and the
16-key block, forced KV splits, a sharp softmax, NaN in every cache slot no
token owns; every run entry point; and the decodes of the llama2-7b and
70B-shaped layers at full size, every row.

Hybrid batches (the prefill tile's FP8 form beside the FP8 decode unit in
the fused kernel): reduced forms of the layer shapes, edge cases (one key,
a chunk that is its whole request, non-causal, GQA 32, pages of 64, a
prefill-only batch), every scheduler mode and launch shape, forced prefill
and decode splits under a sharp softmax, and sampled rows of three layers
at full size."""

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


# ---- hybrid batches ----

def fp8_hybrid_specs():
    rng = np.random.default_rng(93)
    ln = np.clip(np.rint(300 * np.exp(rng.standard_normal(10))), 1, 2400).astype(int)
    return [
        S("f8h_tiny", 8, 8, [(128, 384)], [512] * 4, seed=611, layout="contiguous",
          extra_pages=0, **F8),
        S("f8h_llama3_8b_r", 32, 8, [(300, 1100)], list(rng.integers(1, 1500, 9, endpoint=True)),
          seed=612, **F8),
        S("f8h_llama2_7b_r", 32, 32, [(200, 900)], [700] * 6, seed=613, **F8),
        S("f8h_l70b_r", 64, 8, [(260, 1300)], list(ln), seed=614, **F8),
        S("f8h_batched_r", 32, 8, [(17, 40), (64, 300), (129, 129), (200, 777)],
          list(rng.integers(1, 2000, 20, endpoint=True)), seed=615, **F8),
        S("f8h_one_key", 4, 4, [(1, 1)], [1], seed=616, layout="contiguous", extra_pages=0, **F8),
        S("f8h_qo_eq_kv", 8, 2, [(190, 190)], [33], seed=617, **F8),
        S("f8h_noncausal", 8, 2, [(100, 333)], [64], seed=618, causal=False, **F8),
        S("f8h_gqa32", 64, 2, [(70, 150)], [300, 5], seed=619, **F8),
        S("f8h_page64", 16, 4, [(150, 700), (3, 64)], [65, 1000], seed=620, page_size=64, **F8),
        S("f8h_only_prefill", 8, 8, [(257, 600)], [], seed=621, **F8),
    ]


@pytest.mark.parametrize("spec", fp8_hybrid_specs(), ids=lambda s: s.name)
def test_fp8_hybrid_against_oracle(spec):
    say(f"[fp8-hybrid] {spec.name}")
    b = inputs.make_batch_host(spec, poison=True)
    ref = oracle.batch_attention(b)
    runner = B.BatchRunner(b)
    for path in ("fused", "seq", "streams"):
        say(f"  path {path}")
        compare(run_path(runner, path), ref, f"{spec.name}/{path}")


@pytest.mark.parametrize("mode", ["colocate", "split", "ordered", "one-unit split",
                                  "one-unit colocate", "matched"])
def test_fp8_hybrid_sched_modes(mode):
    spec = fp8_hybrid_specs()[4]
    say(f"[fp8-hybrid] {spec.name}, {mode}")
    tun = {"colocate": B.make_tuning(sched_mode=B.SCHED_COLOCATE),
           "split": B.make_tuning(sched_mode=B.SCHED_SPLIT),
           "ordered": B.make_tuning(sched_mode=B.SCHED_ORDERED),
           "one-unit split": B.make_tuning(sched_mode=B.SCHED_SPLIT,
                                           flags=B.FLAG_ONE_UNIT_PER_WG),
           "one-unit colocate": B.make_tuning(sched_mode=B.SCHED_COLOCATE,
                                              flags=B.FLAG_ONE_UNIT_PER_WG),
           "matched": B.make_tuning(match_sequential=1)}[mode]
    b = inputs.make_batch_host(spec, poison=True)
    ref = oracle.batch_attention(b)
    runner = B.BatchRunner(b, tun)
    f = run_path(runner, "fused")
    compare(f, ref, f"{spec.name}/{mode}")
    if mode == "matched":
        # the same lists and the same tile code: bitwise equal to the sequential path
        s_ = run_path(runner, "seq")
        for k in f:
            assert np.array_equal(f[k], s_[k]), k


@pytest.mark.parametrize("splits", [(1, 1), (3, 2), (7, 16)])
@pytest.mark.parametrize("which", [0, 1, 3, 4], ids=["tiny", "llama3_8b_r", "l70b_r", "batched_r"])
def test_fp8_hybrid_forced_splits_sharp(which, splits):
    # sm_scale = 1: the shapes of the bf16 sharp-softmax tests, and the
    # reduced 70B shape, whose unsplit rows exceed the bar with bf16 P (the
    # FP8 tile's PV runs on fp16 P)
    spec = inputs.with_scale(fp8_hybrid_specs()[which], 1.0)
    ps, ds = splits
    say(f"[fp8-hybrid] {spec.name}, prefill splits {ps}, decode splits {ds}")
    b = inputs.make_batch_host(spec, poison=True)
    ref = oracle.batch_attention(b)
    runner = B.BatchRunner(b, B.make_tuning(prefill_kv_splits=ps, decode_kv_splits=ds))
    for path in ("fused", "seq"):
        compare(run_path(runner, path), ref, f"fp8 hybrid sharp {splits}/{path}")


@pytest.mark.parametrize("name", ["llama3_8b", "l70b_tp1", "batched"])
def test_fp8_hybrid_fullsize_sampled(name):
    import dataclasses
    import torch
    base = inputs.config_spec(name)
    spec = dataclasses.replace(base, name=base.name + "_fp8", kv_dtype="fp8_e4m3")
    say(f"[fp8-fullsize] {spec.name}: generating on device")
    bd = inputs.make_batch_device(spec, poison=True)
    runner = B.BatchRunner(bd)
    rng = np.random.default_rng(7)
    sum_qo = int(sum(spec.prefill_qo_len))
    starts = np.concatenate([[0], np.cumsum(spec.prefill_qo_len)])
    rows = set(int(x) for x in rng.choice(sum_qo, size=min(160, sum_qo), replace=False))
    for a_, b_ in zip(starts[:-1], starts[1:]):       # each chunk's first and last rows
        rows.update((int(a_), int(b_) - 1))
    rows = sorted(rows)
    dkv = np.array(spec.decode_kv_len)
    dec = {int(np.argmax(dkv)), int(np.argmin(dkv)), 0, len(dkv) - 1}
    dec.update(int(x) for x in rng.choice(len(dkv), size=min(8, len(dkv)), replace=False))
    dec = sorted(dec)
    sub = inputs.host_subset(bd, list(range(spec.num_prefill)), dec)
    say(f"  oracle on {len(rows)} prefill rows, {len(dec)} decodes")
    ref = oracle.sample_batch_attention(sub, rows, list(range(len(dec))))
    for path in ("fused", "seq"):
        say(f"  path {path}")
        got = run_path(runner, path)
        g = {"o_prefill": got["o_prefill"][rows], "lse_prefill": got["lse_prefill"][rows],
             "o_decode": got["o_decode"][dec], "lse_decode": got["lse_decode"][dec]}
        compare(g, ref, f"{spec.name}/{path}")
        for k in got:
            assert np.all(np.isfinite(got[k])), (spec.name, path, k)
    del runner, bd
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["l70b_tp1"])
def test_fp8_hybrid_fullsize_every_row(name):
    # every prefill row and decode of the full-size FP8 layer, fused and
    # sequential, against the oracle of the whole batch
    import torch
    spec = inputs.fp8_spec(name)
    say(f"[fp8-fullsize-all] {spec.name}: generating on device")
    bd = inputs.make_batch_device(spec, poison=True)
    runner = B.BatchRunner(bd)
    host = inputs.host_subset(bd, list(range(spec.num_prefill)), list(range(spec.num_decode)))
    say("  oracle on the whole batch")
    ref = oracle.batch_attention(host)
    del host
    for path in ("fused", "seq"):
        say(f"  path {path}")
        compare(run_path(runner, path), ref, f"{spec.name}-all/{path}")
    del runner, bd
    torch.cuda.empty_cache()
