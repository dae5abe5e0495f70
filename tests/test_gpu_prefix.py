"""GPU parity of the shared-prefix (packed) decode path against the fp64
oracle ([PAT] abstract: queries packed by shared prefix, KV splits, a final
online-softmax merge).

Cases: group sizes 1 to 20, 1 to 32 query heads per KV head (workgroup
tiles of 64, 16, 8, 4 and 2 members, the ragged pack of g = 6 and the
partial head block of g = 24), prefixes
that are the whole sequence, ungrouped requests beside groups, pages of 8,
16 and 64 tokens, forced KV splits, a sharp softmax, NaN in every cache slot
no token owns.  The packed path (pod_attn_run) and the unshared baseline of
the same plan (pod_attn_sequential_run) both match the oracle."""

import numpy as np
import pytest

import oracle
from prefill_decode_amd import binding as B
from prefill_decode_amd import inputs
from tests.gpu_util import compare, run_path, say

pytestmark = pytest.mark.gpu


def _spec(name, hq, hkv, dkv, groups, seed, **kw):
    return inputs.custom_spec(name, hq, hkv, [], dkv, seed=seed,
                              prefix_groups=tuple((tuple(m), p) for m, p in groups), **kw)


def prefix_specs():
    rng = np.random.default_rng(77)
    own = lambda n, lo, hi: [int(x) for x in rng.integers(lo, hi, n, endpoint=True)]
    return [
        _spec("p_g8_groups", 32, 4, [512 + x for x in own(11, 1, 700)],
              [((0, 1, 2), 512), (tuple(range(3, 11)), 256)], seed=701),
        _spec("p_g4_17", 16, 4, [96 + x for x in own(17, 0, 300)], [(tuple(range(17)), 96)],
              seed=702),
        _spec("p_mha", 8, 8, [64 + x for x in own(6, 0, 100)] + [33],
              [((0, 1, 2, 3, 4, 5), 64)], seed=703),
        _spec("p_g16", 32, 2, [1024 + x for x in own(4, 0, 64)] + [5, 700],
              [((0, 1, 2, 3), 1024)], seed=704),
        _spec("p_g32", 64, 2, [300, 320, 288], [((0, 1, 2), 288)], seed=705),
        _spec("p_g6_ragged", 12, 2, [128, 129, 130, 131, 200], [((0, 1, 2, 3, 4), 128)],
              seed=706),
        _spec("p_whole", 16, 2, [256, 256, 256], [((0, 1, 2), 256)], seed=707),
        _spec("p_single", 16, 2, [48, 400], [((0,), 48), ((1,), 384)], seed=708),
        _spec("p_page8", 16, 4, [40 + x for x in own(5, 0, 90)], [((0, 1, 2, 3, 4), 40)],
              seed=709, page_size=8),
        _spec("p_g24", 48, 2, [96 + x for x in own(6, 0, 200)], [(tuple(range(6)), 96)],
              seed=711),
        _spec("p_g8_40", 32, 4, [160 + x for x in own(40, 0, 400)],
              [(tuple(range(0, 40, 2)), 160), (tuple(range(1, 40, 2)), 128)], seed=712),
        _spec("p_page64", 32, 8, [640 + x for x in own(6, 1, 500)], [((0, 2, 4), 640),
                                                                      ((1, 3), 576)],
              seed=710, page_size=64),
    ]


@pytest.mark.parametrize("spec", prefix_specs(), ids=lambda s: s.name)
def test_prefix_decode_against_oracle(spec):
    say(f"[prefix] {spec.name}")
    b = inputs.make_batch_host(spec, poison=True)
    ref = oracle.batch_attention(b)
    runner = B.BatchRunner(b)
    for path in ("fused", "seq", "streams"):
        compare(run_path(runner, path), ref, f"{spec.name}/{path}")


@pytest.mark.parametrize("splits", [1, 2, 7])
def test_prefix_forced_splits_sharp(splits):
    spec = inputs.with_scale(prefix_specs()[0], 1.0)
    say(f"[prefix] sharp, splits {splits}")
    b = inputs.make_batch_host(spec, poison=True)
    ref = oracle.batch_attention(b)
    runner = B.BatchRunner(b, B.make_tuning(decode_kv_splits=splits))
    compare(run_path(runner, "fused"), ref, f"prefix sharp splits {splits}")


def test_prefix_plan_rejections():
    p = B.make_params(16, 2)
    with pytest.raises(B.PodError) as e:              # FP8 cache
        B.plan_shared_prefix(B.make_params(16, 2, kv_dtype="fp8_e4m3"), [64, 64], [0, 0], [64])
    assert e.value.status == 2
    with pytest.raises(B.PodError) as e:              # prefix longer than a member
        B.plan_shared_prefix(p, [64, 32], [0, 0], [48])
    assert e.value.status == 1


def test_prefix_fullsize_sampled_rows():
    """The 70B-shaped shared-prefix batch that the benchmark times, every
    row."""
    from tests.gpu_util import compare as cmp
    spec = inputs.config_spec("l70b_prefix")
    say(f"[prefix] {spec.name}")
    b = inputs.make_batch_host(spec, poison=False)
    ref = oracle.batch_attention(b)
    runner = B.BatchRunner(b)
    cmp(run_path(runner, "fused"), ref, spec.name)
