"""GPU parity on seeded random hybrid batches: head layouts (query heads per
KV head 1-32), 0-3 prefill chunks and 0-9 decodes of random lengths, causal
or not, paged (page sizes 1-128) or contiguous, bf16 or FP8 E4M3 caches,
under random tunings (forced KV splits, prefill share, scheduler mode, launch
shape).  Every case runs the fused and the sequential path against the fp64
oracle at the parity bar."""

import numpy as np
import pytest

import oracle
from prefill_decode_amd import binding as B
from prefill_decode_amd import inputs
from tests.gpu_util import compare, run_path, say

pytestmark = pytest.mark.gpu

N_CASES = 24


def _case(i):
    rng = np.random.default_rng([20261204, i])
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 6, 8, 16, 32]))
    fp8 = bool(rng.integers(0, 3) == 0)
    contiguous = not fp8 and bool(rng.integers(0, 5) == 0)
    page = int(rng.choice([16, 32, 128] if fp8 else [1, 8, 16, 32, 128]))
    np_, nd = int(rng.integers(0, 4)), int(rng.integers(0, 10))
    if np_ + nd == 0:
        nd = 1
    pre = []
    for _ in range(np_):
        qo = int(rng.integers(1, 400))
        pre.append((qo, qo + int(rng.integers(0, 900))))
    dec = [int(x) for x in rng.integers(1, 2500, size=nd)]
    kw = dict(causal=bool(rng.integers(0, 4)), kv_dtype="fp8_e4m3" if fp8 else "bf16")
    if contiguous:
        kw.update(layout="contiguous", extra_pages=0)
    else:
        kw.update(page_size=page)
    spec = inputs.custom_spec(f"rand{i}", g * hkv, hkv, pre, dec, seed=7000 + i, **kw)
    tun = {}
    if rng.integers(0, 2):
        tun["prefill_kv_splits"] = int(rng.choice([0, 1, 2, 3, 5, 16]))
        tun["decode_kv_splits"] = int(rng.choice([0, 1, 2, 3, 7, 64]))
    if rng.integers(0, 3) == 0:
        tun["sched_mode"] = int(rng.integers(0, 4))
        tun["prefill_quarters_per_cu"] = int(rng.integers(-1, 9))
    if rng.integers(0, 4) == 0:
        tun["flags"] = B.FLAG_ONE_UNIT_PER_WG
    return spec, tun


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_batch_against_oracle(i):
    spec, tun = _case(i)
    say(f"[random] {spec.name}: hq {spec.num_qo_heads} hkv {spec.num_kv_heads} "
        f"{spec.layout}/{spec.page_size} {spec.kv_dtype} causal {spec.causal} "
        f"prefill {list(zip(spec.prefill_qo_len, spec.prefill_kv_len))} "
        f"decode {list(spec.decode_kv_len)} tuning {tun}")
    b = inputs.make_batch_host(spec, poison=True)
    ref = oracle.batch_attention(b)
    runner = B.BatchRunner(b, B.make_tuning(**tun) if tun else None)
    for path in ("fused", "seq"):
        compare(run_path(runner, path), ref, f"{spec.name}/{path}")
