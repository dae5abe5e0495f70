"""GPU parity at the full workload sizes (the launch configuration the bench
times): every config on sampled rows the oracle computes one by one and on
every row against the fp64 oracle of the whole batch, plus the scheduler
traces on the Llama-3-8B-shaped batch."""

import numpy as np
import pytest

import oracle
from prefill_decode_amd import binding as B
from prefill_decode_amd import inputs
from tests.gpu_util import compare, run_path, say

pytestmark = pytest.mark.gpu


def _sample(spec, rng):
    qo = np.array(spec.prefill_qo_len)
    offs = np.concatenate([[0], np.cumsum(qo)])
    rows = set()
    for r in range(len(qo)):
        a, b = int(offs[r]), int(offs[r + 1])
        rows.update([a, min(a + 1, b - 1), b - 1, max(a, b - 2)])
        rows.update(int(x) for x in rng.integers(a, b, size=min(8, b - a)))
    dkv = np.array(spec.decode_kv_len)
    dec = {int(np.argmax(dkv)), int(np.argmin(dkv)), 0, len(dkv) - 1}
    dec.update(int(x) for x in rng.choice(len(dkv), size=min(8, len(dkv)), replace=False))
    return sorted(rows), sorted(dec)


@pytest.mark.parametrize("name", inputs.CONFIG_NAMES)
def test_fullsize_sampled(name):
    import torch
    spec = inputs.config_spec(name)
    say(f"[fullsize] {name}: generating on device")
    bd = inputs.make_batch_device(spec, poison=True)
    runner = B.BatchRunner(bd)
    rows, dec = _sample(spec, np.random.default_rng(5))
    sub = inputs.host_subset(bd, list(range(spec.num_prefill)), dec)
    say(f"  oracle on {len(rows)} prefill rows, {len(dec)} decodes")
    ref = oracle.sample_batch_attention(sub, rows, list(range(len(dec))))
    for path in ("fused", "seq"):
        say(f"  path {path}")
        got = run_path(runner, path)
        g = {"o_prefill": got["o_prefill"][rows], "lse_prefill": got["lse_prefill"][rows],
             "o_decode": got["o_decode"][dec], "lse_decode": got["lse_decode"][dec]}
        compare(g, ref, f"{name}/{path}")
        # every output row written and finite (full check of the non-sampled rows)
        for k in got:
            assert np.all(np.isfinite(got[k])), (name, path, k)
    del runner, bd
    torch.cuda.empty_cache()


def _every_row(spec, paths, tunings=()):
    import torch
    say(f"[fullsize-all] {spec.name}: generating on device")
    bd = inputs.make_batch_device(spec, poison=True)
    runner = B.BatchRunner(bd, B.make_tuning(flags=B.FLAG_BATCHED_PREFILL))
    host = inputs.host_subset(bd, list(range(spec.num_prefill)), list(range(spec.num_decode)))
    say("  oracle on the whole batch")
    ref = oracle.batch_attention(host)
    del host
    for path in paths:
        say(f"  path {path}")
        compare(run_path(runner, path), ref, f"{spec.name}-all/{path}")
    del runner
    for label, tun in tunings:
        say(f"  fused, {label}")
        r2 = B.BatchRunner(bd, tun)
        compare(run_path(r2, "fused"), ref, f"{spec.name}-all/{label}")
        del r2
    del bd, ref
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", inputs.CONFIG_NAMES)
def test_fullsize_every_row(name):
    # every prefill row and decode of the full-size batch, on the fused and
    # sequential paths and the two comparators, against the fp64 oracle of
    # the whole batch; the llama3-8b layer also under the co-location and
    # ordered scheduler modes
    tunings = ()
    if name == "llama3_8b":
        tunings = (("colocate", B.make_tuning(sched_mode=B.SCHED_COLOCATE)),
                   ("ordered", B.make_tuning(sched_mode=B.SCHED_ORDERED)),
                   ("one-unit split", B.make_tuning(sched_mode=B.SCHED_SPLIT,
                                                    flags=B.FLAG_ONE_UNIT_PER_WG)),
                   ("one-unit colocate", B.make_tuning(sched_mode=B.SCHED_COLOCATE,
                                                       flags=B.FLAG_ONE_UNIT_PER_WG)))
    _every_row(inputs.config_spec(name), ("fused", "seq", "streams", "batched"), tunings)


@pytest.mark.parametrize("n_dec", [32, 64, 128, 256])
def test_fullsize_batched_sweep_every_row(n_dec):
    # the batched mix's decode-count sweep, every row, both paths
    _every_row(inputs.config_spec("batched", n_dec=n_dec), ("fused", "seq"))


def _trace(spec, bd, mode, ref=None):
    runner = B.BatchRunner(bd, B.make_tuning(flags=B.FLAG_TRACE, sched_mode=mode))
    got = run_path(runner, "fused")
    if ref is not None:
        compare(got, ref, f"trace mode {mode}")
    info = runner.plan.info()
    tr = runner.plan.read_trace()
    n_p, n_d = info["prefill_items"], info["decode_items"]
    assert len(tr) == n_p + n_d
    role, unit = tr[:, 2], tr[:, 3]
    # every unit ran exactly once, in the record of its index
    assert np.array_equal(role, np.r_[np.zeros(n_p), np.ones(n_d)].astype(role.dtype))
    assert np.array_equal(unit, np.r_[np.arange(n_p), np.arange(n_d)].astype(unit.dtype))
    assert np.all(tr[:, 5] >= tr[:, 4])
    return info, tr


def test_scheduler_traces():
    spec = inputs.config_spec("llama3_8b")
    say("[trace] llama3_8b")
    bd = inputs.make_batch_device(spec)
    host = inputs.host_subset(bd, list(range(spec.num_prefill)), list(range(spec.num_decode)))
    ref = oracle.batch_attention(host)
    del host
    # co-location on every CU: most CUs run a prefill and a decode unit at once
    info, tr = _trace(spec, bd, B.SCHED_COLOCATE, ref)
    role, slot = tr[:, 2], tr[:, 1]
    both = 0
    slots = np.unique(slot)
    for s in slots:
        m = slot == s
        p, d = tr[m & (role == 0)], tr[m & (role == 1)]
        if len(p) and len(d):
            ov = (np.minimum(p[:, 5][:, None], d[:, 5][None, :]) >
                  np.maximum(p[:, 4][:, None], d[:, 4][None, :]))
            both += int(ov.any())
    say(f"  co-locate: CUs used {len(slots)}, running prefill and decode at once {both}")
    assert len(slots) == 256
    assert both >= 0.5 * len(slots)
    # the automatic choice for this layer: one workgroup per unit with
    # per-CU tickets (every unit once, outputs checked)
    info, tr = _trace(spec, bd, B.SCHED_AUTO, ref)
    assert info["sched_mode"] == B.SCHED_COLOCATE and info["one_unit_per_wg"] == 1
    # CU partition: about q/8 of the CUs start on prefill, and the prefill and
    # decode units overlap in time across the GPU
    info, tr = _trace(spec, bd, B.SCHED_SPLIT, ref)
    assert info["sched_mode"] == B.SCHED_SPLIT
    q = info["prefill_quarters_per_cu"]
    role, slot, t0, t1 = tr[:, 2], tr[:, 1], tr[:, 4], tr[:, 5]
    first = {}
    for i in np.argsort(t0, kind="stable"):
        first.setdefault(int(slot[i]), int(role[i]))
    frac = np.mean([r == 0 for r in first.values()])
    say(f"  split: q {q}, CUs starting on prefill {frac:.3f}")
    assert len(first) == 256 and abs(frac - q / 8) <= 0.1
    p_end, d_start = t1[role == 0].max(), t0[role == 1].min()
    d_end, p_start = t1[role == 1].max(), t0[role == 0].min()
    assert d_start < p_end and p_start < d_end          # the two parts overlap
