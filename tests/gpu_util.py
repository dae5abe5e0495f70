"""Shared helpers of the GPU tests: run a batch through the C ABI and compare
with the fp64 oracle at the stated tolerance."""

import sys

import numpy as np

O_ABS, O_REL, LSE_ABS = 5e-3, 1e-2, 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def compare(got, ref, what=""):
    """Elementwise |O - ref| <= 5e-3 + 1e-2 |ref| and |LSE - ref| <= 1e-3."""
    for part in ("prefill", "decode"):
        o, r = got["o_" + part], ref["o_" + part]
        if r.size == 0:
            continue
        assert np.all(np.isfinite(o)), f"{what} {part}: non-finite output"
        err = np.abs(o - r)
        bound = O_ABS + O_REL * np.abs(r)
        bad = err > bound
        assert not bad.any(), (f"{what} {part}: {int(bad.sum())} O elements out of tolerance, "
                               f"max err {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}")
        le = np.abs(got["lse_" + part] - ref["lse_" + part])
        assert np.all(le <= LSE_ABS), f"{what} {part}: LSE max err {le.max():.3e}"


def run_path(runner, path):
    import torch
    runner.o_prefill.fill_(float("nan"))
    runner.o_decode.fill_(float("nan"))
    runner.lse_prefill.fill_(float("nan"))
    runner.lse_decode.fill_(float("nan"))
    if path == "fused":
        runner.run()
    elif path == "seq":
        runner.sequential_run()
    elif path == "streams":
        runner.streams_run(torch.cuda.Stream())
    elif path == "batched":
        runner.batched_prefill_run()
    else:
        raise ValueError(path)
    torch.cuda.synchronize()
    return runner.outputs()


def bits(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy()
