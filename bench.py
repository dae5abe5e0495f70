"""Benchmark: fused prefill+decode attention of one hybrid batch on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-flush] [--no-cpu]

A step is one pass of the hot path over the batch: pod_attn_run (the fused
kernel that runs every prefill tile and decode split, with the log-sum-exp
merge of KV-split partials).  Inputs (bf16 Q/K/V, page tables) and the plan
are resident in HBM before the timed region.  Before each timed step a 1 GiB
buffer is written to evict the L2 caches and the 256 MB Infinity Cache, so
every step streams its KV cache from HBM; the write is outside the events.
Each step is timed with HIP events recorded on the stream the kernels run on.
The sequential baseline (prefill kernel, decode kernel, merge; its own plan)
is timed the same way in the same run.  The fp64 CPU oracle is timed on the
host cores as a reported baseline.

Prints one JSON line.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DESCR = {
    "tiny": "tiny: 8q/8kv d128; prefill 128@384 causal + 4 decodes @512; contiguous KV",
    "llama3_8b": "llama3-8b layer: 32q/8kv d128; prefill 1024@4096 causal + 64 decodes "
                 "kv~U[1024,4096]; paged 16, random page order",
    "llama2_7b": "llama2-7b MHA layer: 32q/32kv d128; prefill 512@12288 + 128 decodes @8192; "
                 "paged 16",
    "l70b_tp1": "70b TP=1 layer: 64q/8kv d128; prefill 2048@16384 + 256 decodes kv~lognormal"
                "(median 4096, sigma 1, cap 32768); paged 16",
    "batched": "batched multi-prefill: 32q/8kv d128; 4 chunks {128,256,512,640}@U[2048,8192] "
               "+ 192 decodes U[512,16384]; paged 16",
}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(batch_dev, spec, budget_s=20.0):
    """Times the fp64 oracle (as it stands) on the host cores over the whole
    batch, repeated while within `budget_s`; returns µs per layer."""
    from threadpoolctl import threadpool_limits

    import oracle
    from prefill_decode_amd import inputs

    host = inputs.host_subset(batch_dev, list(range(spec.num_prefill)),
                              list(range(spec.num_decode)))
    workers = len(os.sched_getaffinity(0))
    times = []
    with threadpool_limits(1):
        t_all = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            oracle.batch_attention(host, workers=workers)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_all + times[-1] > budget_s or len(times) >= 5:
                break
    return {"value": float(np.median(times)) * 1e6, "unit": "µs/layer", "cores": workers,
            "kind": "oracle",
            "sample": f"whole batch ({spec.name}), fp64 numpy, {len(times)} run(s), median; "
                      f"BLAS 1 thread per worker; CPU {_cpu_model()}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="llama3_8b")
    ap.add_argument("--n-dec", type=int, default=None, help="batched: decode-count sweep point")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--quarters", type=int, default=-1, help="prefill quarters per CU (-1 auto)")
    ap.add_argument("--sched", type=int, default=0, help="0 live, 1 ticket, 2 ordered")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the attention path needs no collectives; see DESIGN.md for how it shards)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from prefill_decode_amd import binding as B
    from prefill_decode_amd import inputs, metrics

    torch.cuda.set_device(0)
    spec = inputs.config_spec(args.config, n_dec=args.n_dec)
    batch = inputs.make_batch_device(spec)
    counts = metrics.algorithmic_counts(spec)
    tuning = B.make_tuning(prefill_quarters_per_cu=args.quarters, sched_mode=args.sched)
    t0 = time.perf_counter()
    runner = B.BatchRunner(batch, tuning)
    torch.cuda.synchronize()
    plan_ms = (time.perf_counter() - t0) * 1e3
    info = runner.plan.info()
    stream = torch.cuda.current_stream()
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def do_flush(i):
        if not args.no_flush:
            flush.fill_(i & 0xFF)

    for i in range(args.warmup):
        runner.run()
        runner.sequential_run()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        do_flush(2 * i)
        ev[i][0].record(stream)
        runner.run()
        ev[i][1].record(stream)
        do_flush(2 * i + 1)
        ev[i][2].record(stream)
        runner.sequential_run()
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    fused_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    seq_ms = np.array([e[2].elapsed_time(e[3]) for e in ev])
    # warm (no flush) back-to-back
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for _ in range(args.steps):
        runner.run()
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / args.steps

    t_fused = float(np.median(fused_ms)) * 1e-3
    t_seq = float(np.median(seq_ms)) * 1e-3
    roof_s = metrics.overlap_roofline_s(counts)
    hbm_bound = counts["bytes"] / metrics.PEAK_HBM_BYTES >= counts["flops"] / metrics.PEAK_BF16_FLOPS
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": counts["bytes"] / t_fused / 1e9,
                "peak": metrics.PEAK_HBM_BYTES / 1e9, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": counts["flops"] / t_fused / 1e12,
                "peak": metrics.PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = "pod_fused_kernel (+ pod_merge_kernel when the plan splits)"

    out = {
        "metric": "fused prefill+decode attn µs/layer; % of overlap roofline; speedup vs sequential",
        "value": t_fused * 1e6,
        "unit": "µs/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_fused * 1e3,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": DESCR.get(args.config, spec.name), "name": spec.name,
                   "num_prefill": spec.num_prefill, "num_decode": spec.num_decode,
                   "cache_flush": not args.no_flush},
        "overlap_roofline_us": roof_s * 1e6,
        "overlap_roofline_frac": roof_s / t_fused,
        "sequential_us": t_seq * 1e6,
        "speedup_vs_sequential": t_seq / t_fused,
        "fused_us_p10_p90": [float(np.percentile(fused_ms, 10)) * 1e3,
                             float(np.percentile(fused_ms, 90)) * 1e3],
        "warm_cache_fused_us": warm_ms * 1e3,
        "achieved_tflops": counts["flops"] / t_fused / 1e12,
        "achieved_hbm_gbs": counts["bytes"] / t_fused / 1e9,
        "algorithmic": {"gflop": counts["flops"] / 1e9, "gbytes": counts["bytes"] / 1e9},
        "plan": {"host_ms": plan_ms, "prefill_items": info["prefill_items"],
                 "decode_items": info["decode_items"], "merge_tasks": info["merge_tasks"],
                 "prefill_quarters_per_cu": info["prefill_quarters_per_cu"],
                 "sched_mode": info["sched_mode"]},
        "wall_s_timed_loop": wall,
        "roofline": roof,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(batch, spec)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
