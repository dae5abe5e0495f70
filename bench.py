"""Benchmark: fused prefill+decode attention of one hybrid batch on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-flush] [--no-cpu]
    python bench.py --pmc-run [--config NAME]          (driver for rocprofv3 counter runs)
    python bench.py --summarize-pmc DIR [--config NAME] (writes profiles/traffic_*.md)
    python bench.py --summarize-stats DIR [--config NAME] (writes profiles/*_stats.md)

A step is one pass of the hot path over the batch: pod_attn_run, i.e. the fused
kernel (every prefill tile and decode split of the batch) and the log-sum-exp
merge of KV-split partials.  Inputs (bf16 Q/K/V, page tables) and the plan are
resident in HBM before the timed region.  Before each timed step a 1 GiB buffer
is written to evict the L2 caches and the 256 MB Infinity Cache, so every step
streams its KV cache from HBM; the write is outside the events.  HIP events
are recorded on the stream the kernels run on: around the whole step, and
(through pod_attn_run_events) immediately around the fused kernel, whose time
the roofline object uses.  The sequential baseline (prefill kernel, decode
kernel, merge; its own plan) is timed the same way in the same run.  The fp64
CPU oracle is timed on the host cores on a bounded sample of the batch.

Prints one JSON line.
"""

import argparse
import glob
import hashlib
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
COPY_BYTES = 1 << 30          # calibration copy for the HBM byte counters
PROFILES = os.path.join(ROOT, "profiles")


def sources_digest():
    """sha256 over the library's kernel and planner sources and its build
    script (compile flags change the kernels too): traffic figures taken from
    counters are only reported while this matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "prefill_decode_amd", "csrc")
    files = [f for f in sorted(glob.glob(os.path.join(csrc, "*"))) if f.endswith((".hip", ".cpp", ".h"))]
    for f in files + [os.path.join(ROOT, "prefill_decode_amd", "build.py")]:
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_file(config):
    return os.path.join(PROFILES, f"traffic_pod_fused_kernel_{config}.md")


def read_traffic(config):
    """HBM bytes per fused launch from the committed counter summary, or None
    when there is none or the kernel sources changed since it was taken."""
    try:
        lines = open(traffic_file(config)).read().splitlines()
    except OSError:
        return None
    kv = {}
    for ln in lines:
        if ":" in ln and ln.startswith("- "):
            k, v = ln[2:].split(":", 1)
            kv[k.strip()] = v.strip().strip("`")
    if kv.get("sources_sha256") != sources_digest():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _row_pairs(spec):
    """Visible keys of every prefill row (global order) and of every decode."""
    rows = []
    for qo, kv in zip(spec.prefill_qo_len, spec.prefill_kv_len):
        pos = np.arange(kv - qo, kv)
        rows.append(pos + 1 if spec.causal else np.full(qo, kv))
    rows = np.concatenate(rows) if rows else np.zeros(0)
    return rows.astype(np.float64), np.asarray(spec.decode_kv_len, dtype=np.float64)


def cpu_baseline(batch_dev, spec, budget_s=15.0):
    """Times the fp64 oracle (as it stands) on the host cores.  A pilot sample
    sizes a bounded sample of evenly spaced prefill rows and decodes (about
    `budget_s` of work, or the whole batch when smaller); the time is scaled to
    the whole batch by the ratio of visible (query, key) pairs."""
    from threadpoolctl import threadpool_limits

    import oracle
    from prefill_decode_amd import inputs

    workers = len(os.sched_getaffinity(0))
    rp, dp = _row_pairs(spec)
    total = rp.sum() + dp.sum()
    n_rows, n_dec = len(rp), len(dp)
    host = inputs.host_subset(batch_dev, list(range(spec.num_prefill)), list(range(n_dec)))

    def pick(frac):
        r = np.unique(np.linspace(0, n_rows - 1, max(1, int(round(frac * n_rows)))).astype(int)) \
            if n_rows else np.zeros(0, int)
        d = np.unique(np.linspace(0, n_dec - 1, max(1, int(round(frac * n_dec)))).astype(int)) \
            if n_dec else np.zeros(0, int)
        return r, d

    def timed(frac):
        r, d = pick(frac)
        with threadpool_limits(1):
            t0 = time.perf_counter()
            oracle.sample_batch_attention(host, r.tolist(), d.tolist(), workers=workers)
            dt = time.perf_counter() - t0
        pairs = (rp[r].sum() if len(r) else 0.0) + (dp[d].sum() if len(d) else 0.0)
        return dt, pairs, len(r), len(d)

    frac = min(1.0, 2.0e7 / max(total, 1.0))          # pilot: about 2e7 pairs
    dt, pairs, _, _ = timed(frac)
    rate = pairs / max(dt, 1e-6)
    frac = min(1.0, budget_s * rate / total)
    dt, pairs, nr, nd = timed(frac)
    est = dt * total / max(pairs, 1.0)
    return {"value": est * 1e6, "unit": "µs/layer", "cores": workers, "kind": "oracle",
            "sample": f"{nr} of {n_rows} prefill rows and {nd} of {n_dec} decodes, evenly "
                      f"spaced ({pairs / total:.3g} of the visible query-key pairs), fp64 numpy, "
                      f"{dt:.1f} s, scaled by pairs; BLAS 1 thread per worker; CPU {_cpu_model()}"}


def pmc_run(args):
    """Driver for `rocprofv3 --pmc` runs: a few fused runs, as many sequential
    runs, and one plain 1 GiB device-to-device copy whose counters calibrate
    the byte counters."""
    import torch

    from prefill_decode_amd import binding as B
    from prefill_decode_amd import inputs

    torch.cuda.set_device(0)
    spec = inputs.config_spec(args.config, n_dec=args.n_dec)
    runner = B.BatchRunner(inputs.make_batch_device(spec))
    for _ in range(args.steps):
        runner.run()
    for _ in range(args.steps):
        runner.sequential_run()
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"pmc-run {args.config}: {args.steps} fused and {args.steps} sequential runs, "
          f"one {COPY_BYTES} B copy", flush=True)


def summarize_pmc(args):
    """Reads the FETCH_SIZE / WRITE_SIZE passes under DIR (DIR/fetch, DIR/write)
    and writes profiles/traffic_pod_fused_kernel_<config>.md."""
    import csv

    def load(sub, counter):
        vals, copy = [], []
        for f in glob.glob(os.path.join(args.summarize_pmc, sub, "**", "*counter_collection.csv"),
                           recursive=True):
            for row in csv.DictReader(open(f)):
                if row.get("Counter_Name") != counter:
                    continue
                name, v = row["Kernel_Name"], float(row["Counter_Value"])
                if "pod_fused_kernel" in name:
                    vals.append(v)
                elif "copy" in name.lower():
                    copy.append(v)
        return vals, copy

    fv, fc = load("fetch", "FETCH_SIZE")
    wv, wc = load("write", "WRITE_SIZE")
    if not (fv and wv and fc and wc):
        sys.exit("summarize-pmc: missing fused or copy dispatches in the counter CSVs")
    f_copy, w_copy = max(fc), max(wc)                      # the 1 GiB copy
    kf, kw = COPY_BYTES / f_copy, COPY_BYTES / w_copy       # bytes per counter unit
    f_b, w_b = float(np.mean(fv)) * kf, float(np.mean(wv)) * kw
    from prefill_decode_amd import inputs, metrics
    spec = inputs.config_spec(args.config, n_dec=args.n_dec)
    alg = metrics.algorithmic_counts(spec)["bytes"]
    d = os.path.abspath(args.summarize_pmc)
    txt = f"""# HBM traffic of pod_fused_kernel — {DESCR.get(args.config, args.config)}

Two `rocprofv3 --pmc` passes (one counter each) over `bench.py --pmc-run`:
{args.steps} fused runs of the batch (then as many sequential runs, not used here) and one plain
{COPY_BYTES}-byte device-to-device copy. The copy's
counters calibrate them: bytes per counter unit = {COPY_BYTES} / (the copy's reading).

Commands (from the repository root; `$D` = a scratch directory):

    cd /tmp && export TMPDIR=/tmp
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d $D/fetch -o run -- python3 bench.py --pmc-run --config {args.config} --steps {args.steps}
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d $D/write -o run -- python3 bench.py --pmc-run --config {args.config} --steps {args.steps}
    python3 bench.py --summarize-pmc $D --config {args.config} --steps {args.steps}

| quantity | value |
|---|---|
| copy FETCH_SIZE (counter units) | {f_copy:.6g} |
| copy WRITE_SIZE (counter units) | {w_copy:.6g} |
| bytes per FETCH_SIZE unit | {kf:.6g} |
| bytes per WRITE_SIZE unit | {kw:.6g} |
| fused FETCH_SIZE per dispatch, mean of {len(fv)} | {np.mean(fv):.6g} |
| fused WRITE_SIZE per dispatch, mean of {len(wv)} | {np.mean(wv):.6g} |
| HBM read bytes per fused launch | {f_b:.6g} |
| HBM write bytes per fused launch | {w_b:.6g} |
| algorithmic bytes of the batch | {alg:.6g} |
| traffic / algorithmic | {(f_b + w_b) / alg:.4f} |

- traffic_bytes_per_launch: `{f_b + w_b:.6g}`
- sources_sha256: `{sources_digest()}`
"""
    os.makedirs(PROFILES, exist_ok=True)
    open(traffic_file(args.config), "w").write(txt)
    print(txt)
    del d


COUNTERS = ["MfmaUtil", "LdsBankConflict", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"]


def summarize_counters(args):
    """Reads one `rocprofv3 --pmc` pass of COUNTERS over `--pmc-run` under DIR
    and writes profiles/counters_<config>.md: MFMA busy share of SIMD cycles
    and LDS bank conflicts per kernel (means over dispatches)."""
    import csv
    from collections import defaultdict

    vals = defaultdict(lambda: defaultdict(list))
    for f in glob.glob(os.path.join(args.summarize_counters, "**", "*counter_collection.csv"),
                       recursive=True):
        for row in csv.DictReader(open(f)):
            name = row["Kernel_Name"]
            for k in ("pod_fused_kernel", "pod_prefill_kernel", "pod_decode_kernel",
                      "pod_merge_kernel"):
                if k in name:
                    vals[k][row["Counter_Name"]].append(float(row["Counter_Value"]))
    if "pod_fused_kernel" not in vals:
        sys.exit("summarize-counters: no fused-kernel dispatches in the counter CSVs")
    lines = []
    for k in ("pod_fused_kernel", "pod_prefill_kernel", "pod_decode_kernel", "pod_merge_kernel"):
        if k not in vals:
            continue
        v = vals[k]
        mean = lambda c: float(np.mean(v[c])) if v.get(c) else float("nan")
        lines.append(f"| `{k}` | {len(v.get('MfmaUtil', []))} | {mean('MfmaUtil'):.1f} | "
                     f"{mean('LdsBankConflict'):.4f} | {mean('SQ_LDS_BANK_CONFLICT'):.4g} | "
                     f"{mean('SQ_LDS_IDX_ACTIVE'):.4g} |")
    cnt = " ".join(COUNTERS)
    txt = f"""# MFMA busy and LDS bank conflicts — {DESCR.get(args.config, args.config)}

One `rocprofv3 --pmc` pass over `bench.py --pmc-run` ({args.steps} fused runs, then {args.steps}
sequential runs). `MfmaUtil` = MFMA-busy cycles summed over SIMDs / (GPU-active cycles × SIMDs), in
percent, for the whole launch (idle SIMDs, launch ramp and tail included). `LdsBankConflict` =
bank-conflict cycles / conflict-free LDS cycles.

Commands (from the repository root; `$D` = a scratch directory):

    cd /tmp && export TMPDIR=/tmp
    rocprofv3 --pmc {cnt} --output-format csv -d $D -o run -- python3 bench.py --pmc-run --config {args.config} --steps {args.steps}
    python3 bench.py --summarize-counters $D --config {args.config} --steps {args.steps}

| kernel | dispatches | MfmaUtil % | LdsBankConflict | SQ_LDS_BANK_CONFLICT | SQ_LDS_IDX_ACTIVE |
|---|---|---|---|---|---|
""" + "\n".join(lines) + f"""

- sources_sha256: `{sources_digest()}`
"""
    os.makedirs(PROFILES, exist_ok=True)
    open(os.path.join(PROFILES, f"counters_{args.config}.md"), "w").write(txt)
    print(txt)


def summarize_stats(args):
    """Reads a `rocprofv3 --kernel-trace --stats --output-format csv` run under
    DIR and writes profiles/pod_fused_kernel_<config>_stats.md."""
    import csv

    files = glob.glob(os.path.join(args.summarize_stats, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        sys.exit("summarize-stats: no kernel_stats.csv under " + args.summarize_stats)
    rows = list(csv.DictReader(open(files[0])))
    lines = []
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].split("(")[0].replace("void ", "")
        if len(name) > 70:
            name = name[:67] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f} |")
    txt = f"""# Kernel times — {DESCR.get(args.config, args.config)}

`rocprofv3 --kernel-trace --stats` over one `bench.py` run ({args.steps} timed steps after {args.warmup} warm-up
steps; each step runs `pod_attn_run` and `pod_attn_sequential_run`, each after a 1 GiB cache-evicting fill).

Commands (from the repository root; `$D` = a scratch directory):

    cd /tmp && export TMPDIR=/tmp
    rocprofv3 --kernel-trace --stats --output-format csv -d $D -o run -- python3 bench.py --config {args.config} --steps {args.steps} --warmup {args.warmup} --no-cpu
    python3 bench.py --summarize-stats $D --config {args.config} --steps {args.steps} --warmup {args.warmup}

| kernel | calls | avg µs | min µs | max µs | % of GPU time |
|---|---|---|---|---|---|
""" + "\n".join(lines) + f"""

- sources_sha256: `{sources_digest()}`
"""
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"pod_fused_kernel_{args.config}_stats.md")
    open(out, "w").write(txt)
    print(txt)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="llama3_8b")
    ap.add_argument("--n-dec", type=int, default=None, help="batched: decode-count sweep point")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--quarters", type=int, default=-1, help="prefill quarters per CU (-1 auto)")
    ap.add_argument("--prefill-splits", type=int, default=0, help="force prefill KV splits (0 auto)")
    ap.add_argument("--decode-splits", type=int, default=0, help="force decode KV splits (0 auto)")
    ap.add_argument("--sched", type=int, default=0,
                    help="0 auto, 1 co-locate on every CU, 2 ordered, 3 CU partition")
    ap.add_argument("--pmc-run", action="store_true")
    ap.add_argument("--summarize-pmc", default=None, metavar="DIR")
    ap.add_argument("--summarize-stats", default=None, metavar="DIR")
    ap.add_argument("--summarize-counters", default=None, metavar="DIR")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(sharded by KV head or by request, each GPU would run this same kernel on its "
              "share with no exchange; this library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.summarize_pmc:
        return summarize_pmc(args)
    if args.summarize_stats:
        return summarize_stats(args)
    if args.summarize_counters:
        return summarize_counters(args)
    if args.pmc_run:
        return pmc_run(args)

    import torch

    from prefill_decode_amd import binding as B
    from prefill_decode_amd import inputs, metrics

    torch.cuda.set_device(0)
    spec = inputs.config_spec(args.config, n_dec=args.n_dec)
    batch = inputs.make_batch_device(spec)
    counts = metrics.algorithmic_counts(spec)
    tuning = B.make_tuning(prefill_quarters_per_cu=args.quarters, sched_mode=args.sched,
                           prefill_kv_splits=args.prefill_splits, decode_kv_splits=args.decode_splits)
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

    def new_ev():
        return torch.cuda.Event(enable_timing=True)

    for i in range(args.warmup):
        runner.run()
        runner.sequential_run()
    torch.cuda.synchronize()

    # timed steps: pod_attn_run and pod_attn_sequential_run, each after a
    # cache-evicting fill, with events only around the whole step
    ev = [[new_ev() for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        e = ev[i]
        do_flush(2 * i)
        e[0].record(stream)
        runner.run()
        e[1].record(stream)
        do_flush(2 * i + 1)
        e[2].record(stream)
        runner.sequential_run()
        e[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    seq_ms = np.array([e[2].elapsed_time(e[3]) for e in ev])
    # the fused kernel alone (events recorded around its launch)
    kv = [[new_ev() for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        do_flush(i)
        runner.run_events(kv[i][0], kv[i][1])
    torch.cuda.synchronize()
    fused_ms = np.array([e[0].elapsed_time(e[1]) for e in kv])
    # warm (no flush) back-to-back
    w0, w1 = new_ev(), new_ev()
    w0.record(stream)
    for _ in range(args.steps):
        runner.run()
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / args.steps

    t_step = float(np.median(step_ms)) * 1e-3
    t_kern = float(np.median(fused_ms)) * 1e-3
    t_seq = float(np.median(seq_ms)) * 1e-3
    roof_s = metrics.overlap_roofline_s(counts)
    hbm_bound = counts["bytes"] / metrics.PEAK_HBM_BYTES >= counts["flops"] / metrics.PEAK_BF16_FLOPS
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": counts["bytes"] / t_kern / 1e9,
                "peak": metrics.PEAK_HBM_BYTES / 1e9, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": counts["flops"] / t_kern / 1e12,
                "peak": metrics.PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = read_traffic(args.config) if args.n_dec is None else None
    roof["kernel"] = "pod_fused_kernel"
    roof["kernel_us"] = t_kern * 1e6

    out = {
        "metric": "fused prefill+decode attn µs/layer; % of overlap roofline; speedup vs sequential",
        "value": t_step * 1e6,
        "unit": "µs/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": DESCR.get(args.config, spec.name), "name": spec.name,
                   "num_prefill": spec.num_prefill, "num_decode": spec.num_decode,
                   "cache_flush": not args.no_flush},
        "overlap_roofline_us": roof_s * 1e6,
        "overlap_roofline_frac": roof_s / t_step,
        "sequential_us": t_seq * 1e6,
        "speedup_vs_sequential": t_seq / t_step,
        "step_us_p10_p90": [float(np.percentile(step_ms, 10)) * 1e3,
                            float(np.percentile(step_ms, 90)) * 1e3],
        "sequential_us_p10_p90": [float(np.percentile(seq_ms, 10)) * 1e3,
                                  float(np.percentile(seq_ms, 90)) * 1e3],
        "warm_cache_step_us": warm_ms * 1e3,
        "achieved_tflops": counts["flops"] / t_step / 1e12,
        "achieved_hbm_gbs": counts["bytes"] / t_step / 1e9,
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
