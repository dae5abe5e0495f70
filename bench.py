"""Benchmark: fused prefill+decode attention of one hybrid batch on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-flush] [--no-cpu]
                    [--no-per-config] [--config-steps K2]
    python bench.py --pmc-run [--config NAME]          (driver for rocprofv3 counter runs)
    python bench.py --summarize-ea DIR [--config NAME]  (writes profiles/traffic_*.md)
    python bench.py --summarize-counters DIR [--config NAME] (writes profiles/counters_*.md)
    python bench.py --summarize-stats DIR [--config NAME] (writes profiles/*_stats.md)

A step is one pass of the hot path over the batch: pod_attn_run, i.e. the fused
kernel (every prefill tile and decode split of the batch) and the log-sum-exp
merge of KV-split partials.  Inputs (bf16 Q/K/V, page tables) and the plan are
resident in HBM before the timed region.  Before each timed step a 1 GiB buffer
is written to evict the L2 caches and the 256 MB Infinity Cache, so every step
streams its KV cache from HBM; the write is outside the events.  HIP events
are recorded on the stream the kernels run on: around the whole step, and, in
as many launches right after the timed steps (through pod_attn_run_events),
immediately around the fused kernel, whose average launch duration the
roofline object uses.  The sequential baseline (prefill kernel, decode
kernel, merge; its own plan) and the pages' comparators (the two kernels on
two streams; every request through the prefill kernel; a persistent launch
over one prefill-then-decode queue) are timed the same way in the same run,
interleaved step by step with the fused path.  The fp64 CPU oracle is timed on
the host cores on a bounded sample of the batch.

The headline workload (default: the 70B-shaped layer at TP = 1, the largest
single-GPU configuration) is timed for exactly --steps steps per path; every
other workload and the batched mix's decode-count sweep follow in
`per_config` with --config-steps steps each.  A streaming-read probe over a
4 GiB buffer gives the attainable HBM read rate (`hbm_read_ceiling`).

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
    "llama2_7b_dec_bf16": "llama2-7b layer's decodes alone: 32q/32kv d128; 128 decodes @8192; "
                          "paged 16; bf16 KV",
    "llama2_7b_dec_fp8": "llama2-7b layer's decodes alone: 32q/32kv d128; 128 decodes @8192; "
                         "paged 16; FP8 E4M3 KV, per-head scales",
    "l70b_tp1_dec_bf16": "70b TP=1 layer's decodes alone: 64q/8kv d128; 256 decodes "
                         "kv~lognormal; paged 16; bf16 KV",
    "l70b_tp1_dec_fp8": "70b TP=1 layer's decodes alone: 64q/8kv d128; 256 decodes "
                        "kv~lognormal; paged 16; FP8 E4M3 KV, per-head scales",
    "l70b_prefix": "70b TP=1 layer, shared-prefix decodes: 64q/8kv d128; 128 decodes in 16 "
                   "groups of 8 sharing a 2048-token prefix + own U[64,1024]; paged 16; "
                   "fused = packed (PAT-style), sequential = unshared decode",
}
for _n in ("llama3_8b", "llama2_7b", "l70b_tp1", "batched"):
    DESCR[_n + "_fp8"] = DESCR[_n] + "; FP8 E4M3 KV, per-head scales"
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


def main_kernel(spec):
    """The kernel pod_attn_run launches for this workload (the roofline's): a
    batch of one kind runs the one kernel it needs."""
    if spec.prefix_groups:
        return "pod_decode_pack_kernel"
    if not spec.prefill_qo_len:
        return "pod_decode_fp8_kernel" if spec.kv_dtype == "fp8_e4m3" else "pod_decode_kernel"
    if not spec.decode_kv_len:
        return "pod_prefill_kernel"
    return "pod_fused_kernel"


def traffic_file(config, kernel):
    return os.path.join(PROFILES, f"traffic_{kernel}_{config}.md")


def read_traffic(config, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when there is none or the kernel sources changed since it was taken."""
    try:
        lines = open(traffic_file(config, kernel)).read().splitlines()
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


def _blas_build():
    """numpy's BLAS library and version, as numpy reports its build."""
    try:
        b = np.__config__.CONFIG["Build Dependencies"]["blas"]
        return f"{b.get('name', '?')} {b.get('version', '?')}"
    except (AttributeError, KeyError, TypeError):
        return "unknown"


def device_info(torch):
    """The GPU and its clocks at the start of the run: the device properties
    torch reports and the current shader / memory clock levels from
    `rocm-smi --showclocks --json` (None when the tool is not there or fails;
    it only reads)."""
    import subprocess
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2**30, 1), "clocks": None}
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                           text=True, timeout=20)
        card = next(iter(json.loads(r.stdout).values()))
        info["clocks"] = {k: v for k, v in card.items()
                          if k.lower().startswith(("sclk", "mclk", "fclk"))}
    except (OSError, subprocess.SubprocessError, ValueError, StopIteration, AttributeError):
        pass
    return info


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
    from prefill_decode_amd import metrics
    flops = metrics.algorithmic_counts(spec)["flops"]
    return {"value": est * 1e6, "unit": "µs/layer", "cores": workers, "kind": "oracle",
            "gflops_fp64": flops / est / 1e9, "blas": _blas_build(),
            "sample": f"{nr} of {n_rows} prefill rows and {nd} of {n_dec} decodes, evenly "
                      f"spaced ({pairs / total:.3g} of the visible query-key pairs), fp64 numpy, "
                      f"{dt:.1f} s, scaled by pairs; BLAS 1 thread per worker; CPU {_cpu_model()}"}


def pmc_run(args):
    """Driver for `rocprofv3 --pmc` runs: a few fused runs (the fused launch
    even where the plan would run the two kernels back to back), as many
    sequential runs, and one plain 1 GiB device-to-device copy."""
    import torch

    from prefill_decode_amd import binding as B
    from prefill_decode_amd import inputs

    torch.cuda.set_device(0)
    spec = inputs.config_spec(args.config, n_dec=args.n_dec)
    batch = inputs.make_batch_device(spec)
    runner = B.BatchRunner(batch)
    if runner.plan.info()["runs_sequential"]:
        # the plan runs the two kernels back to back or on two streams: count
        # the fused launch itself
        runner = B.BatchRunner(batch, B.make_tuning(sched_mode=B.SCHED_SPLIT))
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


# HBM traffic from the L2-to-memory request counters, in bytes by request
# size (no calibration): one pass for reads, one for writes
EA_READ = ["TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum",
           "TCC_EA0_RDREQ_sum"]
EA_WRITE = ["TCC_EA0_WRREQ_64B_sum", "TCC_EA0_WRREQ_sum"]
KERNELS = ("pod_fused_kernel", "pod_prefill_kernel", "pod_decode_kernel", "pod_decode_pack_kernel",
           "pod_decode_fp8_kernel", "pod_merge_kernel")


def _kernel_key(name):
    for k in KERNELS:
        if k in name:
            return k
    return "copy" if "copy" in name.lower() else None


def _load_counters(root):
    """{kernel: {counter: [value per dispatch, in dispatch order]}} from every
    counter CSV under root.  "copy" keeps only the last copy-like dispatch:
    the 1 GiB copy that ends `--pmc-run` (torch's own conversions and fills
    before it match the name too)."""
    import csv
    from collections import defaultdict
    rows = defaultdict(lambda: defaultdict(list))
    for f in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            k = _kernel_key(row["Kernel_Name"])
            if k is not None:
                rows[k][row["Counter_Name"]].append((int(row["Dispatch_Id"]),
                                                     float(row["Counter_Value"])))
    vals = defaultdict(dict)
    for k, cs in rows.items():
        for c, v in cs.items():
            v = sorted(v)
            vals[k][c] = [v[-1][1]] if k == "copy" else [x[1] for x in v]
    return vals


def summarize_ea(args):
    """Reads the EA_READ pass (DIR/rd) and the EA_WRITE pass (DIR/wr) over
    `--pmc-run` and writes profiles/traffic_pod_fused_kernel_<config>.md: HBM
    bytes per dispatch of every kernel, from request counts times request
    sizes; the 1 GiB copy of the same process checks the arithmetic."""
    rd, wr = _load_counters(os.path.join(args.summarize_ea, "rd")), \
        _load_counters(os.path.join(args.summarize_ea, "wr"))

    def rbytes(v, i):
        c32, c64, c128, tot = (v[c][i] for c in EA_READ)
        return 32 * c32 + 64 * c64 + 128 * c128, tot - c32 - c64 - c128

    def wbytes(v, i):
        c64, tot = (v[c][i] for c in EA_WRITE)
        return 64 * c64 + 32 * (tot - c64)

    from prefill_decode_amd import inputs, metrics
    spec = inputs.config_spec(args.config, n_dec=args.n_dec)
    fused = main_kernel(spec)
    if fused not in rd or fused not in wr or "copy" not in rd or "copy" not in wr:
        sys.exit("summarize-ea: missing kernel or copy dispatches in the counter CSVs")
    rows, res = [], {}
    for k in (fused,) + tuple(x for x in KERNELS if x != fused) + ("copy",):
        if k not in rd or k not in wr:
            continue
        r = [rbytes(rd[k], i) for i in range(len(rd[k][EA_READ[0]]))]
        w = [wbytes(wr[k], i) for i in range(len(wr[k][EA_WRITE[0]]))]
        n = min(len(r), len(w))
        rb, wb = float(np.mean([x[0] for x in r])), float(np.mean(w))
        other = int(max(x[1] for x in r))
        res[k] = (rb, wb)
        rows.append(f"| `{k}` | {n} | {rb / 1e6:.2f} | {wb / 1e6:.2f} | {other} |")
    alg = metrics.algorithmic_counts(spec)["bytes"]
    f_b, w_b = res[fused]
    c_r, c_w = res["copy"]
    txt = f"""# HBM traffic — {DESCR.get(args.config, args.config)}

Two `rocprofv3 --pmc` passes over `bench.py --pmc-run` ({args.steps} runs of `pod_attn_run`, as
many of `pod_attn_sequential_run`, then one plain {COPY_BYTES}-byte device-to-device copy). Bytes
are the L2-to-memory requests times their sizes: reads 32 B x `TCC_EA0_RDREQ_32B` + 64 B x
`TCC_EA0_RDREQ_64B` + 128 B x `TCC_EA0_RDREQ_128B` (the last column counts read requests of any
other size: 0 means the three sizes cover every request), writes 64 B x `TCC_EA0_WRREQ_64B` + 32 B x
the rest. The copy reads and writes {COPY_BYTES / 1e6:.2f} MB by construction; measured here:
{c_r / 1e6:.2f} MB read, {c_w / 1e6:.2f} MB written.

Commands (from the repository root; `$D` = a scratch directory):

    cd /tmp && export TMPDIR=/tmp
    rocprofv3 --pmc {" ".join(EA_READ)} --output-format csv -d $D/rd -o run -- python3 bench.py --pmc-run --config {args.config} --steps {args.steps}
    rocprofv3 --pmc {" ".join(EA_WRITE)} --output-format csv -d $D/wr -o run -- python3 bench.py --pmc-run --config {args.config} --steps {args.steps}
    python3 bench.py --summarize-ea $D --config {args.config} --steps {args.steps}

| kernel | dispatches | read MB / dispatch | written MB / dispatch | other-size read requests |
|---|---|---|---|---|
""" + "\n".join(rows) + f"""

Algorithmic bytes of the batch (each Q/K/V/O/LSE byte once): {alg / 1e6:.2f} MB; traffic of
`{fused}` / algorithmic = {(f_b + w_b) / alg:.4f}.

- kernel: `{fused}`
- traffic_bytes_per_launch: `{f_b + w_b:.6g}`
- sources_sha256: `{sources_digest()}`
"""
    os.makedirs(PROFILES, exist_ok=True)
    open(traffic_file(args.config, fused), "w").write(txt)
    print(txt)


COUNTERS = ["MfmaUtil", "VALUBusy", "LdsBankConflict", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"]
# instruction mix per kernel (one pass)
INST_COUNTERS = ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS",
                 "SQ_INSTS_SALU", "SQ_INSTS_VMEM", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES"]


def summarize_counters(args):
    """Reads the COUNTERS pass (DIR/util) and the INST_COUNTERS pass
    (DIR/inst) over `--pmc-run` and writes profiles/counters_<config>.md: MFMA
    and VALU busy shares, LDS bank conflicts and the instruction mix per
    kernel (means over dispatches)."""
    util = _load_counters(os.path.join(args.summarize_counters, "util"))
    inst = _load_counters(os.path.join(args.summarize_counters, "inst"))
    if not util:
        sys.exit("summarize-counters: no kernel dispatches in the counter CSVs")
    lines, mix = [], []
    for k in KERNELS:
        if k not in util:
            continue
        v = util[k]
        mean = lambda c: float(np.mean(v[c])) if v.get(c) else float("nan")
        lines.append(f"| `{k}` | {len(v.get('MfmaUtil', []))} | {mean('MfmaUtil'):.1f} | "
                     f"{mean('VALUBusy'):.1f} | {mean('LdsBankConflict'):.4f} | "
                     f"{mean('SQ_LDS_BANK_CONFLICT'):.4g} | {mean('SQ_LDS_IDX_ACTIVE'):.4g} |")
        if k in inst:
            u = inst[k]
            im = lambda c: float(np.mean(u[c])) if u.get(c) else float("nan")
            mf = im("SQ_INSTS_MFMA")
            mix.append(f"| `{k}` | {mf:.4g} | {im('SQ_INSTS_VALU'):.4g} | "
                       f"{im('SQ_INSTS_VALU_TRANS_F32'):.4g} | {im('SQ_INSTS_LDS'):.4g} | "
                       f"{im('SQ_INSTS_SALU'):.4g} | {im('SQ_INSTS_VMEM'):.4g} | "
                       f"{(im('SQ_INSTS_VALU') - mf) / mf if mf > 0 else float('nan'):.2f} |")
    txt = f"""# MFMA and VALU busy, LDS bank conflicts, instruction mix — {DESCR.get(args.config, args.config)}

Two `rocprofv3 --pmc` passes over `bench.py --pmc-run` ({args.steps} runs of `pod_attn_run`, then
{args.steps} of `pod_attn_sequential_run`). `MfmaUtil` / `VALUBusy` = MFMA-busy / VALU-active cycles
summed over SIMDs / (GPU-active cycles x SIMDs), in percent, for the whole launch (idle SIMDs, launch
ramp and tail included). `LdsBankConflict` = bank-conflict cycles / conflict-free LDS cycles.
Instruction counts are per dispatch, summed over waves (`SQ_INSTS_VALU` includes the MFMAs).

Commands (from the repository root; `$D` = a scratch directory):

    cd /tmp && export TMPDIR=/tmp
    rocprofv3 --pmc {" ".join(COUNTERS)} --output-format csv -d $D/util -o run -- python3 bench.py --pmc-run --config {args.config} --steps {args.steps}
    rocprofv3 --pmc {" ".join(INST_COUNTERS)} --output-format csv -d $D/inst -o run -- python3 bench.py --pmc-run --config {args.config} --steps {args.steps}
    python3 bench.py --summarize-counters $D --config {args.config} --steps {args.steps}

| kernel | dispatches | MfmaUtil % | VALUBusy % | LdsBankConflict | SQ_LDS_BANK_CONFLICT | SQ_LDS_IDX_ACTIVE |
|---|---|---|---|---|---|---|
""" + "\n".join(lines) + """

| kernel | MFMA instrs | VALU instrs | of which exp/log (trans f32) | LDS instrs | SALU instrs | VMEM instrs | non-MFMA VALU per MFMA |
|---|---|---|---|---|---|---|---|
""" + "\n".join(mix) + f"""

- sources_sha256: `{sources_digest()}`
"""
    os.makedirs(PROFILES, exist_ok=True)
    open(os.path.join(PROFILES, f"counters_{args.config}.md"), "w").write(txt)
    print(txt)


def summarize_stats(args):
    """Reads a `rocprofv3 --kernel-trace --stats --output-format csv` run under
    DIR and writes profiles/<kernel>_<config>_stats.md."""
    import csv

    files = glob.glob(os.path.join(args.summarize_stats, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        sys.exit("summarize-stats: no kernel_stats.csv under " + args.summarize_stats)
    rows = list(csv.DictReader(open(files[0])))
    # per-dispatch durations from the trace of the same run (for the median,
    # which the bench's kernel time is too)
    durs, disp = {}, []
    for f in glob.glob(os.path.join(args.summarize_stats, "**", "*kernel_trace.csv"),
                       recursive=True):
        for r in csv.DictReader(open(f)):
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            durs.setdefault(r["Kernel_Name"], []).append((t1 - t0) / 1e3)
            disp.append((t0, t1, r["Kernel_Name"]))
    # dispatches that directly follow the bench's 1 GiB cache-evicting fill
    # (a fill kernel of 50 us or more): the cold-cache launches whose mean the
    # bench reports as the kernel time, without the warm-up and warm-cache ones
    disp.sort()
    cold = {}
    for prev, cur in zip(disp, disp[1:]):
        if "FillFunctor" in prev[2] and prev[1] - prev[0] >= 50_000:
            cold.setdefault(cur[2], []).append((cur[1] - cur[0]) / 1e3)
    lines = []
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].split("(")[0].replace("void ", "")
        if len(name) > 70:
            name = name[:67] + "..."
        med = durs.get(r["Name"])
        med = f"{float(np.median(med)):.1f}" if med else "-"
        c = cold.get(r["Name"])
        c = f"{float(np.mean(c)):.1f} ({len(c)})" if c else "-"
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {c} | {med} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f} |")
    txt = f"""# Kernel times — {DESCR.get(args.config, args.config)}

`rocprofv3 --kernel-trace --stats` over one `bench.py` run ({args.steps} timed steps after {args.warmup} warm-up
steps; each step runs `pod_attn_run` and `pod_attn_sequential_run`, each after a 1 GiB cache-evicting fill).

Commands (from the repository root; `$D` = a scratch directory):

    cd /tmp && export TMPDIR=/tmp
    rocprofv3 --kernel-trace --stats --output-format csv -d $D -o run -- python3 bench.py --config {args.config} --steps {args.steps} --warmup {args.warmup} --no-cpu --no-per-config --paths fused,seq
    python3 bench.py --summarize-stats $D --config {args.config} --steps {args.steps} --warmup {args.warmup}

"avg after fill" is the mean over the dispatches that directly follow a 1 GiB cache-evicting fill (their count
in brackets): the cold-cache launches of the timed steps and of the kernel-alone timing, whose mean the bench
reports as the kernel time. "avg" also counts the warm-up launches (the first ones run cold code and pages) and
the warm-cache loop.

| kernel | calls | avg µs | avg after fill µs (n) | median µs | min µs | max µs | % of GPU time |
|---|---|---|---|---|---|---|---|
""" + "\n".join(lines) + f"""

- sources_sha256: `{sources_digest()}`
"""
    os.makedirs(PROFILES, exist_ok=True)
    from prefill_decode_amd import inputs
    kernel = main_kernel(inputs.config_spec(args.config, n_dec=args.n_dec))
    out = os.path.join(PROFILES, f"{kernel}_{args.config}_stats.md")
    open(out, "w").write(txt)
    print(txt)


PATHS = ("fused", "seq", "streams", "batched", "ordered", "graph")
PATH_NAMES = {
    "fused": "pod_attn_run: one fused launch (+ merge)",
    "seq": "pod_attn_sequential_run: prefill kernel, decode kernel, merge on one stream",
    "streams": "pod_attn_streams_run: prefill and decode kernels on two streams, merge",
    "batched": "pod_attn_batched_prefill_run: every request through the prefill kernel "
               "(decodes as one-row chunks), merge",
    "ordered": "pod_attn_run with the ordered scheduler: one persistent launch over a unified "
               "queue, prefill units first",
    "graph": "pod_attn_run captured once into a HIP graph and replayed (the fused kernel's "
             "self-resetting counters; no launch overhead per kernel)",
    "fused_launch": "where the plan runs the two kernels back to back or on two streams "
                    "(plan.runs_sequential 1 or 2), the fused launch itself (an explicit "
                    "scheduler mode)",
}


class Timer:
    """Events recorded on the stream the kernels run on, with a cache-evicting
    1 GiB fill before each timed call (outside the events)."""

    def __init__(self, torch, flush):
        self.torch = torch
        self.stream = torch.cuda.current_stream()
        self.flush = flush
        self.buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda") if flush else None
        self.n = 0

    def ev(self):
        return self.torch.cuda.Event(enable_timing=True)

    def evict(self):
        if self.buf is not None:
            self.n += 1
            self.buf.fill_(self.n & 0xFF)

    def fused_kernel(self, runner, steps):
        """Launch durations (ms) of the fused kernel alone: events recorded
        by pod_attn_run_events immediately around its launch, on its stream,
        each launch after the cache-evicting fill."""
        kv = [(self.ev(), self.ev()) for _ in range(steps)]
        for a, b in kv:
            self.evict()
            runner.run_events(a, b)
        self.torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in kv])

    def interleaved(self, calls, steps, warmup):
        """Median-ready times (ms) of each named call, the calls interleaved
        step by step so that drift hits them alike; the order rotates every
        step, so that each call follows each other one equally often (a heavy
        call can leave the clocks lower for the next)."""
        for _ in range(warmup):
            for f in calls.values():
                f()
        self.torch.cuda.synchronize()
        evs = {k: [(self.ev(), self.ev()) for _ in range(steps)] for k in calls}
        names = list(calls)
        wall0 = time.perf_counter()
        for i in range(steps):
            for j in range(len(names)):
                k = names[(i + j) % len(names)]
                f = calls[k]
                self.evict()
                evs[k][i][0].record(self.stream)
                f()
                evs[k][i][1].record(self.stream)
        self.torch.cuda.synchronize()
        self.last_wall = time.perf_counter() - wall0
        return {k: np.array([a.elapsed_time(b) for a, b in v]) for k, v in evs.items()}


def read_ceiling(torch, B, timer, reps=5, gib=4):
    """Attainable HBM read rate: the library's streaming-read probe over a
    4 GiB buffer (the 256 MB Infinity Cache can hold under 7% of it), median
    of `reps` reads."""
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda").fill_(3)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    best = {}
    for blocks in (512, 1024, 2048):
        B.probe_read_bw(buf, sink, blocks)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = timer.ev(), timer.ev()
            a.record(timer.stream)
            B.probe_read_bw(buf, sink, blocks)
            b.record(timer.stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        best[blocks] = buf.numel() / (float(np.median(ts)) * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    k = max(best, key=best.get)
    return {"gbs": best[k], "probe_blocks": k, "bytes": gib << 30, "reps": reps,
            "by_blocks": {str(b): round(v, 1) for b, v in best.items()}}


def pct(a, q):
    return float(np.percentile(a, q)) * 1e3


def measure_config(torch, B, inputs, metrics, timer, name, n_dec, steps, warmup, tuning_kw,
                   paths=PATHS, spec=None):
    """Times every path on one workload; returns (runner, fields)."""
    if spec is None:
        spec = inputs.config_spec(name, n_dec=n_dec)
    if spec.prefix_groups:
        # a shared-prefix plan runs the packed path fused and the unshared
        # decode on the sequential and streams paths; it has no batched or
        # ordered variant
        paths = tuple(p for p in paths if p in ("fused", "seq", "streams"))
    if spec.kv_dtype == "fp8_e4m3":
        # the batched-prefill comparator reads bf16 caches only
        paths = tuple(p for p in paths if p != "batched")
    batch = inputs.make_batch_device(spec)
    counts = metrics.algorithmic_counts(spec)
    flags = B.FLAG_BATCHED_PREFILL if "batched" in paths else 0
    t0 = time.perf_counter()
    runner = B.BatchRunner(batch, B.make_tuning(flags=flags, **tuning_kw))
    torch.cuda.synchronize()
    plan_first_ms = (time.perf_counter() - t0) * 1e3
    # warm host planning alone (no device work, no allocation on the device)
    warm = []
    for _ in range(5):
        t0 = time.perf_counter()
        if spec.prefix_groups:
            grp = np.full(spec.num_decode, -1, dtype=np.int32)
            for gi, (m, _pl) in enumerate(spec.prefix_groups):
                grp[list(m)] = gi
            p = B.plan_shared_prefix_host(runner.params, spec.decode_kv_len, grp,
                                          [pl_ for _m, pl_ in spec.prefix_groups],
                                          B.make_tuning(**tuning_kw))
        else:
            p = B.plan_host(runner.params, spec.prefill_qo_len, spec.prefill_kv_len,
                            spec.decode_kv_len, B.make_tuning(flags=flags, **tuning_kw))
        warm.append((time.perf_counter() - t0) * 1e3)
        p.destroy()
    calls = {"fused": runner.run, "seq": runner.sequential_run}
    side = torch.cuda.Stream()
    if "streams" in paths:
        calls["streams"] = lambda: runner.streams_run(side)
    if "batched" in paths:
        calls["batched"] = runner.batched_prefill_run
    ordered = None
    if "ordered" in paths:
        ordered = B.BatchRunner(batch, B.make_tuning(sched_mode=B.SCHED_ORDERED))
        calls["ordered"] = ordered.run
    forced = None
    if runner.plan.info()["runs_sequential"]:
        forced = B.BatchRunner(batch, B.make_tuning(sched_mode=B.SCHED_SPLIT))
        calls["fused_launch"] = forced.run
    graph = None
    if "graph" in paths and spec.prefill_qo_len and spec.decode_kv_len and not spec.prefix_groups:
        # the fused step captured once (hybrid batches: the fused launch + merge)
        runner.run()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            runner.run()
        torch.cuda.synchronize()
        calls["graph"] = graph.replay
    t = timer.interleaved(calls, steps, warmup)
    # the fused kernel alone, as many launches again: events that
    # pod_attn_run_events records immediately around it (recorded inside the
    # timed steps, they would add their own gap to every fused step)
    kern = timer.fused_kernel(runner, steps)
    med = {k: float(np.median(v)) * 1e-3 for k, v in t.items()}
    t_step, t_kern = med["fused"], float(np.mean(kern)) * 1e-3
    roof_s = metrics.overlap_roofline_s(counts)
    info = runner.plan.info()
    f = {
        "workload": DESCR.get(spec.name, DESCR.get(name, spec.name)),
        "kv_dtype": spec.kv_dtype,
        "fused_us": t_step * 1e6,
        "fused_us_p10_p90": [pct(t["fused"], 10), pct(t["fused"], 90)],
        "fused_kernel_us": t_kern * 1e6,
        "fused_kernel_us_median": float(np.median(kern)) * 1e3,
        "sequential_us": med["seq"] * 1e6,
        "sequential_us_p10_p90": [pct(t["seq"], 10), pct(t["seq"], 90)],
        "speedup_vs_sequential": med["seq"] / t_step,
        "comparators_us": {k: med[k] * 1e6 for k in ("streams", "batched", "ordered", "graph",
                                                      "fused_launch") if k in med},
        "overlap_roofline_us": roof_s * 1e6,
        "overlap_roofline_frac_step": roof_s / t_step,
        "overlap_roofline_frac_kernel": roof_s / t_kern,
        "achieved_tflops": counts["flops"] / t_step / 1e12,
        "achieved_hbm_gbs": counts["bytes"] / t_step / 1e9,
        "algorithmic": {"gflop": counts["flops"] / 1e9, "gbytes": counts["bytes"] / 1e9},
        "achieved_hbm_gbs_kernel": counts["bytes"] / t_kern / 1e9,
        "traffic_bytes_per_launch": read_traffic(spec.name, main_kernel(spec)),
        "plan": {"first_call_ms": plan_first_ms, "host_warm_ms": float(np.median(warm)),
                 "prefill_items": info["prefill_items"], "decode_items": info["decode_items"],
                 "merge_tasks": info["merge_tasks"],
                 "prefill_quarters_per_cu": info["prefill_quarters_per_cu"],
                 "sched_mode": info["sched_mode"], "runs_sequential": info["runs_sequential"]},
    }
    del ordered, graph, forced
    return runner, batch, spec, counts, t, kern, f


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="l70b_tp1")
    ap.add_argument("--n-dec", type=int, default=None, help="batched: decode-count sweep point")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="time the headline workload only")
    ap.add_argument("--paths", default=",".join(PATHS),
                    help="paths timed on the headline workload (comma-separated subset of "
                         + ",".join(PATHS) + "; fused and seq are always timed)")
    ap.add_argument("--config-steps", type=int, default=10,
                    help="timed steps per path for the other workloads")
    ap.add_argument("--quarters", type=int, default=-1, help="prefill quarters per CU (-1 auto)")
    ap.add_argument("--prefill-splits", type=int, default=0, help="force prefill KV splits (0 auto)")
    ap.add_argument("--decode-splits", type=int, default=0, help="force decode KV splits (0 auto)")
    ap.add_argument("--sched", type=int, default=0,
                    help="0 auto, 1 co-locate on every CU, 2 ordered, 3 CU partition")
    ap.add_argument("--pmc-run", action="store_true")
    ap.add_argument("--summarize-stats", default=None, metavar="DIR")
    ap.add_argument("--summarize-counters", default=None, metavar="DIR")
    ap.add_argument("--summarize-ea", default=None, metavar="DIR")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(sharded by KV head or by request, each GPU would run this same kernel on its "
              "share with no exchange; this library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.summarize_stats:
        return summarize_stats(args)
    if args.summarize_counters:
        return summarize_counters(args)
    if args.summarize_ea:
        return summarize_ea(args)
    if args.pmc_run:
        return pmc_run(args)

    import torch

    from prefill_decode_amd import binding as B
    from prefill_decode_amd import inputs, metrics

    torch.cuda.set_device(0)
    device = device_info(torch)
    timer = Timer(torch, not args.no_flush)
    tuning_kw = dict(prefill_quarters_per_cu=args.quarters, sched_mode=args.sched,
                     prefill_kv_splits=args.prefill_splits, decode_kv_splits=args.decode_splits)
    # ---- the headline workload: exactly --steps timed steps per path ----
    print(f"bench: {args.config} ({args.steps} steps, {args.warmup} warm-up)", file=sys.stderr,
          flush=True)
    paths = tuple(p for p in PATHS if p in args.paths.split(",") or p in ("fused", "seq"))
    runner, batch, spec, counts, t, kern, head = measure_config(
        torch, B, inputs, metrics, timer, args.config, args.n_dec, args.steps, args.warmup,
        tuning_kw, paths=paths)
    wall = timer.last_wall
    # warm (no eviction) back-to-back fused steps
    w0, w1 = timer.ev(), timer.ev()
    w0.record(timer.stream)
    for _ in range(args.steps):
        runner.run()
    w1.record(timer.stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / args.steps

    t_step, t_kern = head["fused_us"] * 1e-6, head["fused_kernel_us"] * 1e-6
    hbm_bound = counts["bytes"] / metrics.PEAK_HBM_BYTES >= counts["flops"] / metrics.PEAK_BF16_FLOPS
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": counts["bytes"] / t_kern / 1e9,
                "peak": metrics.PEAK_HBM_BYTES / 1e9, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": counts["flops"] / t_kern / 1e12,
                "peak": metrics.PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = head["traffic_bytes_per_launch"]
    roof["kernel"] = main_kernel(spec)
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
        "config": {"workload": head["workload"], "name": spec.name,
                   "num_prefill": spec.num_prefill, "num_decode": spec.num_decode,
                   "cache_flush": not args.no_flush},
        "overlap_roofline_us": head["overlap_roofline_us"],
        "overlap_roofline_frac": head["overlap_roofline_frac_step"],
        "sequential_us": head["sequential_us"],
        "speedup_vs_sequential": head["speedup_vs_sequential"],
        "step_us_p10_p90": head["fused_us_p10_p90"],
        "sequential_us_p10_p90": head["sequential_us_p10_p90"],
        "comparators_us": head["comparators_us"],
        "comparator_paths": PATH_NAMES,
        "warm_cache_step_us": warm_ms * 1e3,
        "achieved_tflops": head["achieved_tflops"],
        "achieved_hbm_gbs": head["achieved_hbm_gbs"],
        "algorithmic": head["algorithmic"],
        "plan": head["plan"],
        "wall_s_timed_loop": wall,
        "roofline": roof,
        "device": device,
    }
    del runner
    torch.cuda.empty_cache()
    out["hbm_read_ceiling"] = read_ceiling(torch, B, timer)
    out["roofline"]["frac_of_read_ceiling"] = roof["achieved"] / out["hbm_read_ceiling"]["gbs"] \
        if hbm_bound else None
    if not args.no_per_config:
        per = {}
        todo = [(n, None) for n in inputs.CONFIG_NAMES] + [("batched", n) for n in (32, 64, 128, 256)]
        for name, nd in todo:
            key = name if nd is None else f"batched_d{nd}"
            if name == args.config and nd == args.n_dec:
                per[key] = head
                continue
            print(f"bench: {key}", file=sys.stderr, flush=True)
            r, *_rest, f = measure_config(torch, B, inputs, metrics, timer, name, nd,
                                          args.config_steps, 2, tuning_kw)
            per[key] = f
            del r, _rest
            torch.cuda.empty_cache()
        # the hybrid layers with an FP8 E4M3 cache (fused FP8 kernel against
        # the FP8 prefill and decode kernels run back to back)
        for name in ("llama3_8b", "llama2_7b", "l70b_tp1", "batched"):
            spec_f = inputs.fp8_spec(name)
            print(f"bench: {spec_f.name}", file=sys.stderr, flush=True)
            r, *_rest, f = measure_config(torch, B, inputs, metrics, timer, name, None,
                                          args.config_steps, 2, tuning_kw,
                                          paths=("fused", "seq", "streams"), spec=spec_f)
            per[spec_f.name] = f
            del r, _rest
            torch.cuda.empty_cache()
        # decode-only batches with a bf16 and an FP8 E4M3 cache: the decodes
        # of the llama2-7b and 70B-shaped layers
        for name in ("llama2_7b", "l70b_tp1"):
            for dt in ("bf16", "fp8_e4m3"):
                spec_d = inputs.decode_only_spec(name, dt)
                print(f"bench: {spec_d.name}", file=sys.stderr, flush=True)
                r, *_rest, f = measure_config(torch, B, inputs, metrics, timer, name, None,
                                              args.config_steps, 2, tuning_kw,
                                              paths=("fused", "seq"), spec=spec_d)
                per[spec_d.name] = f
                del r, _rest
                torch.cuda.empty_cache()
        # decode-only batch with shared prefixes: the packed path (fused
        # field) against the unshared decode of the same batch (sequential)
        spec_p = inputs.config_spec("l70b_prefix")
        print(f"bench: {spec_p.name}", file=sys.stderr, flush=True)
        r, *_rest, f = measure_config(torch, B, inputs, metrics, timer, spec_p.name, None,
                                      args.config_steps, 2, tuning_kw,
                                      paths=("fused", "seq"), spec=spec_p)
        f["algorithmic"]["gbytes_unshared"] = metrics.algorithmic_counts(spec_p)[
            "bytes_unshared"] / 1e9
        per[spec_p.name] = f
        del r, _rest
        torch.cuda.empty_cache()
        out["per_config"] = per
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(batch, spec)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
