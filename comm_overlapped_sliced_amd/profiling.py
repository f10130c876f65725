"""rocprofv3 harness of the benchmark: the counter passes behind the roofline evidence, and the
text summaries kept under profiles/.

    python -m comm_overlapped_sliced_amd.profiling run --raw rocprof_raw
    python -m comm_overlapped_sliced_amd.profiling summarize --raw rocprof_raw --out profiles

`run` launches, one after the other and each under its own time limit, rocprofv3 on bench.py:
  1. --kernel-trace --stats: per-kernel durations of the step (no exposure sweep, no oracle);
  2. --pmc FETCH_SIZE and 3. --pmc WRITE_SIZE (each a run of its own): HBM bytes per dispatch,
     with a plain copy of known size in the same run to scale the counters;
  4. --pmc of the MFMA counters: bf16 MFMA operations (x 512 = flops) and MFMA-busy cycles;
  5. --memory-copy-trace: the emulated transfers (SDMA copies) of the step;
  6. --kernel-trace --stats of the whole benchmark (every section), for its list of kernels;
  7.-9. the resident attention (`attn_run`): kernel trace, then two SQ counter passes.
`--passes a,b` runs only those.
It stops at the first pass that fails. rocprofv3 is the program started, with python after
`--`; this module itself never touches the GPU.

`summarize` reads those outputs and writes, for the GEMM launches of the step (Flash-AG on the
Llama-3.1-70B gate+up share, Flash-RS on the down share):
  - gemm_bf16_kernel_l70b_mlp_step_kernel_trace.md (durations; bench.py's own timing of the
    same run beside them),
  - gemm_bf16_kernel_l70b_mlp_step_hbm_counters.md and traffic.json (bytes per launch, the
    counters' scale from the copy, the algorithmic bytes, and the sha256 of the kernel source
    they were taken on: bench.py reports them only while the source is unchanged),
  - gemm_bf16_kernel_l70b_mlp_step_mfma_counters.md (counted MFMA flops against 2MNK, busy
    cycles per SIMD and the busy share at the nominal and at the sampled shader clock);
  - sdma_copies_l70b_mlp_step_copy_trace.md and all_kernels_l70b_bench_kernel_trace.md from
    passes 5 and 6, attn_kernel_l70b_ulysses_s8192.md from passes 7-9, when their outputs are
    there.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
KERNEL_SRC = os.path.join(HERE, "csrc", "fo_gemm.hip")
CALIB_BYTES = 268435456
COUNTER_STEPS = 3  # timed steps of the counter passes
N_SIMD = 1024  # 256 CUs x 4 SIMDs

ATTN_SEQ = 8192
ATTN_ARGS = ["-m", "comm_overlapped_sliced_amd.attn_run", "--seq", str(ATTN_SEQ)]
# two passes of at most 8 SQ counters each
ATTN_PMC = (["SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES",
             "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_INSTS_VALU", "SQ_INSTS_LDS"],
            ["SQ_WAIT_INST_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY",
             "SQ_INSTS_MFMA", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_VALU_TRANS_F32", "SQ_WAIT_ANY"])
N_SE = 32  # shader engines (SQ_BUSY_CYCLES sums one count per engine)

# the step alone: no exposure sections, no oracle, no clock sampler; a short back-to-back window
# before the timed steps where timing matters (trace, copies), none where only counts do
STEP_ARGS = ["bench.py", "--no-exposure", "--cpu-seconds", "0", "--clock-seconds", "0"]
PASSES = [
    # (name, rocprofv3 options, bench argv, time limit in seconds)
    ("trace", ["--kernel-trace", "--stats"], STEP_ARGS + ["--steps", "10", "--warmup", "3"], 240),
    ("fetch", ["--pmc", "FETCH_SIZE", "--kernel-trace"],
     STEP_ARGS + ["--steps", str(COUNTER_STEPS), "--warmup", "1", "--settle-seconds", "0",
                  "--copy-calibration", str(CALIB_BYTES)], 180),
    ("write", ["--pmc", "WRITE_SIZE", "--kernel-trace"],
     STEP_ARGS + ["--steps", str(COUNTER_STEPS), "--warmup", "1", "--settle-seconds", "0",
                  "--copy-calibration", str(CALIB_BYTES)], 180),
    ("mfma", ["--pmc", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES",
              "--kernel-trace"],
     STEP_ARGS + ["--steps", str(COUNTER_STEPS), "--warmup", "1", "--settle-seconds", "0"], 180),
    ("copies", ["--kernel-trace", "--memory-copy-trace", "--stats"],
     STEP_ARGS + ["--steps", "10", "--warmup", "3", "--settle-seconds", "0.2"], 240),
    # the whole benchmark (every section and sweep), for the list of every kernel it launches
    ("bench", ["--kernel-trace", "--stats"],
     ["bench.py", "--cpu-seconds", "0", "--clock-seconds", "0", "--steps", "10", "--warmup", "3",
      "--settle-seconds", "0.5"], 420),
    # the resident attention on the 70B Ulysses share: its durations, then two counter passes
    ("attn", ["--kernel-trace", "--stats"], ATTN_ARGS + ["--calls", "50"], 180),
    ("attn_pmc1", ["--pmc", *ATTN_PMC[0], "--kernel-trace"], ATTN_ARGS + ["--calls", "3"], 120),
    ("attn_pmc2", ["--pmc", *ATTN_PMC[1], "--kernel-trace"], ATTN_ARGS + ["--calls", "3"], 120),
]

# the step's two GEMM launches: (kind, call, M, K, N, algorithmic read bytes, write bytes)
STEP = {
    "ag": ("fo_ag_gemm", 4096, 8192, 7168,
           4096 * 8192 * 2 + 8192 * 7168 * 2, 4096 * 7168 * 2),
    "rs": ("fo_gemm_rs", 4096, 3584, 8192,
           4096 * 3584 * 2 + 3584 * 8192 * 2 + 7 * 512 * 8192 * 4, 4096 * 8192 * 4),
}


def command(name: str, raw: str, python: str = sys.executable) -> list:
    """The argv of one pass."""
    for n, opts, bargs, _ in PASSES:
        if n == name:
            return (["rocprofv3", *opts, "--output-format", "csv", "-d",
                     os.path.join(raw, n), "-o", n, "--", python, *bargs])
    raise KeyError(name)


def command_text(name: str, raw: str) -> str:
    return " ".join(command(name, raw, "python3"))


def run(raw: str, only=None) -> int:
    os.makedirs(raw, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    for name, _, _, limit in PASSES:
        if only and name not in only:
            continue
        cmd = command(name, raw)
        print(f"pass {name}: {' '.join(cmd)}", flush=True)
        with open(os.path.join(raw, f"{name}.log"), "w") as log:
            try:
                rc = subprocess.run(cmd, cwd=ROOT, env=env, stdout=log, stderr=subprocess.STDOUT,
                                    timeout=limit).returncode
            except subprocess.TimeoutExpired:
                print(f"pass {name}: time limit {limit} s", flush=True)
                return 124
        print(f"pass {name}: rc {rc}", flush=True)
        if rc != 0:
            return rc
    return 0


# ---- summaries --------------------------------------------------------------------------

def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def _short(name: str) -> str:
    m = re.search(r"gemm_bf16_kernel<(\d+), (\d+), (\w+)>", name)
    if m:
        return f"gemm_bf16_kernel<{m.group(1)}, {m.group(2)}, {m.group(3)}>"
    m = re.search(r"(\w+)\(", name)
    return m.group(1) if m else name[:60]


def _timed_line(log: str) -> str:
    with open(log) as f:
        for line in f:
            if line.startswith("timed:"):
                return line.strip()[len("timed: "):]
    return "(no timed line)"


def _step_kernels(trace_csv: str):
    """Names of the step's Flash-AG and Flash-RS launches: bench.py's steps alternate AG and RS,
    so the kernels are the two GEMM instantiations that run equally often with the most calls."""
    counts = collections.Counter()
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            if "gemm_bf16_kernel" in r["Kernel_Name"]:
                counts[r["Kernel_Name"]] += 1
    names = [n for n, _ in counts.most_common()]
    ag = next(n for n in names if "<256, 256" in n)
    rs = next(n for n in names if n != ag)
    return {"ag": ag, "rs": rs}


def _per_dispatch(counter_csv: str):
    """{dispatch id: (kernel, grid, {counter: value})}."""
    out = {}
    with open(counter_csv) as f:
        for r in csv.DictReader(f):
            d = int(r["Dispatch_Id"])
            ent = out.setdefault(d, (r["Kernel_Name"], int(r["Grid_Size"]), {}))
            ent[2][r["Counter_Name"]] = ent[2].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def summarize(raw: str, out_dir: str, sclk_mhz: float | None = None) -> dict:
    sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    os.makedirs(out_dir, exist_ok=True)
    trace_dir = os.path.join(raw, "trace")
    stats_csv = _one(os.path.join(trace_dir, "**", "*kernel_stats.csv"))
    trace_csv = _one(os.path.join(trace_dir, "**", "*kernel_trace.csv"))
    names = _step_kernels(trace_csv)
    timed = _timed_line(os.path.join(raw, "trace.log"))

    # 1. kernel trace
    rows = ["| kernel | launches | total us | average us | min us | max us |",
            "|---|---|---|---|---|---|"]
    avg = {}
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            if "direct_copy" in r["Name"] or "elementwise" in r["Name"]:
                continue
            rows.append(f"| `{_short(r['Name'])}` | {r['Calls']} | "
                        f"{float(r['TotalDurationNs']) / 1e3:.1f} | {float(r['AverageNs']) / 1e3:.1f} | "
                        f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
            for k, n in names.items():
                if r["Name"] == n:
                    avg[k] = float(r["AverageNs"]) / 1e3
    # per-launch durations of the timed steps only (the trace also has the warm-up launches)
    dur = collections.defaultdict(list)
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            for k, n in names.items():
                if r["Kernel_Name"] == n:
                    dur[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    timed_avg = {k: statistics.mean(v[-10:]) for k, v in dur.items() if v}
    cmd = command_text("trace", raw)
    text = f"""# rocprofv3 kernel trace: Flash-AG + Flash-RS step, Llama-3.1-70B MLP rank share (P=8)

Flash-AG: fo_ag_gemm M=4096 K=8192 N=7168 bf16, `{_short(names['ag'])}`.
Flash-RS: fo_gemm_rs M=4096 K=3584 N=8192 with seven fp32 partials, `{_short(names['rs'])}`.
Emulated transfers on SDMA engines, one link per peer, each link an engine pair with every
transfer split across it; each GEMM launch's duration includes its in-kernel waits for them.

Command (from the repository root, TMPDIR=/tmp; `python -m comm_overlapped_sliced_amd.profiling run`
runs it as its first pass):

    {cmd}

Kernel statistics (the back-to-back window, 3 warm-up and 10 timed steps):

{chr(10).join(rows)}

Average of the 10 timed launches in the same trace: Flash-AG {timed_avg.get('ag', float('nan')):.1f} us,
Flash-RS {timed_avg.get('rs', float('nan')):.1f} us. bench.py's own HIP-event timing of the same run:
{timed}.

fo_gemm.hip sha256: {sha}
"""
    with open(os.path.join(out_dir, "gemm_bf16_kernel_l70b_mlp_step_kernel_trace.md"), "w") as f:
        f.write(text)

    # 2. HBM traffic
    fetch = _per_dispatch(_one(os.path.join(raw, "fetch", "**", "*counter_collection.csv")))
    write = _per_dispatch(_one(os.path.join(raw, "write", "**", "*counter_collection.csv")))

    def calib(d, counter):
        vals = [c[counter] for (n, _, c) in d.values() if "copyBuffer" in n and counter in c]
        return max(vals)

    cf, cw = calib(fetch, "FETCH_SIZE"), calib(write, "WRITE_SIZE")
    fs, ws = CALIB_BYTES / (cf * 1024), CALIB_BYTES / (cw * 1024)
    traffic, trows = {}, []
    for kind, name in names.items():
        fv = [c["FETCH_SIZE"] for d, (n, _, c) in sorted(fetch.items()) if n == name]
        wv = [c["WRITE_SIZE"] for d, (n, _, c) in sorted(write.items()) if n == name]
        # the timed launches: the last COUNTER_STEPS of the run
        ft, wt = statistics.mean(fv[-COUNTER_STEPS:]), statistics.mean(wv[-COUNTER_STEPS:])
        b = ft * 1024 * fs + wt * 1024 * ws
        call, M, K, N, ar, aw = STEP[kind]
        traffic[kind] = {"kernel": _short(name), "kernel_source_sha256": sha,
                         "fetch_kib_counter": round(ft, 1), "write_kib_counter": round(wt, 1),
                         "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
                         "bytes_per_launch": int(b), "algorithmic_read_bytes": ar,
                         "algorithmic_write_bytes": aw,
                         "launches": f"the {COUNTER_STEPS} timed ones of {len(fv)}"}
        trows.append(f"| `{_short(name)}` ({call}) | {', '.join(str(round(x)) for x in fv)} | "
                     f"{', '.join(str(round(x)) for x in wv)} | {b / 1e6:.1f} MB | "
                     f"{(ar + aw) / 1e6:.1f} MB | {b / (ar + aw):.2f} |")
    with open(os.path.join(out_dir, "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    text = f"""# HBM traffic of the GEMM kernels (rocprofv3 counters), Llama-3.1-70B MLP rank share

Commands (each a run of its own, from the repository root with TMPDIR=/tmp; passes 2 and 3 of
`python -m comm_overlapped_sliced_amd.profiling run`):

    {command_text('fetch', raw)}
    {command_text('write', raw)}

Calibration: the same runs copy {CALIB_BYTES} bytes with one plain copy kernel
(`__amd_rocclr_copyBuffer`), whose counters read FETCH_SIZE {cf:.0f} KiB and WRITE_SIZE {cw:.0f} KiB;
scale factors (true bytes / counter bytes): fetch {fs:.4f}, write {ws:.4f}.

| kernel | FETCH_SIZE KiB per launch (set-up, warm-up, timed) | WRITE_SIZE KiB per launch | scaled bytes per timed launch | algorithmic read + write bytes | ratio |
|---|---|---|---|---|---|
{chr(10).join(trows)}

Algorithmic bytes: X and W read once, the partials read once (Flash-RS), outputs written once.

fo_gemm.hip sha256: {sha}
"""
    with open(os.path.join(out_dir, "gemm_bf16_kernel_l70b_mlp_step_hbm_counters.md"), "w") as f:
        f.write(text)

    # 3. MFMA counters
    mf_dir = os.path.join(raw, "mfma")
    mf = _per_dispatch(_one(os.path.join(mf_dir, "**", "*counter_collection.csv")))
    mdur = {}
    with open(_one(os.path.join(mf_dir, "**", "*kernel_trace.csv"))) as f:
        for r in csv.DictReader(f):
            mdur[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    lines = []
    for d, (n, _, c) in sorted(mf.items()):
        kind = next((k for k, nm in names.items() if nm == n), None)
        if kind is None:
            continue
        call, M, K, N, _, _ = STEP[kind]
        flops = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", float("nan")) * 512
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / N_SIMD
        t = mdur.get(d, float("nan"))
        at = f"{busy / (t * 1e-6 * sclk_mhz * 1e6):.3f}" if sclk_mhz else "n/a"
        lines.append(f"| {call} | {d} | {t:.1f} | {flops:.4e} | {2 * M * N * K:.4e} | {busy:.0f} | "
                     f"{busy / (t * 1e-6 * 2.4e9):.3f} | {at} |")
    text = f"""# MFMA counters of the GEMM kernels, Llama-3.1-70B MLP rank share (P=8)

Command (from the repository root with TMPDIR=/tmp, a run of its own; pass 4 of
`python -m comm_overlapped_sliced_amd.profiling run`):

    {command_text('mfma', raw)}

MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512. Busy cycles per SIMD = SQ_VALU_MFMA_BUSY_CYCLES /
{N_SIMD} SIMDs. The busy share divides them by the launch's cycles at the nominal 2.4 GHz and at
{f'{sclk_mhz:.0f} MHz, the shader clock the benchmark sampled from the SMU under this load' if sclk_mhz else 'the sampled clock (none given)'}.

| call | dispatch | duration us | MFMA flops (counter) | 2MNK | MFMA busy cycles / SIMD | busy at 2.4 GHz | busy at sampled clock |
|---|---|---|---|---|---|---|---|
{chr(10).join(lines)}

fo_gemm.hip sha256: {sha}
"""
    with open(os.path.join(out_dir, "gemm_bf16_kernel_l70b_mlp_step_mfma_counters.md"), "w") as f:
        f.write(text)
    return traffic


def _col(row: dict, *names):
    """The first of `names` that the CSV row has (rocprofv3's column names vary by version)."""
    for n in names:
        if n in row and row[n] != "":
            return row[n]
    return None


# the step's device-to-device copies, in issue order: Flash-AG 7 peers x 2 row groups x 2 halves,
# then Flash-RS 7 peers x 4 row groups x 2 halves (each link an engine pair, every transfer cut
# in two halves); the engines' warm-up copies come before the first step
STEP_COPIES = (("Flash-AG row-group half (128 of its 256 rows x 8192 bf16)", 7 * 2 * 2, 2 << 20),
               ("Flash-RS row-group half (64 of its 128 rows x 8192 fp32)", 7 * 4 * 2, 2 << 20))


def summarize_copies(raw: str, out_dir: str) -> None:
    """sdma_copies_l70b_mlp_step_copy_trace.md: the emulated transfers of the step's calls. The
    trace has no byte counts, so each copy is named by its place in the step's issue order."""
    d = os.path.join(raw, "copies")
    copy_csv = _one(os.path.join(d, "**", "*memory_copy_trace.csv"))
    d2d, h2d = [], []
    with open(copy_csv) as f:
        for r in csv.DictReader(f):
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            kind = _col(r, "Direction", "Operation", "Kind") or ""
            (d2d if "DEVICE_TO_DEVICE" in kind else h2d).append((t0, t1))
    d2d.sort()
    per_step = sum(n for _, n, _ in STEP_COPIES)
    warm = len(d2d) % per_step
    classes = collections.defaultdict(list)
    classes[("engine warm-up at start-up", None)] = [b - a for a, b in d2d[:warm]]
    for i, (a, b) in enumerate(d2d[warm:]):
        k = i % per_step
        for name, n, size in STEP_COPIES:
            if k < n:
                classes[(name, size)].append(b - a)
                break
            k -= n
    classes[("host to device (input staging)", None)] = [b - a for a, b in h2d]
    rows = ["| copy | bytes (by construction) | copies | median us | p10 / p90 us | GB/s per engine at the median |",
            "|---|---|---|---|---|---|"]
    for (name, size), ts in classes.items():
        if not ts:
            continue
        ts = sorted(t / 1e3 for t in ts)
        med = statistics.median(ts)
        p10, p90 = ts[len(ts) // 10], ts[(9 * len(ts)) // 10]
        gbs = f"{size / (med * 1e-6) / 1e9:.1f}" if size and med > 0 else "n/a"
        rows.append(f"| {name} | {size or 'n/a'} | {len(ts)} | {med:.1f} | {p10:.1f} / {p90:.1f} "
                    f"| {gbs} |")
    steps = (len(d2d) - warm) / per_step
    timed = _timed_line(os.path.join(raw, "copies.log"))
    text = f"""# Emulated transfers: SDMA copy trace, Llama-3.1-70B MLP step (P=8, rank 0)

Command (from the repository root, TMPDIR=/tmp; `python -m comm_overlapped_sliced_amd.profiling
run --raw {raw} --passes copies`):

    {command_text('copies', raw)}

Each link is an engine pair (engines 2k and 2k+1, which share one bandwidth) and every transfer
is cut in two halves, one per engine of the pair, started together. One row group of one peer is
therefore two ~2 MiB copies: per step, Flash-AG 7 peers x 2 row groups of 256 rows x 8192 bf16
and Flash-RS 7 peers x 4 row groups of 128 rows x 8192 fp32, {per_step} copies. This rocprofv3
trace carries no byte counts: each copy is classed by its place in that issue order (the
warm-up copies come first; {steps:.0f} steps traced: the first call, the back-to-back window,
the warm-up and the timed steps).

{chr(10).join(rows)}

A pair moves one 4 MiB row group in about the time of one half; the two halves of a link share
its bandwidth, so the rate per link is about twice the per-engine figure.

rocprofv3's copy tracing logs "bad original signal value in async_copy_handler" for these copies:
the two halves of a transfer count down one completion signal, which its handler does not
expect. The run completed, and its in-kernel waits reported no error. Copy tracing also slows
the step; this run's timed steps: {timed}.
"""
    with open(os.path.join(out_dir, "sdma_copies_l70b_mlp_step_copy_trace.md"), "w") as f:
        f.write(text)


def summarize_bench(raw: str, out_dir: str) -> None:
    """all_kernels_l70b_bench_kernel_trace.md: every kernel the whole benchmark launches."""
    d = os.path.join(raw, "bench")
    stats_csv = _one(os.path.join(d, "**", "*kernel_stats.csv"))
    rows = ["| kernel | launches | total us | average us | min us | max us | % |",
            "|---|---|---|---|---|---|---|"]
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            pct = r.get("Percentage")
            pct = f"{float(pct):.2f}" if pct else "n/a"
            rows.append(f"| `{_short(r['Name'])}` | {r['Calls']} | "
                        f"{float(r['TotalDurationNs']) / 1e3:.1f} | {float(r['AverageNs']) / 1e3:.1f} | "
                        f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {pct} |")
    timed = _timed_line(os.path.join(raw, "bench.log"))
    sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    text = f"""# rocprofv3 kernel trace of the whole benchmark run (all sections), Llama-3.1-70B shares

Every kernel bench.py launches: the sliced GEMMs (Flash-AG, Flash-RS, the monolithic reference,
the SwiGLU-epilogue form), the query-split attention (`attn_kernel`), the SwiGLU activation, the
data-slicing reduce, and the small wait/release kernels of the transfer-only timings. The GEMM
rows mix every variant the benchmark times (slices resident or arriving, one engine pair per
peer or one link, ranks 0 and 7, the 1K-16K-token and 405B workloads), so only the attention and
activation rows come close to single-configuration figures.

Command (from the repository root, TMPDIR=/tmp; `python -m comm_overlapped_sliced_amd.profiling
run --raw {raw} --passes bench`):

    {command_text('bench', raw)}

{chr(10).join(rows)}

The same run's timed steps: {timed}.

fo_gemm.hip sha256: {sha}
"""
    with open(os.path.join(out_dir, "all_kernels_l70b_bench_kernel_trace.md"), "w") as f:
        f.write(text)


def _attn_timed(log: str) -> str:
    with open(log) as f:
        for line in f:
            if line.startswith("attn timed:"):
                return line.strip()[len("attn timed: "):]
    return "(no timed line)"


def summarize_attn(raw: str, out_dir: str) -> None:
    """attn_kernel_l70b_ulysses_s8192.md: durations and counters of the resident attention."""
    src = os.path.join(HERE, "csrc", "fo_attn.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    stats_csv = _one(os.path.join(raw, "attn", "**", "*kernel_stats.csv"))
    row = None
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            if "attn_kernel" in r["Name"]:
                row = r
    cnt, dur = {}, []
    for name in ("attn_pmc1", "attn_pmc2"):
        disp = _per_dispatch(_one(os.path.join(raw, name, "**", "*counter_collection.csv")))
        ids = sorted(d for d, (n, _, _) in disp.items() if "attn_kernel" in n)[-3:]
        for c in ATTN_PMC[0 if name == "attn_pmc1" else 1]:
            cnt[c] = statistics.mean(disp[d][2].get(c, float("nan")) for d in ids)
        with open(_one(os.path.join(raw, name, "**", "*kernel_trace.csv"))) as f:
            t = {int(r["Dispatch_Id"]): (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                 for r in csv.DictReader(f)}
        dur += [t[d] for d in ids if d in t]
    us = statistics.mean(dur)
    cycles = cnt["SQ_BUSY_CYCLES"] / N_SE
    mfma = cnt["SQ_INSTS_MFMA"]
    lines = [
        f"| counted MFMA instructions (32x32x16 bf16) | {mfma:.4g} |",
        f"| kernel cycles: SQ_BUSY_CYCLES / {N_SE} shader engines | {cycles:.4g} "
        f"({cycles / us:.0f} MHz over the {us:.1f} us launches) |",
        f"| MFMA busy share: SQ_VALU_MFMA_BUSY_CYCLES / {N_SIMD} SIMDs / kernel cycles | "
        f"{cnt['SQ_VALU_MFMA_BUSY_CYCLES'] / N_SIMD / cycles:.3f} |",
        f"| VALU instructions other than MFMA, per MFMA | "
        f"{(cnt['SQ_INSTS_VALU'] - mfma) / mfma:.2f} |",
        f"| transcendental (exp2) instructions per MFMA | {cnt['SQ_INSTS_VALU_TRANS_F32'] / mfma:.2f} |",
        f"| VALU issue: SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES | "
        f"{cnt['SQ_ACTIVE_INST_VALU'] / cnt['SQ_WAVE_CYCLES']:.3f} |",
        f"| LDS issue: SQ_ACTIVE_INST_LDS / SQ_WAVE_CYCLES | "
        f"{cnt['SQ_ACTIVE_INST_LDS'] / cnt['SQ_WAVE_CYCLES']:.3f} |",
        f"| LDS bank conflicts: SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE | "
        f"{cnt['SQ_LDS_BANK_CONFLICT'] / cnt['SQ_LDS_IDX_ACTIVE']:.4f} |",
        f"| waiting to issue: SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (second pass / first) | "
        f"{cnt['SQ_WAIT_INST_ANY'] / cnt['SQ_WAVE_CYCLES']:.3f} |",
        f"| waiting on LDS: SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES (second pass / first) | "
        f"{cnt['SQ_WAIT_INST_LDS'] / cnt['SQ_WAVE_CYCLES']:.3f} |",
    ]
    raw_rows = "\n".join(f"| {c} | {cnt[c]:.4e} |" for c in ATTN_PMC[0] + ATTN_PMC[1])
    stat = (f"{row['Calls']} launches, average {float(row['AverageNs']) / 1e3:.1f} us, min "
            f"{float(row['MinNs']) / 1e3:.1f}, max {float(row['MaxNs']) / 1e3:.1f}" if row else "n/a")
    text = f"""# rocprofv3: query-split attention (`attn_kernel`), Llama-3.1-70B Ulysses share, S = {ATTN_SEQ}

Resident attention (`fo_attn_ref`): 8 query heads, 1 key/value head of dimension 128, causal,
{ATTN_SEQ} tokens; seeded inputs of the bench's attention workload. Algorithmic work 4 d hq
(pairs attended) = 137.5 GFLOP.

Commands (from the repository root, TMPDIR=/tmp; `python -m comm_overlapped_sliced_amd.profiling
run --raw {raw} --passes attn,attn_pmc1,attn_pmc2`):

    {command_text('attn', raw)}
    {command_text('attn_pmc1', raw)}
    {command_text('attn_pmc2', raw)}

Kernel trace: {stat}. attn_run's own timing of the same run: {_attn_timed(os.path.join(raw, 'attn.log'))}.

Counters (mean over the three timed launches of each counter run):

| quantity | value |
|---|---|
{chr(10).join(lines)}

Raw counter sums per launch:

| counter | value |
|---|---|
{raw_rows}

fo_attn.hip sha256: {sha}
"""
    with open(os.path.join(out_dir, f"attn_kernel_l70b_ulysses_s{ATTN_SEQ}.md"), "w") as f:
        f.write(text)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(prog="python -m comm_overlapped_sliced_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--raw", default="rocprof_raw")
    r.add_argument("--passes", default="", help="comma-separated pass names (default: all)")
    s = sub.add_parser("summarize")
    s.add_argument("--raw", default="rocprof_raw")
    s.add_argument("--out", default="profiles")
    s.add_argument("--sclk-mhz", type=float, default=None)
    a = ap.parse_args(argv)
    if a.cmd == "run":
        return run(a.raw, [p for p in a.passes.split(",") if p])
    if os.path.isdir(os.path.join(a.raw, "trace")):
        print(json.dumps(summarize(a.raw, a.out, a.sclk_mhz), indent=1))
    if os.path.isdir(os.path.join(a.raw, "copies")):
        summarize_copies(a.raw, a.out)
    if os.path.isdir(os.path.join(a.raw, "bench")):
        summarize_bench(a.raw, a.out)
    if all(os.path.isdir(os.path.join(a.raw, n)) for n in ("attn", "attn_pmc1", "attn_pmc2")):
        summarize_attn(a.raw, a.out)
    return 0


if __name__ == "__main__":
    sys.exit(main())
