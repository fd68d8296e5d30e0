"""DF11 decompression throughput on one MI355X.

One step = one batched decompression of the Llama-3-8B-shaped transformer block
(q, k, v, o, gate, up, down; one DF11 stream, shared codebook, ~218M BF16
weights) into a scratch buffer, with the compressed stream already resident in
HBM.  Prints one JSON line.  --workload picks another input: the same block
with a codebook per weight (seven streams, one batched launch), or a single
stream (LM-head-sized 128256x4096, the 2^28 stress stream, ...).

  step      = a decode of the next of R device copies of the stream (each with
              its own output), R chosen so that between two uses of a copy
              the others move at least 768 MiB: no step finds its data in the
              L2 or the 256 MB MALL, as in a model that decodes each block
              once per forward
  value     = K * (algorithmic bytes per step) / (host wall time of the K
              timed steps), GB/s
  algorithmic bytes per step = EncodedExponent + PackedSignMantissa + Gaps
              + output positions + LUTs + CodeLengths (all unpadded) read,
              plus 2 bytes per BF16 weight written
  roofline  = the same bytes / (HIP events on the launch stream around the K
              timed steps / K) against the 8 TB/s HBM peak
  extras    = hot_kernel_ms (one copy decoded back to back), and
              flushed_kernel_ms_median (50 launches, each after a 1 GiB read,
              each between events recorded around it)
  cpu_baseline = the CPU oracle's tree-walk decoder on the same data, over
              the stream's groups on the job's share of host cores, and on one
              core
Before the W warmup steps the script decodes for SETTLE_S seconds, so that the
GPU clocks have settled whatever W is.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

REPO = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, REPO)

HBM_PEAK_GBPS = 8000.0
FLUSHED_LAUNCHES = 50  # launches after a 1 GiB read, after the timed ones
SETTLE_S = 0.15  # seconds of decoding before the warmup steps (GPU clocks)
DEFAULT_WORKLOAD = "llama3_8b_block"
WORKLOAD_CHOICES = ["llama3_8b_block", "llama3_8b_block_per_weight", "lm_head_128256x4096", "stress_2p28_zipf",
                    "mlp_14336x4096_t5", "proj_4096x4096_outliers", "single_1024x1024"]
METRIC = "DF11 decompress GB/s (compressed in + BF16 out) and % of MI355X HBM peak"
KERNEL_SRC = os.path.join(REPO, "entropy_decoding_df11_amd", "csrc", "df11_decode.hip")
PMC_SUMMARY = os.path.join(REPO, "profiles", "df11_decode_kernel_llama3_8b_block_pmc.json")


def _kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic_from_profile():
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel source; else None."""
    try:
        with open(PMC_SUMMARY) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != _kernel_hash():
        return None
    return d.get("hbm_bytes_per_launch")


# Host threads of the CPU baseline: a one-GPU job gets a share of 16 of the
# host's cores, whatever the machine's core count.
CPU_SHARE = 16


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_baselines(flat: np.ndarray, args) -> dict:
    """The oracle (test infrastructure) timed on the host: its tree-walk
    decoder over the whole stream on one core, and the same decoder over the
    stream's independent groups on every core of the job's share.  The rANS
    oracle has only the one-thread decoder."""
    import oracle
    usable = len(os.sched_getaffinity(0))
    cpu = {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": _cpu_model()}
    if args.coder == "rans":
        s = oracle.rans_encode(flat)
        t0 = time.perf_counter()
        out = oracle.rans_decode(s)
        dt = time.perf_counter() - t0
        algo = oracle.rans_compressed_bytes(s) + 2 * s["n_elements"]
        return {"value": round(algo / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"the whole {args.workload} data as one rANS stream ({flat.size} weights) decoded on one "
                          f"thread in {dt:.2f} s; output {'matches' if np.array_equal(out, flat) else 'DIFFERS FROM'} "
                          "the original weights", **cpu}
    threads = args.cpu_threads or min(usable, CPU_SHARE)
    s = oracle.encode(flat)
    algo = (s["total_bits"] + 7) // 8 + s["n_elements"] + (5 * s["n_threads"] + 7) // 8 \
        + 4 * (s["n_groups"] + 1) + 256 * (s["n_luts"] + 1) + 2 * s["n_elements"]
    out = np.zeros_like(flat)
    t0 = time.perf_counter()
    oracle.decode_groups_parallel(s, 0, s["n_groups"], out, threads)
    dt_all = time.perf_counter() - t0
    ok_all = bool(np.array_equal(out, flat))
    t0 = time.perf_counter()
    out1 = oracle.decode_treewalk(s)
    dt_one = time.perf_counter() - t0
    ok_one = bool(np.array_equal(out1, flat))
    outcome = lambda ok: "matches" if ok else "DIFFERS FROM"  # noqa: E731
    return {
        "value": round(algo / dt_all / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": f"the whole {args.workload} data as one stream ({flat.size} weights), tree-walk decode split by "
                  f"groups over {threads} threads (the job's share of the host, {usable} CPUs usable) in "
                  f"{dt_all:.2f} s; output {outcome(ok_all)} the original weights",
        "one_core": {"value": round(algo / dt_one / 1e9, 4), "unit": "GB/s", "cores": 1,
                     "sample": f"the same stream, tree-walk decode of every code in order on one thread in "
                               f"{dt_one:.2f} s; output {outcome(ok_one)} the original weights"},
        **cpu,
    }


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _pmc_per_dispatch(run_dir, counter):
    """{dispatch id: (kernel name, grid size, counter summed over instances)}"""
    per = {}
    for r in _read_csv(os.path.join(run_dir, "run_counter_collection.csv")):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        name, grid, v = per.get(d, (r["Kernel_Name"], int(r["Grid_Size"]), 0.0))
        per[d] = (name, grid, v + float(r["Counter_Value"]))
    return per


def _phase_rows(rows, bench):
    """Split a kernel's trace rows (in start order) into the bench run's
    phases, in the order the run launches them (bench["launches"])."""
    phases, at = {}, 0
    for name, count in bench["launches"].items():
        phases[name] = rows[at:at + count]
        at += count
    if at != len(rows):
        raise SystemExit(f"summarize: {len(rows)} launches in the trace, the bench line accounts for {at}")
    return phases


def summarize_decode_trace(prof_dir: str, sub: str, kernel: str, title: str, command: str, out_name: str) -> None:
    """profiles/ summary of a rocprofv3 --kernel-trace --stats run of this
    script (prof_dir/sub, its bench line in prof_dir/sub.json): the stats
    table, then the kernel's launches split into the run's phases, each
    phase's average duration from the trace timestamps against the bench
    line's own event timing of that phase."""
    with open(os.path.join(prof_dir, sub + ".json")) as f:
        bench = json.loads(f.read().strip().splitlines()[-1])
    stats = _read_csv(os.path.join(prof_dir, sub, "run_kernel_stats.csv"))
    rows = [r for r in _read_csv(os.path.join(prof_dir, sub, "run_kernel_trace.csv")) if kernel in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    phases = _phase_rows(rows, bench)
    algo = bench["config"]["compressed_bytes"] + 2 * bench["config"]["n_elements"]
    us = lambda rs: [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rs]  # noqa: E731
    lines = [f"# {title}: rocprofv3 kernel trace", "",
             "Command (from the repository root on a one-GPU MI355X machine; R = repository root, "
             "D = a directory for the raw results):", "", "    " + command, "",
             "| kernel | calls | average us | min us | max us | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in stats[:6]:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {r['Percentage']}% |")
    bench_us = {"timed": bench["kernel_ms"] * 1e3, "hot": bench["hot_kernel_ms"] * 1e3,
                "flushed": bench["flushed_kernel_ms_median"] * 1e3}
    lines += ["", f"The {kernel} launches of the run, by phase (trace timestamps; {algo} algorithmic bytes per "
              "launch).  The bench line times the timed and hot phases with HIP events around all of their "
              "launches (gaps between launches included) and the flushed phase with events around each launch "
              "(median):", "",
              "| phase | launches | trace average us | trace median us | min us | max us | GB/s (trace average) "
              "| of 8 TB/s | bench line us | trace / bench |", "|---|---|---|---|---|---|---|---|---|---|"]
    for name, rs in phases.items():
        if not rs:
            continue
        v = us(rs)
        avg = float(np.mean(v))
        b = bench_us.get(name)
        lines.append(f"| {name} | {len(v)} | {avg:.2f} | {float(np.median(v)):.2f} | {min(v):.2f} | {max(v):.2f} | "
                     f"{algo / (avg * 1e-6) / 1e9:.1f} | {algo / (avg * 1e-6) / 1e9 / HBM_PEAK_GBPS:.3f} | "
                     + (f"{b:.2f} | {avg / b:.3f} |" if b else "| |"))
    t = us(phases["timed"])
    lines += ["", f"Roofline basis (timed phase: every launch decodes the next of "
              f"{bench['rotation_copies']} copies, so none finds its data cached): trace average "
              f"{np.mean(t):.2f} us against the bench line's {bench_us['timed']:.2f} us, "
              f"frac {algo / (np.mean(t) * 1e-6) / 1e9 / HBM_PEAK_GBPS:.4f} from the trace against "
              f"{bench['roofline']['frac']:.4f} on the bench line.", "",
              "Bench line of the traced run:", "", "    " + json.dumps(bench), ""]
    with open(os.path.join(REPO, "profiles", out_name), "w") as f:
        f.write("\n".join(lines))


def summarize_traffic(prof_dir: str, commands: dict) -> None:
    """The HBM-traffic summary from two PMC runs of this script (prof_dir/fetch
    with --pmc FETCH_SIZE, prof_dir/write with --pmc WRITE_SIZE; the bench
    line of the fetch run in prof_dir/fetch.json).  FETCH_SIZE and WRITE_SIZE
    are KiB per dispatch; each is scaled by the ratio of known bytes to
    counted bytes of the plain copy kernel the same run launches (10 copies of
    a buffer of known size).  The median over the decode dispatches."""
    with open(os.path.join(prof_dir, "fetch.json")) as f:
        bench = json.loads(f.read().strip().splitlines()[-1])
    algo = bench["config"]["compressed_bytes"] + 2 * bench["config"]["n_elements"]
    copy_bytes = algo // 2

    def split(per):
        dec = [v for (name, _, v) in per.values() if "df11_decode" in name]
        cpy = [v for (name, _, v) in per.values() if "copyBuffer" in name and abs(v * 1024 - copy_bytes) < 0.6 * copy_bytes]
        return dec, cpy

    fetch_dec, fetch_cpy = split(_pmc_per_dispatch(os.path.join(prof_dir, "fetch"), "FETCH_SIZE"))
    write_dec, write_cpy = split(_pmc_per_dispatch(os.path.join(prof_dir, "write"), "WRITE_SIZE"))
    if not (fetch_dec and fetch_cpy and write_dec and write_cpy):
        raise SystemExit("summarize: decode or copy dispatches missing from the PMC runs")
    kib = lambda xs: float(np.median(xs))  # noqa: E731
    fetch_scale = copy_bytes / (kib(fetch_cpy) * 1024)
    write_scale = copy_bytes / (kib(write_cpy) * 1024)
    read_b = kib(fetch_dec) * 1024 * fetch_scale
    write_b = kib(write_dec) * 1024 * write_scale
    pmc = {
        "kernel": "df11_decode_kernel",
        "workload": "llama3_8b_block",
        "kernel_source_sha256_16": _kernel_hash(),
        "commands": {"fetch": commands["fetch"], "write": commands["write"]},
        "decode_fetch_kib_per_dispatch": kib(fetch_dec),
        "decode_write_kib_per_dispatch": kib(write_dec),
        "copy_bytes_per_dispatch": copy_bytes,
        "copy_fetch_kib_per_dispatch": kib(fetch_cpy),
        "copy_write_kib_per_dispatch": kib(write_cpy),
        "fetch_scale": round(fetch_scale, 4),
        "write_scale": round(write_scale, 4),
        "hbm_read_bytes_per_launch": int(read_b),
        "hbm_write_bytes_per_launch": int(write_b),
        "hbm_bytes_per_launch": int(read_b + write_b),
        "algorithmic_bytes_per_launch": algo,
        "traffic_over_algorithmic": round((read_b + write_b) / algo, 4),
    }
    with open(PMC_SUMMARY, "w") as f:
        json.dump(pmc, f, indent=1)
        f.write("\n")


def summarize_linear_profile(prof_dir: str, command: str) -> None:
    """profiles/ summary of a rocprofv3 --kernel-trace --stats run of
    bench.py --linear-tokens (prof_dir/lin_trace and prof_dir/lin.json).
    Every step launches the seven matrices in the same order, so the i-th
    fused launch of the run is matrix i mod 7; the first 1 + warmup steps
    are left out of the averages."""
    with open(os.path.join(prof_dir, "lin.json")) as f:
        bench = json.loads(f.read().strip().splitlines()[-1])
    names = list(bench["config"]["shapes"])
    rows = [r for r in _read_csv(os.path.join(prof_dir, "lin_trace", "run_kernel_trace.csv"))
            if "df11_linear_kernel" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    skip = (1 + bench["warmup"]) * len(names)
    per = {nm: [] for nm in names}
    for i, r in enumerate(rows):
        if i >= skip:
            per[names[i % len(names)]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    stats = _read_csv(os.path.join(prof_dir, "lin_trace", "run_kernel_stats.csv"))
    T = bench["config"]["tokens"]
    lines = [f"# df11_linear_kernel on llama3_8b_block_linear ({T} token{'s' if T > 1 else ''}): "
             "rocprofv3 kernel trace", "",
             "Command (from the repository root on a one-GPU MI355X machine):", "", "    " + command, "",
             "| kernel | calls | average us | min us | max us | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in stats[:8]:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {r['Percentage']}% |")
    lines += ["", "Fused launches per matrix after the warmup (trace timestamps) against the bench line's "
              "dispatch events:", "", "| matrix | shape | launches | average us | min us | bench line us |",
              "|---|---|---|---|---|---|"]
    total = 0.0
    for nm in names:
        v = per[nm]
        total += float(np.mean(v))
        lines.append(f"| {nm} | {bench['config']['shapes'][nm]} | {len(v)} | {np.mean(v):.2f} | {min(v):.2f} | "
                     f"{bench['per_matrix_us'][nm]:.2f} |")
    comp = bench["config"]["compressed_bytes"]
    lines += ["", f"Sum of the seven averages: {total:.1f} us per step for {comp} compressed bytes "
              f"({comp / (total * 1e-6) / 1e9:.0f} GB/s of compressed weights).", "",
              "Bench line of the traced run:", "", "    " + json.dumps(bench), ""]
    with open(os.path.join(REPO, "profiles", f"df11_linear_kernel_llama3_8b_block_t{T}_trace.md"), "w") as f:
        f.write("\n".join(lines))


def summarize_matmul_profile(prof_dir: str, sub: str, command: str) -> None:
    """profiles/ summary of a rocprofv3 --kernel-trace --stats run of
    bench.py --matmul-tokens T (prof_dir/sub, its line in prof_dir/sub.json):
    the stats table and the seven-product batched kernel's timed launches
    (trace timestamps) against the bench line."""
    with open(os.path.join(prof_dir, sub + ".json")) as f:
        bench = json.loads(f.read().strip().splitlines()[-1])
    stats = _read_csv(os.path.join(prof_dir, sub, "run_kernel_stats.csv"))
    rows = [r for r in _read_csv(os.path.join(prof_dir, sub, "run_kernel_trace.csv"))
            if "df11_gemm_batch_kernel" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    n = bench["launches"]
    timed = rows[n["check"] + n["warmup"]:n["check"] + n["warmup"] + n["timed"]]
    us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in timed]
    T = bench["config"]["tokens"]
    avg = float(np.mean(us))
    hbm = bench["config"]["compressed_bytes"] + sum(2 * T * c + 4 * T * r for r, c in bench["config"]["shapes"].values())
    lines = [f"# df11_gemm_batch_kernel on llama3_8b_block_matmul ({T} token{'s' if T > 1 else ''}): "
             "rocprofv3 kernel trace", "", "Command (from the repository root on a one-GPU MI355X machine; "
             "R = repository root, D = a directory for the raw results):", "", "    " + command, "",
             "| kernel | calls | average us | min us | max us | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in stats[:8]:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {r['Percentage']}% |")
    lines += ["", f"The {len(us)} timed launches of the batched fused kernel (all seven products in one launch; the "
              "kernel calls above also count the forward's smaller batches): trace average "
              f"{avg:.2f} us (min {min(us):.2f}, max {max(us):.2f}); {hbm / (avg * 1e-6) / 1e9:.1f} GB/s of "
              f"compressed weights + x + y, {hbm / (avg * 1e-6) / 1e9 / HBM_PEAK_GBPS:.3f} of 8 TB/s; "
              f"{2.0 * T * bench['config']['n_elements'] / (avg * 1e-6) / 1e12:.2f} TFLOP/s.  The bench line's "
              f"events give {bench['kernel_ms'] * 1e3:.2f} us per step (the fused kernel plus one zeroing kernel).",
              ""]
    # The forward's launches: one fill of the seven outputs, then q, k, v; o; gate, up; down (a batched
    # kernel for two or three products, the one-stream kernel for one), eagerly issued and graph-replayed.
    trace = sorted(_read_csv(os.path.join(prof_dir, sub, "run_kernel_trace.csv")),
                   key=lambda r: int(r["Start_Timestamp"]))
    is_gemm = lambda r: "df11_gemm_kernel" in r["Kernel_Name"] or "df11_gemm_batch_kernel" in r["Kernel_Name"]  # noqa: E731
    seqs = [trace[i:i + 5] for i in range(len(trace) - 4)
            if "Fill" in trace[i]["Kernel_Name"] and all(is_gemm(r) for r in trace[i + 1:i + 5])]
    if seqs:
        names = ["fill", "q, k, v", "o", "gate, up", "down"]
        shapes = bench["config"]["shapes"]
        weights = [0, sum(r * c for k, (r, c) in shapes.items() if k in ("q_proj", "k_proj", "v_proj")),
                   shapes["o_proj"][0] * shapes["o_proj"][1],
                   sum(r * c for k, (r, c) in shapes.items() if k in ("gate_proj", "up_proj")),
                   shapes["down_proj"][0] * shapes["down_proj"][1]]
        rate = avg / bench["config"]["n_elements"]  # us per weight in the one-launch product
        lines += [f"The forward's launches ({len(seqs)} sequences of a fill and four products, eager and graph "
                  "replays; medians): each launch against its weights at the one-launch product's rate.", "",
                  "| launch | kernel | us | gap before, us | us at the one-launch rate |", "|---|---|---|---|---|"]
        for j, nm in enumerate(names):
            dur = float(np.median([(int(q[j]["End_Timestamp"]) - int(q[j]["Start_Timestamp"])) / 1e3 for q in seqs]))
            gap = float(np.median([(int(q[j]["Start_Timestamp"]) - int(q[j - 1]["End_Timestamp"])) / 1e3
                                   for q in seqs])) if j else 0.0
            found = re.search(r"(df11_\w+<[^(]*?>|\w*Fill\w*)", seqs[0][j]["Kernel_Name"])
            kern = found.group(1) if found else seqs[0][j]["Kernel_Name"][:40]
            lines.append(f"| {nm} | `{kern}` | {dur:.2f} | {gap:.2f} | "
                         + (f"{weights[j] * rate:.2f} |" if weights[j] else "|"))
        total = float(np.median([(int(q[4]["End_Timestamp"]) - int(q[0]["Start_Timestamp"])) / 1e3 for q in seqs]))
        lines += ["", f"Fill start to down's end: {total:.2f} us (median).", ""]
    lines += ["Bench line of the traced run:", "", "    " + json.dumps(bench), ""]
    with open(os.path.join(REPO, "profiles", f"df11_gemm_kernel_llama3_8b_block_t{T}_trace.md"), "w") as f:
        f.write("\n".join(lines))


# The two rocprofv3 --pmc passes of the instruction-mix summary.  Each stays
# within one pass's hardware limits (8 SQ counters, counting those that the
# derived metrics VALUBusy, LDSBankConflict and VALUUtilization read, and one
# GRBM counter).
COUNTER_PASSES = {
    "sq_a": "VALUBusy LDSBankConflict SQ_WAVES SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_SALU SQ_LDS_IDX_ACTIVE "
            "SQ_LDS_BANK_CONFLICT",
    "sq_b": "VALUUtilization SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_INSTS_VMEM_RD "
            "SQ_INSTS_VMEM_WR",
}


def summarize_counters(prof_dir: str, kernel: str, title: str, bench_args: str, source: str, out_name: str) -> None:
    """profiles/ summary of the COUNTER_PASSES runs of `bench.py bench_args`
    (prof_dir/<kernel>_sq_a and _sq_b): every counter of the kernel's
    dispatches (median over them; rocprofv3 has already reduced each over the
    chip), rocprofv3's derived VALUBusy, LDSBankConflict and VALUUtilization,
    and per-wave instruction counts."""
    med = {}
    for sub in COUNTER_PASSES:
        per = {}
        for r in _read_csv(os.path.join(prof_dir, f"{kernel}_{sub}", "run_counter_collection.csv")):
            if kernel in r["Kernel_Name"]:
                per.setdefault(r["Counter_Name"], {})[int(r["Dispatch_Id"])] = float(r["Counter_Value"])
        if not per:
            raise SystemExit(f"summarize: no {kernel} dispatches in the {sub} counter run")
        for name, by_dispatch in per.items():
            med[name] = float(np.median(list(by_dispatch.values())))
    waves = med["SQ_WAVES"]
    with open(os.path.join(REPO, source), "rb") as f:
        src_hash = hashlib.sha256(f.read()).hexdigest()[:16]
    pre = "cd /tmp && export TMPDIR=/tmp && "
    lines = [f"# {title}: rocprofv3 counters", "",
             f"Kernel source `{source}`, sha256 prefix {src_hash}.  Commands (from the repository root on a "
             "one-GPU MI355X machine; R = repository root, D = a directory for the raw results):", ""]
    for sub, counters in COUNTER_PASSES.items():
        lines.append(f"    {pre}rocprofv3 --pmc {counters} -d $D/{kernel}_{sub} -o run --output-format csv "
                     f"-- python3 $R/bench.py {bench_args}")
    lines += ["", "Each value is the median over the kernel's dispatches in the run.", "",
              "| counter | value | per wave |", "|---|---|---|"]
    for name in sorted(med):
        per_wave = f"{med[name] / waves:.1f}" if name.startswith("SQ_INSTS") else ""
        lines.append(f"| {name} | {med[name]:.6g} | {per_wave} |")
    lines += ["",
              f"- VALUBusy {med['VALUBusy']:.1f}%: the share of the kernel's time that the vector ALUs issue "
              "(rocprofv3's derived metric, SQ_ACTIVE_INST_VALU over CUs and GRBM_GUI_ACTIVE).",
              f"- VALUUtilization {med['VALUUtilization']:.1f}%: lanes active per VALU instruction.",
              f"- LDSBankConflict {med['LDSBankConflict']:.1f}%: the share of the kernel's time the LDS stalls on "
              f"bank conflicts; conflict cycles are {100 * med['SQ_LDS_BANK_CONFLICT'] / med['SQ_LDS_IDX_ACTIVE']:.0f}% "
              "of the cycles the LDS spends on indexed operations (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE).",
              f"- Instructions per wave: {med['SQ_INSTS_VALU'] / waves:.0f} VALU, {med['SQ_INSTS_SALU'] / waves:.0f} "
              f"SALU, {med['SQ_INSTS_LDS'] / waves:.0f} LDS, {med['SQ_INSTS_VMEM_RD'] / waves:.0f} vector-memory "
              f"reads, {med['SQ_INSTS_VMEM_WR'] / waves:.0f} vector-memory writes.",
              f"- Waves wait on something {100 * med['SQ_WAIT_ANY'] / med['SQ_WAVE_CYCLES']:.0f}% of their "
              f"resident cycles, on LDS issue {100 * med['SQ_WAIT_INST_LDS'] / med['SQ_WAVE_CYCLES']:.1f}%.", ""]
    with open(os.path.join(REPO, "profiles", out_name), "w") as f:
        f.write("\n".join(lines))


def _per_step_counters(prof_dir: str, kernel: str, first: int, per_step: int) -> tuple:
    """Counters of `kernel` from the COUNTER_PASSES runs in prof_dir/<kernel>_<pass>:
    per-step totals of the SQ_ counters (the first `first` dispatches in
    dispatch order if first > 0, `per_step` dispatches to a step) and the
    medians of rocprofv3's derived percentages."""
    totals, pct, steps = {}, {}, 0.0
    for sub in COUNTER_PASSES:
        per = {}
        for r in _read_csv(os.path.join(prof_dir, f"{kernel}_{sub}", "run_counter_collection.csv")):
            if kernel in r["Kernel_Name"]:
                per.setdefault(r["Counter_Name"], {})[int(r["Dispatch_Id"])] = float(r["Counter_Value"])
        if not per:
            raise SystemExit(f"summarize: no {kernel} dispatches in the {sub} counter run")
        for name, by_dispatch in per.items():
            ids = sorted(by_dispatch)
            if first:
                ids = ids[:first]
            vals = [by_dispatch[i] for i in ids]
            if name.startswith("SQ_"):
                steps = len(ids) / per_step
                totals[name] = sum(vals) / steps
            else:
                pct[name] = float(np.median(vals))
    return totals, pct


def summarize_product_counters(prof_dir: str) -> None:
    """profiles/ comparison of the one-token fused products' counters: the
    row-order product (df11_linear_kernel, seven launches a step, bench.py
    --linear-tokens 1) against the matrix-core product (df11_gemm_batch_kernel,
    one launch a step, bench.py --matmul-tokens 1), as totals per step over
    the block's seven matrices."""
    lin, lin_pct = _per_step_counters(prof_dir, "df11_linear_kernel", 0, 7)
    with open(os.path.join(prof_dir, "mm_pmc.json")) as f:
        launches = json.loads(f.read().strip().splitlines()[-1])["launches"]
    first = launches["check"] + launches["settle"] + launches["warmup"] + launches["timed"]
    mm, mm_pct = _per_step_counters(prof_dir, "df11_gemm_batch_kernel", first, 1)
    pre = "cd /tmp && export TMPDIR=/tmp && "
    lines = ["# One-token fused product on llama3_8b_block: row-order against matrix-core kernel counters", "",
             "Commands (from the repository root on a one-GPU MI355X machine; R = repository root, "
             "D = a directory for the raw results):", ""]
    for kernel, bench_args in (("df11_linear_kernel", "--linear-tokens 1 --steps 3 --warmup 2 --no-cpu-baseline"),
                               ("df11_gemm_batch_kernel", "--matmul-tokens 1 --steps 3 --warmup 2")):
        for sub, counters in COUNTER_PASSES.items():
            lines.append(f"    {pre}rocprofv3 --pmc {counters} -d $D/{kernel}_{sub} -o run --output-format csv "
                         f"-- python3 $R/bench.py {bench_args}")
    lines += ["", "Before: the row-order product (`df11_linear_kernel`, dot products, one launch per matrix). "
              "After: the matrix-core product (`df11_gemm_batch_kernel`, tiles fed to "
              "`v_mfma_f32_16x16x32_bf16`, the seven matrices in one launch). Instruction and cycle counts "
              "are totals per step (all seven matrices); percentages are medians over the dispatches.", "",
              "| counter | row-order (before) | matrix-core (after) | after / before |", "|---|---|---|---|"]
    for name in sorted(lin):
        if name in mm:
            lines.append(f"| {name} | {lin[name]:.4g} | {mm[name]:.4g} | {mm[name] / lin[name]:.2f} |")
    for name in sorted(lin_pct):
        if name in mm_pct:
            lines.append(f"| {name} (%) | {lin_pct[name]:.1f} | {mm_pct[name]:.1f} | |")
    moved = sorted(((mm[n] / lin[n], n) for n in lin if n in mm and n.startswith("SQ_INSTS") and lin[n] > 0))
    lines += ["", "Instruction counts that moved most (after / before): "
              + ", ".join(f"{n} {r:.2f}" for r, n in moved[:3]) + ".",
              f"Wave-cycles per step {lin['SQ_WAVE_CYCLES']:.4g} before, {mm['SQ_WAVE_CYCLES']:.4g} after; waves "
              f"wait on something {100 * lin['SQ_WAIT_ANY'] / lin['SQ_WAVE_CYCLES']:.0f}% of their cycles before, "
              f"{100 * mm['SQ_WAIT_ANY'] / mm['SQ_WAVE_CYCLES']:.0f}% after.", ""]
    with open(os.path.join(REPO, "profiles", "fused_product_llama3_8b_block_t1_counters.md"), "w") as f:
        f.write("\n".join(lines))


def summarize_product_traffic(prof_dir: str) -> None:
    """profiles/ summary of the one-token matrix-core product's HBM traffic:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the batched kernel's
    seven-product launches in two PMC runs of bench.py --matmul-tokens 1
    (prof_dir/mm_fetch, prof_dir/mm_write, the first run's bench line in
    prof_dir/mm_fetch.json), scaled by the copy-kernel factors of the
    decoder's committed traffic summary (the same counters on the same GPU).
    Reads should be about the compressed weights plus x, and writes about y
    alone: W's BF16 never reaches HBM."""
    with open(PMC_SUMMARY) as f:
        cal = json.load(f)
    with open(os.path.join(prof_dir, "mm_fetch.json")) as f:
        bench = json.loads(f.read().strip().splitlines()[-1])
    launches = bench["launches"]
    first = launches["check"] + launches["settle"] + launches["warmup"] + launches["timed"]

    def kib(sub, counter):
        per = _pmc_per_dispatch(os.path.join(prof_dir, sub), counter)
        ids = sorted(d for d, (name, _, _) in per.items() if "df11_gemm_batch_kernel" in name)[:first]
        if not ids:
            raise SystemExit(f"summarize: no df11_gemm_batch_kernel dispatches in {sub}")
        return float(np.median([per[d][2] for d in ids])), len(ids)

    fetch_kib, n_f = kib("mm_fetch", "FETCH_SIZE")
    write_kib, n_w = kib("mm_write", "WRITE_SIZE")
    read_b = fetch_kib * 1024 * cal["fetch_scale"]
    write_b = write_kib * 1024 * cal["write_scale"]
    cfg = bench["config"]
    T = cfg["tokens"]
    comp = cfg["compressed_bytes"]
    shapes = list(cfg["shapes"].values())
    x_b = 2 * T * sum({c for _, c in shapes})  # matrices with the same in_features share one x
    y_b = 4 * T * sum(r for r, _ in shapes)
    bf16_b = 2 * cfg["n_elements"]
    pre = "cd /tmp && export TMPDIR=/tmp && "
    cmd = pre + "rocprofv3 --pmc {c} -d $D/{sub} -o run --output-format csv -- python3 $R/bench.py --matmul-tokens 1 " \
                "--steps 3 --warmup 2"
    lines = ["# df11_gemm_batch_kernel on llama3_8b_block (1 token): HBM traffic", "",
             "Commands (from the repository root on a one-GPU MI355X machine; R = repository root, D = a directory "
             "for the raw results):", "",
             "    " + cmd.format(c="FETCH_SIZE", sub="mm_fetch") + " > $D/mm_fetch.json",
             "    " + cmd.format(c="WRITE_SIZE", sub="mm_write"), "",
             f"Medians over the {n_f} and {n_w} seven-product launches of the runs; KiB scaled by the copy-kernel "
             f"factors of `df11_decode_kernel_llama3_8b_block_pmc.json` (FETCH_SIZE x{cal['fetch_scale']}, "
             f"WRITE_SIZE x{cal['write_scale']}).", "",
             "| | bytes per launch | against |", "|---|---|---|",
             f"| HBM reads | {read_b / 1e6:.1f} MB | compressed weights {comp / 1e6:.1f} MB + x {x_b / 1e3:.1f} KB: "
             f"{read_b / (comp + x_b):.3f}x |",
             f"| HBM writes | {write_b / 1e6:.3f} MB | y {y_b / 1e3:.1f} KB; the BF16 weights would be "
             f"{bf16_b / 1e6:.1f} MB |", "",
             f"Raw: FETCH_SIZE {fetch_kib:.1f} KiB, WRITE_SIZE {write_kib:.1f} KiB per dispatch.", ""]
    with open(os.path.join(REPO, "profiles", "df11_gemm_batch_kernel_llama3_8b_block_t1_traffic.md"), "w") as f:
        f.write("\n".join(lines))


def integration(args, dev) -> int:
    """Forward of a synthetic model of Llama-3-8B-shaped blocks: resident BF16
    weights, DF11 blocks decoded in line before each block, DF11 blocks
    decoded on a side stream (capped grid) while the previous block computes,
    and, at 1..8 tokens, DF11 blocks (a stream per weight) whose projections
    decode inside their products (runtime.fused_block_forward); at up to 16
    tokens also the resident, in-line and fused forwards captured into HIP
    graphs and replayed."""
    import torch
    from entropy_decoding_df11_amd import df11, runtime, workloads
    blocks, resident, per_weight, tiled = [], [], [], []
    t0 = time.perf_counter()
    for b in range(args.blocks):
        flat, views = workloads.gen_block(seed=1000 + b)
        parts = [(nm, flat[o:o + r * c].reshape(r, c)) for nm, o, (r, c) in views]
        blocks.append(df11.compress_block(parts, device=dev))
        per_weight.append(df11.compress_block(parts, device=dev, codebook="per_weight"))
        tiled.append(df11.compress_block(parts, device=dev, codebook="per_weight", layout="mfma_tiles"))
        resident.append({nm: torch.from_numpy(a.astype(np.int16)).to(dev).view(torch.bfloat16) for nm, a in parts})
    t_prep = time.perf_counter() - t0
    overlap = runtime.BlockDecoder(blocks, device=dev, overlap=True, decode_workgroups=args.overlap_workgroups)
    inline = runtime.BlockDecoder(blocks, device=dev, overlap=False)
    rows = []

    def fused_forward(x):
        for blk in per_weight:
            x = runtime.fused_block_forward(x, blk)
        return x

    def tiled_forward(x):
        for blk in tiled:
            x = runtime.fused_block_forward(x, blk)
        return x

    for tokens in (1, 2, 4, 8, 16, 256, 4096):
        rng = np.random.default_rng(tokens)
        x = workloads.f32_to_bf16_bits(rng.standard_normal(tokens * 4096) * 0.5).reshape(tokens, 4096)
        x = torch.from_numpy(x.astype(np.int16)).to(dev).view(torch.bfloat16)
        res = {}
        ref = None
        for name, src in (("resident", resident), ("df11_overlap", overlap), ("df11_inline", inline)):
            for _ in range(3):
                y = runtime.model_forward(x, src)
            torch.cuda.synchronize()
            if ref is None:
                ref = y
            elif not torch.equal(y.view(torch.int16), ref.view(torch.int16)):
                print(f"integration: {name} output differs from resident weights", file=sys.stderr)
                return 1
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                runtime.model_forward(x, src)
            e1.record()
            torch.cuda.synchronize()
            res[name] = round(e0.elapsed_time(e1) / 10, 4)
        row = {"tokens": tokens, "ms_per_forward": res,
               "df11_overlap_vs_resident": round(res["df11_overlap"] / res["resident"], 3),
               "df11_inline_vs_resident": round(res["df11_inline"] / res["resident"], 3)}
        for name, fwd, limit in (("df11_fused", fused_forward, 8), ("df11_fused_tiles", tiled_forward, 256)):
            if tokens > limit:
                continue
            for _ in range(3):
                y = fwd(x)
            torch.cuda.synchronize()
            # float32 sums in another order: close to, not equal to, the resident forward
            dev_max = float((y.float() - ref.float()).abs().max())
            if dev_max > 0.05 * float(ref.float().abs().max()):
                print(f"integration: the {name} forward is far from the resident-weight forward", file=sys.stderr)
                return 1
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                fwd(x)
            e1.record()
            torch.cuda.synchronize()
            res[name] = round(e0.elapsed_time(e1) / 10, 4)
            row[f"{name}_vs_resident"] = round(res[name] / res["resident"], 3)
            row[f"{name}_max_abs_diff_over_max_abs"] = round(dev_max / float(ref.float().abs().max()), 5)
        if tokens <= 16:
            # The same forwards captured into HIP graphs (runtime.CapturedForward):
            # at a few tokens a forward is many small launches.
            graphs = {"resident_graph": lambda x: runtime.model_forward(x, resident),
                      "df11_inline_graph": lambda x: runtime.model_forward(x, inline)}
            if tokens <= 8:
                graphs["df11_fused_graph"] = fused_forward
            graphs["df11_fused_tiles_graph"] = tiled_forward
            for name, fwd in graphs.items():
                g = runtime.CapturedForward(fwd, x)
                y = g(x)
                torch.cuda.synchronize()
                if name.startswith("df11_fused"):
                    ok = float((y.float() - ref.float()).abs().max()) <= 0.05 * float(ref.float().abs().max())
                else:
                    ok = torch.equal(y.view(torch.int16), ref.view(torch.int16))
                if not ok:
                    print(f"integration: the {name} replay differs from the resident-weight forward", file=sys.stderr)
                    return 1
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(10):
                    g(x)
                e1.record()
                torch.cuda.synchronize()
                res[name] = round(e0.elapsed_time(e1) / 10, 4)
                del g
            row["df11_inline_graph_vs_resident_graph"] = round(res["df11_inline_graph"] / res["resident_graph"], 3)
            if tokens <= 8:
                row["df11_fused_graph_vs_resident_graph"] = round(res["df11_fused_graph"] / res["resident_graph"], 3)
            row["df11_fused_tiles_graph_vs_resident_graph"] = round(res["df11_fused_tiles_graph"]
                                                                   / res["resident_graph"], 3)
        rows.append(row)
    comp = sum(b.tensor.compressed_bytes() for b in blocks)
    raw = sum(2 * b.n_elements for b in blocks)
    print(json.dumps({"integration": "synthetic model forward", "blocks": args.blocks,
                      "weights_per_block": int(blocks[0].n_elements),
                      "overlap_decode_workgroups": args.overlap_workgroups, "compressed_over_bf16": round(comp / raw, 4),
                      "outputs": "in line and overlapped: bit-identical to the resident-weight forward; fused "
                                 "(row-order product up to 8 tokens, matrix-core product on tile-ordered weights up "
                                 "to 64): float32 sums in another order; the tile-ordered forward at 256 tokens "
                                 "decodes each block and runs the resident GEMMs (runtime.FUSED_MAX_TOKENS_TILES)",
                      "host_prep_s": round(t_prep, 1),
                      "results": rows}), flush=True)
    return 0


def linear_bench(args, dev) -> int:
    """One step = y = x W^T for each of the seven Llama-3-8B block matrices
    (each its own DF11 stream) at --linear-tokens tokens, with the decode
    fused into the product (df11_linear), compressed weights resident in HBM.
    value = compressed bytes + x + y per step / wall time; the roofline uses
    the fused kernels' own durations (dispatch events, in a second pass of
    the same steps).  The same run times resident BF16
    weights (torch F.linear) and decode-then-F.linear for comparison."""
    import torch
    import torch.nn.functional as F
    from entropy_decoding_df11_amd import df11, workloads
    T = args.linear_tokens
    stream = torch.cuda.current_stream(dev)
    t0 = time.perf_counter()
    flat, views = workloads.gen_block()
    mats = []
    for nm, o, (r, c) in views:
        w = np.ascontiguousarray(flat[o:o + r * c])
        t = df11.compress(w, shape=(r, c), device=dev, decode_table_bits=args.decode_table_bits)
        wd = torch.from_numpy(w.view(np.int16)).to(dev).view(torch.bfloat16).reshape(r, c)
        rng = np.random.default_rng(r * 7 + c)
        xb = workloads.f32_to_bf16_bits(rng.standard_normal(T * c) * 0.5).reshape(T, c)
        x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
        y = torch.empty((T, r), dtype=torch.float32, device=dev)
        mats.append((nm, r, c, t, wd, x, y))
    t_prep = time.perf_counter() - t0
    n = int(flat.size)
    comp = sum(m[3].compressed_bytes() for m in mats)
    algo_bytes = comp + sum(2 * T * m[2] + 4 * T * m[1] for m in mats)

    def step(evs=None):
        for i, (_, _, _, t, _, x, y) in enumerate(mats):
            t.linear(x, out=y, events=None if evs is None else evs[i])

    # Check every output against a float64 product of the same BF16 values,
    # within the float32 summation bound (each product exact, in_features
    # additions): |y - ref| <= 1.01 * in_features * 2^-24 * sum |x w|.
    step()
    torch.cuda.synchronize()
    for nm, r, c, t, wd, x, y in mats:
        ref = x.double() @ wd.double().T
        bound = 1.01 * c * 2.0 ** -24 * (x.double().abs() @ wd.double().abs().T)
        if not bool(((y.double() - ref).abs() <= bound).all()):
            print(f"bench: fused linear of {nm} is outside the float32 bound", file=sys.stderr)
            return 1
    del ref, bound

    # Timed steps (wall clock), then the same steps again with each fused
    # kernel's own start and end recorded (dispatch events), for the roofline.
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in mats]
           for _ in range(args.steps)]
    for e in (ev for row in evs for pair in row for ev in pair):
        e.record(stream)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    kern_ms = [sum(a.elapsed_time(b) for a, b in row) for row in evs]
    per_matrix_us = {m[0]: round(float(np.mean([evs[i][j][0].elapsed_time(evs[i][j][1])
                                                 for i in range(args.steps)])) * 1e3, 2)
                     for j, m in enumerate(mats)}
    mean_ms = float(np.mean(kern_ms))
    achieved = algo_bytes / (mean_ms * 1e-3) / 1e9

    def timed(fn, reps=50, windows=3):
        """ms per call of fn: the best of `windows` windows of `reps` calls.
        A window can take a one-off host stall (the first window of the
        batched products has measured 4x its steady state)."""
        for _ in range(10):
            fn()
        best = float("inf")
        for _ in range(windows):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b) / reps)
        return best

    scratch = torch.empty(max(m[1] * m[2] for m in mats), dtype=torch.bfloat16, device=dev)
    resident_ms = timed(lambda: [F.linear(m[5], m[4]) for m in mats])
    decode_gemm_ms = timed(lambda: [F.linear(m[5], m[3].decompress(out=scratch[:m[1] * m[2]].view(m[1], m[2])))
                                    for m in mats])
    fused_ms = timed(step)
    # As a forward issues them: q, k, v on one x in one launch, o, gate and
    # up on one x in one launch, down (df11_linear_batch).
    by = {m[0]: m for m in mats}

    def step_batched():
        df11.linear_batch([by[n][3] for n in ("q_proj", "k_proj", "v_proj")], by["q_proj"][5])
        by["o_proj"][3].linear(by["o_proj"][5], out=by["o_proj"][6])
        df11.linear_batch([by[n][3] for n in ("gate_proj", "up_proj")], by["gate_proj"][5])
        by["down_proj"][3].linear(by["down_proj"][5], out=by["down_proj"][6])

    batched_ms = timed(step_batched)
    result = {
        "metric": "DF11 decode fused into y = x W^T: GB/s of compressed weights + x + y per step",
        "value": round(args.steps * algo_bytes / wall / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama3_8b_block_linear",
            "tokens": T,
            "shapes": {m[0]: [m[1], m[2]] for m in mats},
            "streams": len(mats),
            "codebook": "per_weight",
            "n_elements": n,
            "compressed_bytes": comp,
            "decode_table_bits": args.decode_table_bits,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": None,
        },
        "kernel_ms_mean": round(mean_ms, 5),
        "per_matrix_us": per_matrix_us,
        "same_run_ms_per_step": {"fused_df11": round(fused_ms, 4),
                                 "fused_df11_qkv_and_gate_up_batched": round(batched_ms, 4),
                                 "resident_bf16_F_linear": round(resident_ms, 4),
                                 "decode_then_F_linear": round(decode_gemm_ms, 4)},
        "outputs": "within the float32 summation bound of a float64 product",
        "host_prep_s": round(t_prep, 1),
    }
    if not args.no_cpu_baseline:
        import oracle  # test infrastructure: the CPU baseline only
        nm, r, c, t, wd, x, y = mats[0]
        w = np.ascontiguousarray(flat[:r * c])
        s = oracle.encode(w)
        xb = x.view(torch.int16).cpu().numpy().view(np.uint16)
        c0 = time.perf_counter()
        reps = 0
        while True:
            oracle.linear(s, xb, r)
            reps += 1
            if time.perf_counter() - c0 > 10.0:
                break
        cpu_s = (time.perf_counter() - c0) / reps
        sample_bytes = (s["enc"].nbytes + s["sm"].nbytes + s["gaps"].nbytes + s["out_pos"].nbytes
                        + 2 * T * c + 4 * T * r)
        result["cpu_baseline"] = {
            "value": round(sample_bytes / cpu_s / 1e9, 4),
            "unit": "GB/s",
            "cores": 1,
            "kind": "oracle",
            "sample": f"{nm} ({r}x{c}) at {T} tokens: oracle tree-walk decode then a float64 matmul, "
                      f"{reps} run(s), {cpu_s:.2f} s each",
        }
    print(json.dumps(result), flush=True)
    return 0


MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak


def matmul_bench(args, dev) -> int:
    """One step = y = x W^T for each of the seven Llama-3-8B block matrices
    (each its own DF11 stream in MFMA tile order) at --matmul-tokens tokens,
    on the matrix cores with the decode fused in (df11_matmul), compressed
    weights resident in HBM.  The same run times resident BF16 weights
    (torch F.linear) and decode-then-F.linear.  The roofline is HBM-bound
    (compressed bytes + x + y per step over the step time) while the
    product's arithmetic intensity is under MI355X's flop:byte balance
    (2.5 PFLOP/s over 8 TB/s), matrix-core-bound (2 T flops per weight
    against 2.5 PFLOP/s) above it."""
    import torch
    import torch.nn.functional as F
    from entropy_decoding_df11_amd import df11, workloads
    T = args.matmul_tokens
    stream = torch.cuda.current_stream(dev)
    t0 = time.perf_counter()
    flat, views = workloads.gen_block()
    mats = []
    xs = {}
    for nm, o, (r, c) in views:
        w = np.ascontiguousarray(flat[o:o + r * c])
        t = df11.compress(w, shape=(r, c), device=dev, layout="mfma_tiles")
        wd = torch.from_numpy(w.view(np.int16)).to(dev).view(torch.bfloat16).reshape(r, c)
        if c not in xs:
            rng = np.random.default_rng(c)
            xb = workloads.f32_to_bf16_bits(rng.standard_normal(T * c) * 0.5).reshape(T, c)
            xs[c] = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
        y = torch.empty((T, r), dtype=torch.float32, device=dev)
        mats.append((nm, r, c, t, wd, xs[c], y))
    t_prep = time.perf_counter() - t0
    n = int(flat.size)
    del flat
    comp = sum(m[3].compressed_bytes() for m in mats)
    hbm_bytes = comp + sum(2 * T * m[2] + 4 * T * m[1] for m in mats)
    flops = 2.0 * T * n

    tensors, xlist, ylist = [m[3] for m in mats], [m[5] for m in mats], [m[6] for m in mats]

    def step():  # the seven products in one launch (df11_matmul_batch)
        df11.matmul_batch(tensors, xlist, outs=ylist)

    by = {m[0]: m for m in mats}

    # As runtime.fused_block_forward issues them: the seven outputs are views
    # of one buffer zeroed by one fill, then four accumulating launches (q, k,
    # v; o; gate, up; down).
    fwd_buf = torch.empty(sum(T * m[1] for m in mats), dtype=torch.float32, device=dev)
    fwd_y = dict(zip(by, torch.split(fwd_buf, [T * m[1] for m in mats])))

    def step_forward():
        fwd_buf.zero_()
        for group in (("q_proj", "k_proj", "v_proj"), ("o_proj",), ("gate_proj", "up_proj"), ("down_proj",)):
            df11.matmul_batch([by[g][3] for g in group], [by[g][5] for g in group],
                              outs=[fwd_y[g].view(T, by[g][1]) for g in group], accumulate=True)

    def step_seven():  # one launch per product
        for _, _, _, t, _, x, y in mats:
            t.matmul(x, out=y)

    # Every output against a float64 product of the same BF16 values, within
    # the float32 summation bound: |y - ref| <= 1.01 * in_features * 2^-24 * sum |x w|.
    step()
    torch.cuda.synchronize()
    for nm, r, c, t, wd, x, y in mats:
        rows = torch.arange(0, T, max(1, T // 64), device=dev)  # every token up to 64, a sample above
        xd = x[rows].double()
        ref = xd @ wd.double().T
        bound = 1.01 * c * 2.0 ** -24 * (xd.abs() @ wd.double().abs().T)
        if not bool(((y[rows].double() - ref).abs() <= bound).all()):
            print(f"bench: matmul of {nm} is outside the float32 bound", file=sys.stderr)
            return 1
    del ref, bound, xd

    def timed(fn, reps):
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps, (time.perf_counter() - w0) * 1e3 / reps

    # Settle the clocks as the decode line does (the first launches of a
    # process run slow), then the warmup steps.
    settle = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < SETTLE_S:
        step()
        settle += 1
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    fused_ms, wall_ms = timed(step, args.steps)
    forward_ms, _ = timed(step_forward, max(3, args.steps // 2))
    seven_ms, _ = timed(step_seven, max(3, args.steps // 2))
    scratch = torch.empty(max(m[1] * m[2] for m in mats), dtype=torch.bfloat16, device=dev)
    resident_ms, _ = timed(lambda: [F.linear(m[5], m[4]) for m in mats], max(3, args.steps // 2))
    decode_gemm_ms, _ = timed(lambda: [F.linear(m[5], m[3].decompress(out=scratch[:m[1] * m[2]].view(m[1], m[2])))
                                       for m in mats], max(3, args.steps // 2))

    # The forward's launches and the resident products captured into HIP
    # graphs and replayed: the kernels alone, without the host issuing them.
    def captured(fn):
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for _ in range(2):
                fn()
        stream.wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            out = fn()
        return g, out

    step_forward()
    torch.cuda.synchronize()
    eager_forward = fwd_buf.clone()
    g_forward, _ = captured(step_forward)
    g_resident, resident_outs = captured(lambda: [F.linear(m[5], m[4]) for m in mats])
    forward_graph_ms, _ = timed(g_forward.replay, max(3, args.steps // 2))
    resident_graph_ms, _ = timed(g_resident.replay, max(3, args.steps // 2))
    # the last replays against the eager results (float32 sums in another order for the fused products)
    torch.cuda.synchronize()
    scale = float(eager_forward.abs().max())
    resident_far = any(float((o.float() - F.linear(m[5], m[4]).float()).abs().max())
                       > 1e-2 * float(o.float().abs().max()) for o, m in zip(resident_outs, mats))
    if float((fwd_buf - eager_forward).abs().max()) > 1e-4 * scale or resident_far:
        print("bench: a graph replay differs from the eager products", file=sys.stderr)
        return 1
    del g_forward, g_resident, resident_outs, eager_forward
    intensity = flops / hbm_bytes
    compute_bound = intensity > MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    tflops = flops / (fused_ms * 1e-3) / 1e12
    gbps = hbm_bytes / (fused_ms * 1e-3) / 1e9
    roof = ({"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": round(tflops / MFMA_PEAK_TFLOPS, 4), "traffic": None} if compute_bound else
            {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
             "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None})
    result = {
        "metric": "DF11 decode fused into y = x W^T on the matrix cores: "
                  + ("TFLOP/s" if compute_bound else "GB/s of compressed weights + x + y"),
        "value": round(tflops if compute_bound else hbm_bytes / (wall_ms * 1e-3) / 1e9, 2),
        "unit": "TFLOP/s" if compute_bound else "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3_8b_block_matmul", "tokens": T,
                   "shapes": {m[0]: [m[1], m[2]] for m in mats}, "streams": len(mats), "codebook": "per_weight",
                   "layout": "mfma_tiles", "n_elements": n, "compressed_bytes": comp},
        "roofline": roof,
        "kernel_ms": round(fused_ms, 5),
        "kernel_ms_note": "HIP events around the timed steps / steps: one zeroing kernel and one batched fused "
                          "kernel for the seven products",
        "arithmetic_intensity_flop_per_byte": round(intensity, 2),
        "achieved_tflops": round(tflops, 2),
        "achieved_hbm_gbps": round(gbps, 1),
        "same_run_ms_per_step": {"fused_df11_matmul": round(fused_ms, 4),
                                 "fused_df11_matmul_as_a_forward_issues_it": round(forward_ms, 4),
                                 "fused_df11_matmul_seven_launches": round(seven_ms, 4),
                                 "resident_bf16_F_linear": round(resident_ms, 4),
                                 "decode_then_F_linear": round(decode_gemm_ms, 4),
                                 "fused_df11_matmul_as_a_forward_issues_it_graph": round(forward_graph_ms, 4),
                                 "resident_bf16_F_linear_graph": round(resident_graph_ms, 4)},
        "outputs": "within the float32 summation bound of a float64 product (every token up to 64, a sample above)",
        # launches of the batched fused kernel with all seven products, in order (then the forward's
        # four batches per step, then single-product kernels)
        "launches": {"check": 1, "settle": settle, "warmup": args.warmup + 3, "timed": args.steps},
        "host_prep_s": round(t_prep, 1),
    }
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # The GPU's clocks take some tens of milliseconds of sustained load to
    # settle: after 100 launches (~15 ms) the decode is within ~1.5% of its
    # steady state, after 300 (~40 ms) within noise (1000 measure the same).
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--decode-table-bits", type=int, default=11)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=WORKLOAD_CHOICES,
                    help="the Llama-3-8B block (default), the same with a codebook per weight (one batched "
                         "launch), or one of the single-stream workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layout", choices=["rows", "mfma_tiles"], default="rows",
                    help="element order of each weight (llama3_8b_block_per_weight): its own, or the matrix-core "
                         "product's tile order (decompressed back to row-major)")
    ap.add_argument("--no-decode-table", action="store_true",
                    help="launch with the page's arrays alone: every workgroup derives the first-level decode "
                         "table in LDS from the LUTs and CodeLengths")
    ap.add_argument("--cpu-threads", type=int, default=0, help="oracle threads (default: usable host cores)")
    ap.add_argument("--integration", action="store_true",
                    help="instead of the decode line, time a synthetic model forward over full-size blocks with "
                         "resident BF16 weights, with DF11 blocks decoded on a side stream just before use, and "
                         "with DF11 blocks decoded in line")
    ap.add_argument("--blocks", type=int, default=4, help="blocks of the --integration model")
    ap.add_argument("--overlap-workgroups", type=int, default=512,
                    help="workgroup cap of the side-stream decode in --integration (0: no cap)")
    ap.add_argument("--coder", choices=["huffman", "rans"], default="huffman",
                    help="entropy coder of the exponents: the page's Huffman format, or the rANS alternative")
    ap.add_argument("--linear-tokens", type=int, default=0,
                    help="time the decode fused into y = x W^T over the block's seven matrices at this many "
                         "tokens (1..8) instead of the decompression")
    ap.add_argument("--matmul-tokens", type=int, default=0,
                    help="time the decode fused into y = x W^T on the matrix cores (weights in MFMA tile order) "
                         "over the block's seven matrices at this many tokens, against resident BF16 and "
                         "decode-then-F.linear")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write the profiles/ summaries from rocprofv3 runs of this script under DIR, then exit")
    args = ap.parse_args()

    if args.summarize_profiles:
        pre = "cd /tmp && export TMPDIR=/tmp && "   # R = repository root, D = a directory for the raw results
        have = lambda sub: os.path.isdir(os.path.join(args.summarize_profiles, sub))
        trace = pre + "rocprofv3 --kernel-trace --stats -d $D/{sub} -o run --output-format csv -- python3 " \
                      "$R/bench.py {args} > $D/{sub}.json"
        if have("trace"):
            summarize_decode_trace(args.summarize_profiles, "trace", "df11_decode_kernel",
                                   "df11_decode_kernel on llama3_8b_block",
                                   trace.format(sub="trace", args="--gpus 1 --steps 20 --warmup 5"),
                                   "df11_decode_kernel_llama3_8b_block_trace.md")
        if have("fetch") and have("write"):
            pmc = pre + "rocprofv3 --pmc {c} -d $D/{sub} -o run --output-format csv -- python3 $R/bench.py " \
                        "--steps 3 --warmup 2 --no-cpu-baseline"
            summarize_traffic(args.summarize_profiles, {
                "fetch": pmc.format(c="FETCH_SIZE", sub="fetch") + " > $D/fetch.json",
                "write": pmc.format(c="WRITE_SIZE", sub="write")})
        if have("lin_trace"):
            summarize_linear_profile(args.summarize_profiles,
                                     pre + "rocprofv3 --kernel-trace --stats -d $D/lin_trace -o run --output-format csv "
                                           "-- python3 $R/bench.py --linear-tokens 1 --steps 50 --warmup 20 "
                                           "--no-cpu-baseline > $D/lin.json")
        for T in (1, 16, 64, 256):
            if have(f"mm{T}"):
                summarize_matmul_profile(args.summarize_profiles, f"mm{T}",
                                         trace.format(sub=f"mm{T}", args=f"--matmul-tokens {T} --steps 20 --warmup 5"))
        if have("pw_tiles_trace"):
            summarize_decode_trace(args.summarize_profiles, "pw_tiles_trace", "df11_decode_pairs_batch_kernel",
                                   "df11_decode_pairs_batch_kernel on llama3_8b_block_per_weight (MFMA tile order "
                                   "back to row-major)",
                                   trace.format(sub="pw_tiles_trace",
                                                args="--workload llama3_8b_block_per_weight --layout mfma_tiles "
                                                     "--steps 20 --warmup 5 --no-cpu-baseline"),
                                   "df11_decode_pairs_batch_kernel_llama3_8b_block_per_weight_tiles_trace.md")
        if have("rans_trace"):
            summarize_decode_trace(args.summarize_profiles, "rans_trace", "df11_rans_decode",
                                   "df11_rans_decode_kernel on llama3_8b_block (rANS coder)",
                                   trace.format(sub="rans_trace", args="--coder rans --steps 20 --warmup 5 "
                                                                      "--no-cpu-baseline"),
                                   "df11_rans_decode_kernel_llama3_8b_block_trace.md")
        counter_runs = [("df11_decode_kernel", "df11_decode_kernel on llama3_8b_block",
                         "--steps 3 --warmup 2 --no-cpu-baseline", "entropy_decoding_df11_amd/csrc/df11_decode.hip",
                         "df11_decode_kernel_llama3_8b_block_counters.md"),
                        ("df11_decode_pairs_batch_kernel",
                         "df11_decode_pairs_batch_kernel on llama3_8b_block_per_weight (MFMA tile order back to "
                         "row-major)",
                         "--workload llama3_8b_block_per_weight --layout mfma_tiles --steps 3 --warmup 2 "
                         "--no-cpu-baseline", "entropy_decoding_df11_amd/csrc/df11_decode.hip",
                         "df11_decode_pairs_batch_kernel_llama3_8b_block_per_weight_tiles_counters.md"),
                        ("df11_decode_batch_kernel", "df11_decode_batch_kernel on llama3_8b_block_per_weight (row order)",
                         "--workload llama3_8b_block_per_weight --steps 3 --warmup 2 --no-cpu-baseline",
                         "entropy_decoding_df11_amd/csrc/df11_decode.hip",
                         "df11_decode_batch_kernel_llama3_8b_block_per_weight_counters.md"),
                        ("df11_rans_decode_kernel", "df11_rans_decode_kernel on llama3_8b_block (rANS coder)",
                         "--coder rans --steps 3 --warmup 2 --no-cpu-baseline",
                         "entropy_decoding_df11_amd/csrc/df11_rans_decode.hip",
                         "df11_rans_decode_kernel_llama3_8b_block_counters.md")]
        for kernel, title, bench_args, source, out_name in counter_runs:
            if all(have(f"{kernel}_{sub}") for sub in COUNTER_PASSES):
                summarize_counters(args.summarize_profiles, kernel, title, bench_args, source, out_name)
        if have("mm_fetch") and have("mm_write"):
            summarize_product_traffic(args.summarize_profiles)
        if all(have(f"{k}_{sub}") for k in ("df11_linear_kernel", "df11_gemm_batch_kernel") for sub in COUNTER_PASSES) \
                and os.path.exists(os.path.join(args.summarize_profiles, "mm_pmc.json")):
            summarize_product_counters(args.summarize_profiles)
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: DF11 decoding needs no exchange between GPUs, and every "
              "GPU would decode its own streams; run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    from entropy_decoding_df11_amd import df11, workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if args.integration:
        return integration(args, dev)
    if args.linear_tokens:
        return linear_bench(args, dev)
    if args.matmul_tokens:
        return matmul_bench(args, dev)
    wl = args.workload
    t0 = time.perf_counter()
    if wl.startswith("llama3_8b_block"):
        flat, views = workloads.gen_block()
    else:
        flat, views = workloads.make(wl), None
    t_gen = time.perf_counter() - t0
    n = int(flat.size)
    t0 = time.perf_counter()
    config = {"workload": wl}
    if args.coder == "rans":
        if wl.endswith("_per_weight"):
            print("bench: the rANS coder takes the block as one stream (llama3_8b_block)", file=sys.stderr)
            return 2
        first = df11.rans_compress(flat, shape=(n,), device=dev)
        h, comp = first.header, first.compressed_bytes()
        config["coder"] = "rans"
        config["rans"] = {"prob_bits": int(h.prob_bits), "lanes": int(h.lanes), "steps": int(h.steps),
                          "segments": int(h.n_segments), "words": int(h.n_words)}
        out_elems = n
    elif views is not None:
        codebook = "per_weight" if wl.endswith("_per_weight") else "shared"
        first = df11.compress_block([(nm, flat[o:o + r * c].reshape(r, c)) for nm, o, (r, c) in views], device=dev,
                                    decode_table_bits=args.decode_table_bits, codebook=codebook,
                                    layout=args.layout)
        if args.layout != "rows":
            config["layout"] = args.layout
        config["shapes"] = {name: list(shape) for name, _, shape in views}
        config["codebook"] = codebook
        if codebook == "shared":
            h, comp = first.tensor.header, first.tensor.compressed_bytes()
        else:
            h, comp = first.tensors[0].header, first.compressed_bytes()
            config["streams"] = len(first.tensors)
        out_elems = first.n_elements
    else:
        first = df11.compress(flat, shape=(n,), device=dev, decode_table_bits=args.decode_table_bits)
        h, comp = first.header, first.compressed_bytes()
        out_elems = n
    t_enc = time.perf_counter() - t0
    algo_bytes = comp + 2 * n
    if args.no_decode_table and args.coder == "huffman":
        for t in ([first] if views is None else [first.tensor] if codebook == "shared" else first.tensors):
            t.use_decode_table(False)
        config["decode_table"] = "derived in LDS by every workgroup"

    # Copies of the compressed stream in other device buffers, each with an
    # output of its own.  Step i decodes copy i mod R; between two uses of a
    # copy the others move at least 768 MiB (three times the 256 MB MALL), so
    # every step finds its stream and output in neither the L2 nor the MALL,
    # as a model that decodes each block once per forward does.
    rotate = min(256, 1 + -(-(768 << 20) // algo_bytes))
    copies = [first] + [first.clone() for _ in range(rotate - 1)]
    outs = [torch.empty(out_elems, dtype=torch.bfloat16, device=dev) for _ in copies]

    def decoder(obj, out):
        if args.coder == "rans" or views is None:
            return lambda: obj.decompress(out=out)
        return lambda: obj.decompress(scratch=out)

    decoders = [decoder(c, o) for c, o in zip(copies, outs)]
    # The first launch of every copy; a block's decode returns its per-weight
    # views, which follow the original data's order.
    firsts = [d() for d in decoders]
    parts = [[v.reshape(-1) for v in f.values()] if isinstance(f, dict) else [f.reshape(-1)] for f in firsts]
    torch.cuda.synchronize()

    def check(i):
        got = torch.cat(parts[i]).view(torch.int16).cpu().numpy().view(np.uint16)
        return np.array_equal(got, flat)

    if not all(check(i) for i in range(rotate)):
        print(f"bench: decoded {wl} differs from the original weights", file=sys.stderr)
        return 1

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # The GPU's clocks need some tens of milliseconds of sustained load to
    # settle (the first ~60 block launches run 5-15% slow): before the
    # warmup steps, decode for SETTLE_S seconds, so that the measurement is
    # the steady state whatever the warmup count.
    settle = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(rotate):
            decoders[settle % rotate]()
            settle += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        decoders[i % rotate]()
    torch.cuda.synchronize()

    # Timed steps: K launches over the rotating copies, bracketed by a pair
    # of HIP events on the launch stream (the kernel time per launch, gaps
    # between launches included) and by the host clock (the whole-job time).
    e0, e1 = ev(), ev()
    wall0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        decoders[i % rotate]()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    kern_ms = e0.elapsed_time(e1) / args.steps
    achieved = algo_bytes / (kern_ms * 1e-3) / 1e9
    value = args.steps * algo_bytes / wall / 1e9

    # Hot caches, for comparison: the same copy decoded back to back, so
    # whatever of it the L2 and the MALL keep serves the next launch.
    for _ in range(5):
        decoders[0]()
    h0, h1 = ev(), ev()
    h0.record(stream)
    for _ in range(args.steps):
        decoders[0]()
    h1.record(stream)
    torch.cuda.synchronize()
    hot_ms = h0.elapsed_time(h1) / args.steps

    # The flushed-cache recipe: FLUSHED_LAUNCHES launches, each after reading
    # 1 GiB (so that neither the L2 nor the MALL holds the stream), each
    # timed by events recorded around it (so the time includes the launch's
    # dispatch); the median.  The flush reads rather than writes: written
    # lines would be dirty, and the timed launch would pay for their write-back.
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    flushed = [(ev(), ev()) for _ in range(FLUSHED_LAUNCHES)]
    for a, b in flushed:
        torch.sum(flush, dim=0, out=sink)
        a.record(stream)
        decoders[0]()
        b.record(stream)
    torch.cuda.synchronize()
    flushed_ms = float(np.median([a.elapsed_time(b) for a, b in flushed]))
    del flush

    # Verification round: every output overwritten with a pattern, one more
    # rotation of launches, every copy compared with the original weights.
    for o in outs:
        o.view(torch.int16).fill_(0x5A5A)
    for d in decoders:
        d()
    torch.cuda.synchronize()
    if not all(check(i) for i in range(rotate)):
        print(f"bench: the repeated launches decoded {wl} wrongly", file=sys.stderr)
        return 1

    # A plain copy kernel over the same byte count, as the achievable-bandwidth reference.
    src = torch.empty(algo_bytes // 2, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    c0, c1 = ev(), ev()
    c0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 10 * 2 * src.numel() / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    traffic = _traffic_from_profile() if wl == DEFAULT_WORKLOAD and args.coder == "huffman" else None
    gbps = lambda ms: round(algo_bytes / (ms * 1e-3) / 1e9, 1)  # noqa: E731
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {
            **config,
            "n_elements": n,
            "bits_per_weight": round(8 * comp / n, 4),
            "compressed_bytes": comp,
            **({"decode_table_bits": args.decode_table_bits, "max_code_len": int(h.max_len),
                "n_luts": int(h.n_luts)} if args.coder == "huffman" else {}),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
        },
        "kernel_ms": round(kern_ms, 5),
        "cache": f"value and roofline: each step decodes the next of {rotate} copies of the stream (each with its "
                 "own output), so no step finds its data in the L2 or the 256 MB MALL; kernel_ms = HIP events "
                 "around the timed steps / steps (launch gaps included)",
        "hot_kernel_ms": round(hot_ms, 5),
        "hot": f"one copy decoded back to back ({args.steps} launches, events around them): whatever of the "
               f"stream the caches keep serves the next launch; {gbps(hot_ms)} GB/s",
        "flushed_kernel_ms_median": round(flushed_ms, 5),
        "flushed": f"median of {FLUSHED_LAUNCHES} launches, each after a 1 GiB read and between events recorded "
                   f"around it (its dispatch included); {gbps(flushed_ms)} GB/s",
        "launches": {"check": rotate, "settle": settle, "warmup": args.warmup, "timed": args.steps,
                     "hot": args.steps + 5, "flushed": FLUSHED_LAUNCHES, "verify": rotate},
        "rotation_copies": rotate,
        "copy_kernel_GBps": round(copy_gbps, 1),
        "frac_of_copy": round(achieved / copy_gbps, 4),
        "host_gen_s": round(t_gen, 2),
        "host_encode_s": round(t_enc, 2),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _cpu_baselines(flat, args)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
