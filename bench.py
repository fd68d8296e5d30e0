"""DF11 decompression throughput on one MI355X.

One step = one batched decompression of the Llama-3-8B-shaped transformer block
(q, k, v, o, gate, up, down; one DF11 stream, shared codebook, ~218M BF16
weights) into one scratch buffer, with the compressed stream already resident
in HBM.  Prints one JSON line.  --workload picks another input: the same block
with a codebook per weight (seven streams, one batched launch), or a single
stream (LM-head-sized 128256x4096, the 2^28 stress stream, ...).

  value     = K * (algorithmic bytes per step) / (wall time of K back-to-back
              launches), GB/s
  algorithmic bytes per step = EncodedExponent + PackedSignMantissa + Gaps
              + output positions + LUTs + CodeLengths (all unpadded) read,
              plus 2 bytes per BF16 weight written
  roofline  = the same bytes / the decode kernel's mean duration over K more
              launches (a pair of HIP events per launch that the kernel
              dispatch itself records on its stream, hipExtLaunchKernel)
              against the 8 TB/s HBM peak;
              kernel_ms_cold_median times 20 more launches, each after a 1 GiB
              read that flushes the L2 and the MALL
  cpu_baseline = the CPU oracle's tree-walk decoder, group-parallel over the
              host's cores, on the same workload
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

REPO = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, REPO)

HBM_PEAK_GBPS = 8000.0
COLD_LAUNCHES = 20  # cold-cache launches after the timed ones
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


def _cpu_baseline(flat: np.ndarray, threads: int):
    import oracle
    s = oracle.encode(flat)
    out = np.zeros_like(flat)
    t0 = time.perf_counter()
    oracle.decode_groups_parallel(s, 0, s["n_groups"], out, threads)
    dt = time.perf_counter() - t0
    ok = bool(np.array_equal(out, flat))
    algo = (s["total_bits"] + 7) // 8 + s["n_elements"] + (5 * s["n_threads"] + 7) // 8 \
        + 4 * (s["n_groups"] + 1) + 256 * (s["n_luts"] + 1) + 2 * s["n_elements"]
    return algo / dt / 1e9, dt, ok


def _cpu_baseline_rans(flat: np.ndarray):
    """The oracle's rANS decoder (one host thread) on the whole stream."""
    import oracle
    s = oracle.rans_encode(flat)
    t0 = time.perf_counter()
    out = oracle.rans_decode(s)
    dt = time.perf_counter() - t0
    algo = oracle.rans_compressed_bytes(s) + 2 * s["n_elements"]
    return algo / dt / 1e9, dt, bool(np.array_equal(out, flat))


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


def summarize_profiles(prof_dir: str, commands: dict) -> None:
    """Turn the rocprofv3 output of one kernel-trace run and two PMC runs of this
    script into the committed summaries under profiles/.

    prof_dir holds trace/ (--kernel-trace --stats), fetch/ (--pmc FETCH_SIZE),
    write/ (--pmc WRITE_SIZE) and bench.json (the JSON line of the trace run).
    FETCH_SIZE and WRITE_SIZE are KiB per dispatch.  Each is scaled by the ratio
    of known bytes to counted bytes of the plain copy kernel the same run
    launches (10 copies of a buffer of known size)."""
    stats = _read_csv(os.path.join(prof_dir, "trace", "run_kernel_stats.csv"))
    with open(os.path.join(prof_dir, "bench.json")) as f:
        bench = json.loads(f.read().strip().splitlines()[-1])
    trace = [r for r in _read_csv(os.path.join(prof_dir, "trace", "run_kernel_trace.csv"))
             if "df11_decode" in r["Kernel_Name"]]
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    timed = trace[-(bench["steps"] + COLD_LAUNCHES):-COLD_LAUNCHES]
    timed_us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in timed]
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
    kib = lambda xs: float(np.median(xs))
    fetch_scale = copy_bytes / (kib(fetch_cpy) * 1024)
    write_scale = copy_bytes / (kib(write_cpy) * 1024)
    read_b = kib(fetch_dec) * 1024 * fetch_scale
    write_b = kib(write_dec) * 1024 * write_scale

    dec_row = [r for r in stats if "df11_decode" in r["Name"]]
    lines = ["# df11_decode_kernel on llama3_8b_block: rocprofv3 kernel trace", "",
             "Command (from the repository root on a one-GPU MI355X box):", "",
             "    " + commands["trace"], "",
             "| kernel | calls | average us | min us | max us | share of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in stats[:6]:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {r['Percentage']}% |")
    avg_all = float(dec_row[0]["AverageNs"]) / 1e3
    avg_us = float(np.mean(timed_us))
    lines += ["", f"The table averages every decode launch of the run, warmup included ({avg_all:.2f} us).  "
              f"Over the {len(timed_us)} timed launches (those before the last {COLD_LAUNCHES}, which run after a "
              f"cache flush) the decode kernel averages "
              f"{avg_us:.2f} us (min {min(timed_us):.2f}, max {max(timed_us):.2f}) for {algo} algorithmic bytes: "
              f"{algo / (avg_us * 1e-6) / 1e9:.1f} GB/s, {algo / (avg_us * 1e-6) / 1e9 / HBM_PEAK_GBPS:.3f} of 8 TB/s.  "
              f"The same run's bench line measured {bench['kernel_ms_mean'] * 1e3:.2f} us per launch with the events "
              f"that the kernel dispatch records (df11_decompress_timed).", "",
             "Bench line of the traced run:", "", "    " + json.dumps(bench), ""]
    os.makedirs(os.path.dirname(PMC_SUMMARY), exist_ok=True)
    with open(os.path.join(os.path.dirname(PMC_SUMMARY), "df11_decode_kernel_llama3_8b_block_trace.md"), "w") as f:
        f.write("\n".join(lines))
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
             "Command (from the repository root on a one-GPU MI355X box):", "", "    " + command, "",
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


def summarize_kernel_trace(prof_dir: str, sub: str, kernel: str, title: str, command: str, out_name: str) -> None:
    """profiles/ summary of a rocprofv3 --kernel-trace --stats run of this
    script (prof_dir/sub, its bench line in prof_dir/sub.json): the stats
    table and the kernel's average over the run's timed launches (the
    `steps` launches of `kernel` before the cold-cache ones) against the
    bench line's event timing."""
    with open(os.path.join(prof_dir, sub + ".json")) as f:
        bench = json.loads(f.read().strip().splitlines()[-1])
    stats = _read_csv(os.path.join(prof_dir, sub, "run_kernel_stats.csv"))
    rows = [r for r in _read_csv(os.path.join(prof_dir, sub, "run_kernel_trace.csv")) if kernel in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    timed = rows[-(bench["steps"] + COLD_LAUNCHES):-COLD_LAUNCHES]
    timed_us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in timed]
    algo = bench["config"]["compressed_bytes"] + 2 * bench["config"]["n_elements"]
    avg = float(np.mean(timed_us))
    lines = [f"# {title}: rocprofv3 kernel trace", "", "Command (from the repository root on a one-GPU MI355X box):",
             "", "    " + command, "", "| kernel | calls | average us | min us | max us | share of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in stats[:6]:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {r['Percentage']}% |")
    lines += ["", f"Over the {len(timed_us)} timed launches (those before the last {COLD_LAUNCHES}, which run "
              f"after a cache flush) the kernel averages "
              f"{avg:.2f} us (min {min(timed_us):.2f}, max {max(timed_us):.2f}) for {algo} algorithmic bytes: "
              f"{algo / (avg * 1e-6) / 1e9:.1f} GB/s, {algo / (avg * 1e-6) / 1e9 / HBM_PEAK_GBPS:.3f} of 8 TB/s.  "
              f"The bench line measured {bench['kernel_ms_mean'] * 1e3:.2f} us per launch with the events that "
              f"the kernel dispatch records.", "", "Bench line of the traced run:", "", "    " + json.dumps(bench), ""]
    with open(os.path.join(REPO, "profiles", out_name), "w") as f:
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
             "one-GPU MI355X box; R = repository root, D = R/gpurun_out/prof):", ""]
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
    blocks, resident, per_weight = [], [], []
    t0 = time.perf_counter()
    for b in range(args.blocks):
        flat, views = workloads.gen_block(seed=1000 + b)
        parts = [(nm, flat[o:o + r * c].reshape(r, c)) for nm, o, (r, c) in views]
        blocks.append(df11.compress_block(parts, device=dev))
        per_weight.append(df11.compress_block(parts, device=dev, codebook="per_weight"))
        resident.append({nm: torch.from_numpy(a.astype(np.int16)).to(dev).view(torch.bfloat16) for nm, a in parts})
    t_prep = time.perf_counter() - t0
    overlap = runtime.BlockDecoder(blocks, device=dev, overlap=True, decode_workgroups=args.overlap_workgroups)
    inline = runtime.BlockDecoder(blocks, device=dev, overlap=False)
    rows = []

    def fused_forward(x):
        for blk in per_weight:
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
        if tokens <= 8:
            for _ in range(3):
                y = fused_forward(x)
            torch.cuda.synchronize()
            # float32 sums in another order: close to, not equal to, the resident forward
            dev_max = float((y.float() - ref.float()).abs().max())
            if dev_max > 0.05 * float(ref.float().abs().max()):
                print("integration: the fused forward is far from the resident-weight forward", file=sys.stderr)
                return 1
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                fused_forward(x)
            e1.record()
            torch.cuda.synchronize()
            res["df11_fused"] = round(e0.elapsed_time(e1) / 10, 4)
            row["df11_fused_vs_resident"] = round(res["df11_fused"] / res["resident"], 3)
            row["df11_fused_max_abs_diff_over_max_abs"] = round(dev_max / float(ref.float().abs().max()), 5)
        if tokens <= 16:
            # The same forwards captured into HIP graphs (runtime.CapturedForward):
            # at a few tokens a forward is many small launches.
            graphs = {"resident_graph": lambda x: runtime.model_forward(x, resident),
                      "df11_inline_graph": lambda x: runtime.model_forward(x, inline)}
            if tokens <= 8:
                graphs["df11_fused_graph"] = fused_forward
            for name, fwd in graphs.items():
                g = runtime.CapturedForward(fwd, x)
                y = g(x)
                torch.cuda.synchronize()
                if name == "df11_fused_graph":
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
        rows.append(row)
    comp = sum(b.tensor.compressed_bytes() for b in blocks)
    raw = sum(2 * b.n_elements for b in blocks)
    print(json.dumps({"integration": "synthetic model forward", "blocks": args.blocks,
                      "weights_per_block": int(blocks[0].n_elements),
                      "overlap_decode_workgroups": args.overlap_workgroups, "compressed_over_bf16": round(comp / raw, 4),
                      "outputs": "in line and overlapped: bit-identical to the resident-weight forward; fused: "
                                 "float32 sums in another order",
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
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write the profiles/ summaries from rocprofv3 runs of this script under DIR, then exit")
    args = ap.parse_args()

    if args.summarize_profiles:
        pre = "cd /tmp && export TMPDIR=/tmp && "   # R = repository root, D = R/gpurun_out/prof
        have = lambda sub: os.path.isdir(os.path.join(args.summarize_profiles, sub))
        if have("trace"):
            summarize_profiles(args.summarize_profiles, {
                "trace": pre + "rocprofv3 --kernel-trace --stats -d $D/trace -o run --output-format csv "
                               "-- python3 $R/bench.py --steps 100 --warmup 300 --no-cpu-baseline > $D/bench.json",
                "fetch": pre + "rocprofv3 --pmc FETCH_SIZE -d $D/fetch -o run --output-format csv "
                               "-- python3 $R/bench.py --steps 3 --warmup 2 --no-cpu-baseline",
                "write": pre + "rocprofv3 --pmc WRITE_SIZE -d $D/write -o run --output-format csv "
                               "-- python3 $R/bench.py --steps 3 --warmup 2 --no-cpu-baseline",
            })
        if have("lin_trace"):
            summarize_linear_profile(args.summarize_profiles,
                                     pre + "rocprofv3 --kernel-trace --stats -d $D/lin_trace -o run --output-format csv "
                                           "-- python3 $R/bench.py --linear-tokens 1 --steps 50 --warmup 20 "
                                           "--no-cpu-baseline > $D/lin.json")
        if have("rans_trace"):
            summarize_kernel_trace(args.summarize_profiles, "rans_trace", "df11_rans_decode",
                                   "df11_rans_decode_kernel on llama3_8b_block (rANS coder)",
                                   pre + "rocprofv3 --kernel-trace --stats -d $D/rans_trace -o run --output-format csv "
                                         "-- python3 $R/bench.py --coder rans --steps 100 --warmup 300 "
                                         "--no-cpu-baseline > $D/rans_trace.json",
                                   "df11_rans_decode_kernel_llama3_8b_block_trace.md")
        counter_runs = [("df11_decode_kernel", "df11_decode_kernel on llama3_8b_block",
                         "--steps 3 --warmup 2 --no-cpu-baseline", "entropy_decoding_df11_amd/csrc/df11_decode.hip",
                         "df11_decode_kernel_llama3_8b_block_counters.md"),
                        ("df11_rans_decode_kernel", "df11_rans_decode_kernel on llama3_8b_block (rANS coder)",
                         "--coder rans --steps 3 --warmup 2 --no-cpu-baseline",
                         "entropy_decoding_df11_amd/csrc/df11_rans_decode.hip",
                         "df11_rans_decode_kernel_llama3_8b_block_counters.md")]
        for kernel, title, bench_args, source, out_name in counter_runs:
            if all(have(f"{kernel}_{sub}") for sub in COUNTER_PASSES):
                summarize_counters(args.summarize_profiles, kernel, title, bench_args, source, out_name)
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
        t = df11.rans_compress(flat, shape=(n,), device=dev)
        out = torch.empty(n, dtype=torch.bfloat16, device=dev)
        h, comp = t.header, t.compressed_bytes()
        config["coder"] = "rans"
        config["rans"] = {"prob_bits": int(h.prob_bits), "lanes": int(h.lanes), "steps": int(h.steps),
                          "segments": int(h.n_segments), "words": int(h.n_words)}
        decode = lambda ev=None: t.decompress(out=out, events=ev)  # noqa: E731
        decoded = lambda: out.view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
    elif views is not None:
        codebook = "per_weight" if wl.endswith("_per_weight") else "shared"
        blk = df11.compress_block([(nm, flat[o:o + r * c].reshape(r, c)) for nm, o, (r, c) in views], device=dev,
                                  decode_table_bits=args.decode_table_bits, codebook=codebook)
        scratch = torch.empty(blk.n_elements, dtype=torch.bfloat16, device=dev)
        config["shapes"] = {name: list(shape) for name, _, shape in views}
        config["codebook"] = codebook
        if codebook == "shared":
            h, comp = blk.tensor.header, blk.tensor.compressed_bytes()
            decode = lambda ev=None: blk.decompress(scratch=scratch, events=ev)  # noqa: E731
        else:
            h, comp = blk.tensors[0].header, blk.compressed_bytes()
            config["streams"] = len(blk.tensors)
            decode = lambda ev=None: blk.decompress(scratch=scratch, events=ev)  # noqa: E731

        def decoded():
            if codebook == "shared":
                return scratch[:n].view(torch.int16).cpu().numpy().view(np.uint16)
            outs = blk.decompress(scratch=scratch)  # cached views; decodes once more
            torch.cuda.synchronize()
            return np.concatenate([outs[nm].reshape(-1).view(torch.int16).cpu().numpy().view(np.uint16)
                                   for nm, _, _ in views])
    else:
        t = df11.compress(flat, shape=(n,), device=dev, decode_table_bits=args.decode_table_bits)
        out = torch.empty(n, dtype=torch.bfloat16, device=dev)
        h, comp = t.header, t.compressed_bytes()
        decode = lambda ev=None: t.decompress(out=out, events=ev)  # noqa: E731
        decoded = lambda: out.view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
    t_enc = time.perf_counter() - t0
    algo_bytes = comp + 2 * n

    # Check the decode first: the copy back and the comparison leave the GPU
    # idle long enough for its clocks to drop, which the warmup then undoes.
    decode()
    torch.cuda.synchronize()
    if not np.array_equal(decoded(), flat):
        print(f"bench: decoded {wl} differs from the original weights", file=sys.stderr)
        return 1

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for e in starts + ends:  # create the events outside the timed region
        e.record(stream)
    for _ in range(args.warmup):
        decode()
    torch.cuda.synchronize()
    # Whole-job time: back-to-back launches as an application issues them.
    wall0 = time.perf_counter()
    for i in range(args.steps):
        decode()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    # Kernel time: the same launches again, each recording its kernel's own
    # start and end (dispatch events; recording them widens the gap between
    # launches by ~4.5 us, so the wall time above is taken without them).
    # The check of the output comes after both: the copy to the host idles
    # the GPU long enough for its clocks to drop.
    for i in range(args.steps):
        decode((starts[i], ends[i]))
    torch.cuda.synchronize()
    kern_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    if not np.array_equal(decoded(), flat):
        print(f"bench: the timed launches decoded {wl} wrongly", file=sys.stderr)
        return 1
    mean_ms = float(np.mean(kern_ms))
    achieved = algo_bytes / (mean_ms * 1e-3) / 1e9
    value = args.steps * algo_bytes / wall / 1e9

    # Cold caches: COLD_LAUNCHES more launches, each after reading 1 GiB so that neither
    # the L2 nor the 256 MB MALL holds the stream (outside the timed launch;
    # the hot numbers above come from back-to-back launches).  The flush reads
    # rather than writes: written lines would be dirty, and the timed launch
    # would pay for writing them back.
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    cold_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(COLD_LAUNCHES)]
    sink = torch.empty((), dtype=torch.float32, device=dev)
    for ev in cold_ev:
        torch.sum(flush, dim=0, out=sink)
        decode(ev)
    torch.cuda.synchronize()
    cold_ms = float(np.median([a.elapsed_time(b) for a, b in cold_ev]))
    del flush
    if not np.array_equal(decoded(), flat):
        print(f"bench: the cold-cache launches decoded {wl} wrongly", file=sys.stderr)
        return 1

    # A plain copy kernel over the same byte count, as the achievable-bandwidth reference.
    src = torch.empty(algo_bytes // 2, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 10 * 2 * src.numel() / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    traffic = _traffic_from_profile() if wl == DEFAULT_WORKLOAD and args.coder == "huffman" else None
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
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
        "kernel_ms_mean": round(mean_ms, 5),
        "kernel_ms_min": round(float(np.min(kern_ms)), 5),
        "kernel_ms_cold_median": round(cold_ms, 5),
        "cache": "kernel_ms_mean and roofline: back-to-back launches (hot caches; a stream larger than the "
                 "256 MB MALL is read from HBM anyway); kernel_ms_cold_median: after reading 1 GiB",
        "copy_kernel_GBps": round(copy_gbps, 1),
        "frac_of_copy": round(achieved / copy_gbps, 4),
        "host_gen_s": round(t_gen, 2),
        "host_encode_s": round(t_enc, 2),
    }
    if not args.no_cpu_baseline:
        threads = args.cpu_threads or len(os.sched_getaffinity(0))
        threads = min(threads, 16)
        if args.coder == "rans":
            cpu_gbps, cpu_s, ok = _cpu_baseline_rans(flat)
            threads, how = 1, "rANS decode on one thread"
        else:
            cpu_gbps, cpu_s, ok = _cpu_baseline(flat, threads)
            how = f"tree-walk decode split by groups over {threads} threads"
        result["cpu_baseline"] = {
            "value": round(cpu_gbps, 3),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"the whole {wl} data as one stream ({n} weights), {how}; {cpu_s:.2f} s wall; output "
                      f"{'matches' if ok else 'DIFFERS FROM'} the original weights",
        }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
