"""DF11 decompression throughput on one MI355X.

One step = one batched decompression of the Llama-3-8B-shaped transformer block
(q, k, v, o, gate, up, down; one DF11 stream, shared codebook, ~218M BF16
weights) into one scratch buffer, with the compressed stream already resident
in HBM.  Prints one JSON line.

  value     = K * (algorithmic bytes per step) / (timed wall time), GB/s
  algorithmic bytes per step = EncodedExponent + PackedSignMantissa + Gaps
              + output positions + LUTs + CodeLengths (all unpadded) read,
              plus 2 bytes per BF16 weight written
  roofline  = the same bytes / the decode kernel's mean duration (HIP events
              around each launch on its stream) against the 8 TB/s HBM peak
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


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-table-bits", type=int, default=11)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0, help="oracle threads (default: usable host cores)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: DF11 decoding needs no exchange between GPUs, and every "
              "GPU would decode its own streams; run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    from entropy_decoding_df11_amd import df11, workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    flat, views = workloads.gen_block()
    t_gen = time.perf_counter() - t0
    t0 = time.perf_counter()
    blk = df11.compress_block([(n, flat[o:o + r * c].reshape(r, c)) for n, o, (r, c) in views], device=dev,
                              decode_table_bits=args.decode_table_bits)
    t_enc = time.perf_counter() - t0
    t = blk.tensor
    h = t.header
    n = int(h.n_elements)
    comp = t.compressed_bytes()
    algo_bytes = comp + 2 * n
    scratch = torch.empty(n, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    for _ in range(args.warmup):
        blk.decompress(scratch=scratch)
    torch.cuda.synchronize()
    got = scratch.view(torch.int16).cpu().numpy().view(np.uint16)
    if not np.array_equal(got, flat):
        print("bench: decoded block differs from the original weights", file=sys.stderr)
        return 1

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        blk.decompress(scratch=scratch)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    kern_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    mean_ms = float(np.mean(kern_ms))
    achieved = algo_bytes / (mean_ms * 1e-3) / 1e9
    value = args.steps * algo_bytes / wall / 1e9

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

    traffic = _traffic_from_profile()
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
            "workload": "llama3_8b_block",
            "shapes": {name: list(shape) for name, _, shape in views},
            "n_elements": n,
            "codebook": "shared",
            "bits_per_weight": round(8 * comp / n, 4),
            "compressed_bytes": comp,
            "decode_table_bits": args.decode_table_bits,
            "max_code_len": int(h.max_len),
            "n_luts": int(h.n_luts),
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
        "copy_kernel_GBps": round(copy_gbps, 1),
        "frac_of_copy": round(achieved / copy_gbps, 4),
        "host_gen_s": round(t_gen, 2),
        "host_encode_s": round(t_enc, 2),
    }
    if not args.no_cpu_baseline:
        threads = args.cpu_threads or len(os.sched_getaffinity(0))
        threads = min(threads, 16)
        cpu_gbps, cpu_s, ok = _cpu_baseline(flat, threads)
        result["cpu_baseline"] = {
            "value": round(cpu_gbps, 3),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"the whole llama3_8b_block stream ({n} weights), tree-walk decode split by groups "
                      f"over {threads} threads; {cpu_s:.2f} s wall; output {'matches' if ok else 'DIFFERS FROM'} "
                      f"the original weights",
        }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
