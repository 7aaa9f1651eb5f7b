"""Benchmark: 2^28 u32 key + u32 value LSD radix sort on one MI355X.

One step = one full sort (clear, all-pass histogram, 4 sweep passes of 8-bit
digits) of 2^28 seeded synthetic pairs already resident in HBM, out of place
from an input the loop never writes.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--dist uniform|and3]
                    [--no-cpu-baseline]

roofline: the dominant kernel is the sweep pass; its algorithmic traffic is
16 B per pair (read key + value, write key + value), so
achieved = 16 * n / (average sweep launch time), against 8 TB/s HBM peak.
The average launch time comes from HIP events the library records around each
sweep launch inside the timed region.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
N = 1 << 28
DIGIT_BITS = 8
BYTES_PER_PAIR_PER_PASS = 16
# HBM bytes per sweep launch of the current sweep kernel (512 x 24 tile, ballot
# ranking) measured by rocprofv3 FETCH_SIZE and WRITE_SIZE over this benchmark,
# each scaled by the copy-kernel calibration (x2.0 and x1.0); set to None when
# the kernel changes until the counters are taken again.
MEASURED_SWEEP_TRAFFIC = 4_735_635_251


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(min_seconds: float = 10.0, max_runs: int = 3):
    """Single-threaded oracle on the benchmark's own input, repeated until at
    least min_seconds of CPU work (at most max_runs sorts)."""
    import oracle
    import workloads

    keys, vals = workloads.pairs_c3(N, "uniform")
    runs, total = 0, 0.0
    while runs < max_runs and (runs == 0 or total < min_seconds):
        t0 = time.perf_counter()
        oracle.radix_sort_pairs(keys, vals, 0, 32, DIGIT_BITS)
        total += time.perf_counter() - t0
        runs += 1
    return {
        "value": round(runs * N / total / 1e9, 5),
        "unit": "Gkeys/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"the whole 2^28-pair uniform workload (value = index), 4-pass 8-bit LSD sort by the "
                  f"plain C oracle, single thread, {runs} run(s) in {total:.2f} s",
        "host_cpus": os.cpu_count(),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--dist", default="uniform", choices=["uniform", "and3"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import lsd_radix_sort_amd as lrs
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    lrs.load_library()
    dev = torch.device("cuda:0")

    log(f"generating {N} pairs ({args.dist})")
    keys, vals = workloads.pairs_c3(N, args.dist)
    k_in = torch.from_numpy(keys.view(np.int32)).to(dev)
    v_in = torch.from_numpy(vals.view(np.int32)).to(dev)
    del keys, vals
    k_out = torch.empty_like(k_in)
    v_out = torch.empty_like(v_in)
    ws = torch.empty(lrs.radix_sort_workspace_size(N, 0, 32, DIGIT_BITS, True), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        lrs.radix_sort_pairs(k_in, v_in, 0, 32, DIGIT_BITS, keys_out=k_out, values_out=v_out, workspace=ws)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    with lrs.KernelTimer() as kt:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    gkeys = N / (ms_per_step / 1e3) / 1e9

    passes = 32 // DIGIT_BITS
    sweep_ms = kt.ms["sweep"] / max(kt.launches["sweep"], 1)
    hist_ms = kt.ms["histogram"] / max(kt.launches["histogram"], 1)
    clear_ms = kt.ms["clear"] / max(kt.launches["clear"], 1)
    sweep_bytes = BYTES_PER_PAIR_PER_PASS * N
    achieved = sweep_bytes / (sweep_ms / 1e3) / 1e9

    # copy yardstick: 2 GiB -> 2 GiB with the library's copy kernel
    src = k_in.view(torch.uint8)
    dst = k_out.view(torch.uint8)
    with lrs.KernelTimer() as ct:
        for _ in range(5):
            lrs.copy_probe(src, dst)
    copy_ms = ct.ms["copy"] / max(ct.launches["copy"], 1)
    copy_gbs = 2 * src.numel() / (copy_ms / 1e3) / 1e9
    log(f"sort {ms_per_step:.3f} ms/step, {gkeys:.2f} Gkeys/s; sweep {sweep_ms:.3f} ms/pass = "
        f"{achieved:.0f} GB/s; histogram {hist_ms:.3f} ms; clear {clear_ms:.3f} ms; copy {copy_gbs:.0f} GB/s")

    traffic = None
    if MEASURED_SWEEP_TRAFFIC is not None:
        traffic = MEASURED_SWEEP_TRAFFIC
    result = {
        "metric": "Gkeys/s and achieved HBM GB/s (% of peak), 2^28 u32 key-value radix sort",
        "value": round(gkeys, 4),
        "unit": "Gkeys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {
            "workload": f"2^28 u32 key + u32 value pairs (value = original index), {args.dist} keys, "
                        f"8-bit digits, 4 LSD passes",
            "n": N, "digit_bits": DIGIT_BITS, "passes": passes, "key_distribution": args.dist,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "sweep_kernel<8-bit digit, u32 key, u32 value> (one LSD pass)",
            "bytes_per_launch": sweep_bytes,
            "avg_launch_ms": round(sweep_ms, 4),
        },
        "per_kernel_ms": {"clear": round(clear_ms, 4), "histogram": round(hist_ms, 4),
                          "sweep_per_pass": round(sweep_ms, 4)},
        "hbm_gbs_per_pass": round(achieved, 1),
        "copy_probe_gbs": round(copy_gbs, 1),
        "frac_of_copy": round(achieved / copy_gbs, 4),
    }
    del k_in, v_in, k_out, v_out, ws
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
