"""Benchmark: LSD radix sort on one MI355X.

Default workload (the headline): 2^28 u32 key + u32 value pairs, value =
original index, uniform keys, 8-bit digits, 4 passes.  One step = one full
sort (clear, all-pass histogram, one sweep per pass) of seeded synthetic data
already resident in HBM, out of place from an input the loop never writes.
Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--scan lookback|reduce-then-scan] [--lib PATH]
    python bench.py --graph-sweep     (eager vs HIP-graph replay, 1K .. 1M keys)

Other workloads (same line format, for the record): c1_keys_1k_4bit,
c2_keys_4m_4bit, c2_keys_4m_8bit, c3_pairs_2p28_and3, c4_fp16_1024x65536_asc,
c5_bf16_4096x4096_desc, f32_pairs_2p28_desc, i32_keys_2p28_asc,
f64_pairs_2p27_asc, u32_pairs_2p29_uniform, u32_pairs_2p30_uniform.

roofline: the dominant kernel is the sweep (one LSD pass).  achieved = the
algorithmic bytes of the sweep launches of one sort (pairs: 16 B per pair per
pass; keys: 8 B per key per pass; 8-byte keys with a u32 value: 24 B; fp16/bf16
rows of at most 65,536 with their int64 index, which travel between passes as
one word key << 16 | column: 6, 8, ..., 8, 14 B per element from the first to
the last pass; longer rows 8, 12, ..., 12, 16 B) / their summed duration, from
HIP events on the sort's stream inside the timed region (stamped by the timed
dispatches themselves).  Rows of at most 8192 elements are sorted by one
whole-row resident launch instead (read once, write once: 8 B/key, 16 B/pair,
12 B per fp16/bf16 element with its int64 index).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
HEADLINE = "c3_pairs_2p28_uniform"
# Device-code sources whose text fixes the dominant kernels and their launch
# shapes; their hash ties a counter measurement to the kernel it was taken on.
KERNEL_SOURCES = ("lsd_radix_sort_amd/csrc/lrs_kernels.h", "lsd_radix_sort_amd/csrc/lrs_launch.h",
                  "lsd_radix_sort_amd/csrc/lrs_launch_impl.h")
# HBM bytes per launch of the dominant kernel, from two rocprofv3 --pmc runs of
# this benchmark (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled
# by what the same counter reads for the library's copy kernel of known size;
# keyed by workload, with the hash of KERNEL_SOURCES the counters were taken
# on.  A workload whose kernels have changed since reports traffic null.
MEASURED_TRAFFIC = {
    HEADLINE: {"kernel_sha16": "50625c0fa304a713", "bytes_per_launch": 4_457_457_045,
               "source": "profiles/sweep_kernel_2p28_pairs_uniform_hbm_traffic.md"},
    # the mean over the four passes' launches
    "c4_fp16_1024x65536_asc": {"kernel_sha16": "50625c0fa304a713", "bytes_per_launch": 607_610_695,
                               "source": "profiles/sweep_kernel_fp16_1024x65536_asc_kernel_trace.md"},
    "c5_bf16_4096x4096_desc": {"kernel_sha16": "50625c0fa304a713", "bytes_per_launch": 201_426_119,
                               "source": "profiles/row_resident_kernel_bf16_4096x4096_desc_kernel_trace.md"},
    "i32_keys_2p28_asc": {"kernel_sha16": "50625c0fa304a713", "bytes_per_launch": 2_255_819_267,
                          "source": "profiles/sweep_kernel_2p28_i32_keys_kernel_trace.md"},
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


WORKLOADS = {
    "c1_keys_1k_4bit": dict(kind="keys", n=1024, end_bit=12, b=4, desc="1,024 u32 keys uniform in [0,4096), "
                            "keys only, 4-bit digits, 3 passes (bits 0-11)"),
    "c2_keys_4m_4bit": dict(kind="keys", n=1 << 22, end_bit=32, b=4, desc="4,194,304 u32 keys, full range, "
                            "keys only, 4-bit digits, 8 passes"),
    "c2_keys_4m_8bit": dict(kind="keys", n=1 << 22, end_bit=32, b=8, desc="4,194,304 u32 keys, full range, "
                            "keys only, 8-bit digits, 4 passes"),
    "c3_pairs_2p28_uniform": dict(kind="pairs", n=1 << 28, end_bit=32, b=8, dist="uniform",
                                  desc="2^28 u32 key + u32 value pairs (value = original index), uniform keys, "
                                       "8-bit digits, 4 LSD passes"),
    "c3_pairs_2p28_and3": dict(kind="pairs", n=1 << 28, end_bit=32, b=8, dist="and3",
                               desc="2^28 u32 key + u32 value pairs (value = original index), keys = AND of 3 "
                                    "uniform words, 8-bit digits, 4 LSD passes"),
    "c4_fp16_1024x65536_asc": dict(kind="rows", rows=1024, cols=65536, dtype="fp16", descending=False, b=4,
                                   desc="fp16 (1024, 65536) N(0,1) rows, ascending, int64 column index, 4-bit "
                                        "digits, 4 passes"),
    "c5_bf16_4096x4096_desc": dict(kind="rows", rows=4096, cols=4096, dtype="bf16", descending=True, b=8,
                                   desc="bf16 (4096, 4096) 64-level N(0,1) rows, descending, int64 column index, "
                                        "8-bit digits, 2 passes"),
    "f32_pairs_2p28_desc": dict(kind="pairs", typed="f32", descending=True, n=1 << 28, end_bit=32, b=8,
                                desc="2^28 fp32 N(0,1) keys + u32 value pairs (value = original index), "
                                     "descending, 8-bit digits, 4 passes"),
    "i32_keys_2p28_asc": dict(kind="keys", typed="i32", descending=False, n=1 << 28, end_bit=32, b=8,
                              desc="2^28 uniform int32 keys, keys only, ascending, 8-bit digits, 4 passes"),
    "u32_pairs_2p29_uniform": dict(kind="pairs", n=1 << 29, end_bit=32, b=8, dist="uniform",
                                   desc="2^29 u32 key + u32 value pairs (value = original index), uniform keys, "
                                        "8-bit digits, 4 passes (32-bit sweep; byte offsets past 2^31)"),
    "u32_pairs_2p30_uniform": dict(kind="pairs", n=1 << 30, end_bit=32, b=8, dist="uniform",
                                   desc="2^30 u32 key + u32 value pairs (value = original index), uniform keys, "
                                        "8-bit digits, 4 passes (64-bit look-back words and store addresses)"),
    "f64_pairs_2p27_asc": dict(kind="pairs", typed="f64", descending=False, n=1 << 27, end_bit=64, b=8,
                               key_bytes=8, desc="2^27 fp64 N(0,1) keys + u32 value pairs (value = original "
                                                 "index), ascending, 8-bit digits, 8 passes"),
}


def sweep_bytes(w) -> int:
    """Algorithmic bytes of all sweep launches of one sort of workload w."""
    P = -(-w["end_bit"] // w["b"]) if w["kind"] != "rows" else 16 // w["b"]
    kb = w.get("key_bytes", 4)
    if w["kind"] == "keys":
        return 2 * kb * w["n"] * P
    if w["kind"] == "pairs":
        return (2 * kb + 8) * w["n"] * P
    n = w["rows"] * w["cols"]
    total = 0
    for p in range(P):
        if w["cols"] <= 65536:
            # key << 16 | column as one u32 word between passes
            read = 2 if p == 0 else 4           # pattern, then words
            write = 2 + 8 if p == P - 1 else 4  # words, then pattern + int64 index
        else:
            read = 2 + (4 if p > 0 else 0)          # 16-bit pattern (+ u32 index after the first pass)
            write = 2 + (8 if p == P - 1 else 4)    # pattern + u32 index (int64 on the last pass)
        total += read + write
    return n * total


def resident_bytes(w) -> int:
    """Algorithmic bytes of one whole-row resident sort: read once, write once."""
    if w["kind"] == "keys":
        return 8 * w["n"]
    if w["kind"] == "pairs":
        return 16 * w["n"]
    return 12 * w["rows"] * w["cols"]  # 16-bit pattern in; pattern + int64 index out


def kernel_sources_sha16() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(name: str):
    """HBM bytes per launch of the dominant kernel from the counter runs, or
    None if there are none for the kernels as they are now."""
    m = MEASURED_TRAFFIC.get(name)
    if m is None or m["kernel_sha16"] != kernel_sources_sha16():
        return None
    return m["bytes_per_launch"]


def cpu_baseline(min_seconds: float = 10.0, max_runs: int = 3):
    """Single-threaded oracle on the headline workload's own input, repeated
    until at least min_seconds of CPU work (at most max_runs sorts); plus the
    context figure of std::sort on one core over the first 2^24 of its keys."""
    import oracle
    import workloads

    n = 1 << 28
    keys, vals = workloads.pairs_c3(n, "uniform")
    runs, total = 0, 0.0
    while runs < max_runs and (runs == 0 or total < min_seconds):
        t0 = time.perf_counter()
        oracle.radix_sort_pairs(keys, vals, 0, 32, 8)
        total += time.perf_counter() - t0
        runs += 1
    m = 1 << 24
    std_s = oracle.std_sort_seconds(keys[:m])
    return {
        "value": round(runs * n / total / 1e9, 5),
        "unit": "Gkeys/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"the whole 2^28-pair uniform workload (value = index), 4-pass 8-bit LSD sort by the "
                  f"plain C oracle, single thread, {runs} run(s) in {total:.2f} s",
        "host_cpus": os.cpu_count(),
        "std_sort_context": {"value": round(m / std_s / 1e9, 5), "unit": "Gkeys/s", "cores": 1,
                             "sample": f"std::sort of the first 2^24 keys of the same workload (keys only), "
                                       f"one core, {std_s:.2f} s"},
    }


def graph_sweep(sizes, digit_bits: int, reps: int):
    """Per-sort time of u32 keys-only sorts launched eagerly and replayed from a
    captured HIP graph, at each size; prints a markdown table to stderr and
    returns the rows."""
    import numpy as np
    import torch

    import lsd_radix_sort_amd as lrs
    import workloads

    rows = []
    log(f"| keys | launches per sort | eager us/sort | graph replay us/sort | graph / eager |")
    log("|---:|---:|---:|---:|---:|")
    for n in sizes:
        keys = workloads.random_u32(20_000 + n % 997, n)
        k_in = torch.from_numpy(keys.view(np.int32)).cuda()
        k_out = torch.empty_like(k_in)
        ws = torch.empty(max(1, lrs.radix_sort_workspace_size(n, 0, 32, digit_bits)), dtype=torch.uint8,
                         device="cuda")

        def run():
            lrs.radix_sort_keys(k_in, 0, 32, digit_bits, out=k_out, workspace=ws)

        timer = lrs.KernelTimer()
        lrs.radix_sort_keys(k_in, 0, 32, digit_bits, out=k_out, workspace=ws,
                            options=lrs.SortOptions(timer=timer))
        torch.cuda.synchronize()
        launches = sum(timer.read()[1].values())
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        result = {}
        for mode in ("eager", "graph"):
            call = run if mode == "eager" else g.replay
            for _ in range(10):
                call()
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(reps):
                call()
            t1.record()
            torch.cuda.synchronize()
            result[mode] = t0.elapsed_time(t1) * 1e3 / reps
        got = k_out.cpu().numpy().view(np.uint32)
        assert np.array_equal(got, np.sort(keys)), f"n={n}: sort result wrong"
        row = {"n": n, "launches": launches, "eager_us": round(result["eager"], 2),
               "graph_us": round(result["graph"], 2), "ratio": round(result["graph"] / result["eager"], 3)}
        rows.append(row)
        log(f"| {n:,} | {launches} | {row['eager_us']} | {row['graph_us']} | {row['ratio']} |")
    return rows


def tile_trace_report(rec, sweeps: int, clock_mhz: float, sweep_ms: float):
    """Phase times of the sweep tiles of one sort from the library's tile
    records (rec: int64 array [sweeps * tiles, 12], launches in order).
    Prints a table per launch to stderr and returns a summary dict."""
    import numpy as np

    names = ["load + rank", "local scans", "reorder + look-back", "key write-out issue",
             "payload load + reorder", "payload write-out issue"]
    tiles = rec.shape[0] // sweeps
    out = {"tiles_per_launch": int(tiles), "launches": []}
    us = 1.0 / clock_mhz
    log(f"{sweeps} sweep launches of {tiles} tiles; clock {clock_mhz:g} MHz")
    log("| launch | span us | tile us (median) | " + " | ".join(f"{n} (median us)" for n in names) + " |")
    log("|---:|---:|---:|" + "---:|" * len(names))
    for L in range(sweeps):
        r = rec[L * tiles:(L + 1) * tiles].astype(np.int64)
        t = r[:, :7]
        span = (t[:, 6].max() - t[:, 0].min()) * us
        phases = np.diff(t, axis=1) * us
        med = np.median(phases, axis=0)
        lat = np.median(t[:, 6] - t[:, 0]) * us
        out["launches"].append({"span_us": round(float(span), 1), "tile_us": round(float(lat), 2),
                                "phase_median_us": [round(float(x), 2) for x in med],
                                "phase_mean_us": [round(float(x), 2) for x in phases.mean(axis=0)]})
        log(f"| {L} | {span:.1f} | {lat:.2f} | " + " | ".join(f"{x:.2f}" for x in med) + " |")
    # where the tiles ran: the XCD each tile's workgroup reports against the
    # XCD its index is dealt to (chunk c of 16 consecutive tiles to XCD c % 8)
    r = rec[:tiles].astype(np.int64)
    idx = np.arange(tiles)
    xcc = r[:, 7] & 0xF
    expect = (idx // 16) % 8
    blk_xcd = r[:, 9] % 8
    cu = (r[:, 8] >> 8) & 0xF
    se = (r[:, 8] >> 13) & 0x7
    places = np.unique(xcc * 1000 + se * 100 + cu).size
    walk = rec[:, 10].astype(np.int64)
    polls = rec[:, 11].astype(np.int64)
    out.update({"tiles_on_dealt_xcd": int((xcc == expect).sum()), "workgroup_xcd_is_index_mod_8": int((xcc == blk_xcd).sum()),
                "distinct_xcd_se_cu": int(places), "sweep_ms_timer": sweep_ms,
                "lookback_predecessors_median": float(np.median(walk)), "lookback_predecessors_p90": float(np.percentile(walk, 90)),
                "lookback_polls_median": float(np.median(polls)), "lookback_polls_p90": float(np.percentile(polls, 90))})
    log(f"look-back of digit 0: predecessors added up median {np.median(walk):g} (p90 {np.percentile(walk, 90):g}), "
        f"polls median {np.median(polls):g} (p90 {np.percentile(polls, 90):g})")
    log(f"launch 0: {out['tiles_on_dealt_xcd']} of {tiles} tiles ran on the XCD their index is dealt to; "
        f"XCD = workgroup index mod 8 for {out['workgroup_xcd_is_index_mod_8']}; "
        f"{places} distinct (XCD, shader engine, CU) places")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--dist", default=None, choices=["uniform", "and3"],
                    help="shorthand for the 2^28-pair workload with this key distribution")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--scan", default="lookback", choices=["lookback", "reduce-then-scan"],
                    help="offset strategy of single-row sorts (the A/B of the two)")
    ap.add_argument("--graph-sweep", action="store_true",
                    help="instead of the workload: eager vs HIP-graph replay per-sort time of u32 keys-only "
                         "sorts from 1K to 1M keys (table on stderr, one JSON line)")
    ap.add_argument("--tile-trace", action="store_true",
                    help="after the warm-up, one sort with the tile phase records of a library built with "
                         "-DLRS_TILE_TRACE=1 (pass it with --lib); phase table on stderr, one JSON line")
    ap.add_argument("--tile-trace-out", default=None,
                    help="with --tile-trace: also save the raw records (int64 [launches * tiles, 12]) as .npy")
    ap.add_argument("--lib", default=None,
                    help="library file to time instead of the in-tree build (a variant built with "
                         "python -m lsd_radix_sort_amd.build -D... --out PATH)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    if args.graph_sweep:
        import torch

        import lsd_radix_sort_amd as lrs
        if args.lib is not None:
            lrs.LIB_PATH = os.path.abspath(args.lib)
        lrs.load_library()
        out = {}
        for b in (4, 8):
            log(f"u32 keys only, {32 // b} passes of {b}-bit digits")
            out[f"b{b}"] = graph_sweep([1024, 4096, 16384, 65536, 262144, 1 << 20], b, max(args.steps, 50))
        print(json.dumps({"metric": "per-sort time, eager launches vs HIP-graph replay", "unit": "us",
                          "graph_sweep": out}), flush=True)
        return
    name = args.workload
    if args.dist is not None:
        name = f"c3_pairs_2p28_{args.dist}"
    w = WORKLOADS[name]

    import numpy as np
    import torch

    import lsd_radix_sort_amd as lrs
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.lib is not None:
        lrs.LIB_PATH = os.path.abspath(args.lib)
    lrs.load_library()
    dev = torch.device("cuda:0")
    timer = lrs.KernelTimer()
    untimed = lrs.SortOptions(scan=args.scan)
    timed = lrs.SortOptions(scan=args.scan, timer=timer)

    log(f"generating {name}")
    if w["kind"] == "keys" and "typed" in w:
        keys = workloads.keys_i32_uniform(w["n"])
        k_in = torch.from_numpy(keys.view(np.int32)).to(dev)
        del keys
        n_keys = w["n"]
        k_out = torch.empty_like(k_in)
        ws = torch.empty(lrs.radix_sort_workspace_size(n_keys, 0, 32, w["b"], False), dtype=torch.uint8, device=dev)

        def step(opts):
            lrs.radix_sort_keys_typed(k_in, w["descending"], w["typed"], 0, 32, w["b"], out=k_out, workspace=ws,
                                      options=opts)
        copy_pair = (k_in.view(torch.uint8), k_out.view(torch.uint8))
    elif w["kind"] == "keys":
        keys = workloads.keys_c1(w["n"]) if w["n"] == 1024 else workloads.keys_c2(w["n"])
        k_in = torch.from_numpy(keys.view(np.int32)).to(dev)
        n_keys = w["n"]
        k_out = torch.empty_like(k_in)
        ws = torch.empty(max(1, lrs.radix_sort_workspace_size(n_keys, 0, w["end_bit"], w["b"], False)),
                         dtype=torch.uint8, device=dev)

        def step(opts):
            lrs.radix_sort_keys(k_in, 0, w["end_bit"], w["b"], out=k_out, workspace=ws, options=opts)
        scratch = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
        copy_pair = (scratch[: 1 << 27], scratch[1 << 27:])
    elif w["kind"] == "pairs" and "typed" in w:
        if w["typed"] == "f64":
            keys = workloads.keys_f64_normal(w["n"])
            k_in = torch.from_numpy(keys.view(np.int64)).to(dev).view(torch.float64)
        else:
            keys = workloads.keys_f32_normal(w["n"])
            k_in = torch.from_numpy(keys.view(np.int32)).to(dev).view(torch.float32)
        del keys
        v_in = torch.arange(w["n"], dtype=torch.int32, device=dev)
        n_keys = w["n"]
        k_out = torch.empty_like(k_in)
        v_out = torch.empty_like(v_in)
        ws = torch.empty(lrs.radix_sort_typed_workspace_size(n_keys, w["typed"], 0, w["end_bit"], w["b"], True),
                         dtype=torch.uint8, device=dev)

        def step(opts):
            lrs.radix_sort_pairs_typed(k_in, v_in, w["descending"], w["typed"], 0, w["end_bit"], w["b"],
                                       keys_out=k_out, values_out=v_out, workspace=ws, options=opts)
        copy_pair = (k_in.view(torch.uint8), k_out.view(torch.uint8))
    elif w["kind"] == "pairs":
        keys, vals = workloads.pairs_c3(w["n"], w["dist"])
        k_in = torch.from_numpy(keys.view(np.int32)).to(dev)
        v_in = torch.from_numpy(vals.view(np.int32)).to(dev)
        del keys, vals
        n_keys = w["n"]
        k_out = torch.empty_like(k_in)
        v_out = torch.empty_like(v_in)
        ws = torch.empty(lrs.radix_sort_workspace_size(n_keys, 0, 32, w["b"], True), dtype=torch.uint8, device=dev)

        def step(opts):
            lrs.radix_sort_pairs(k_in, v_in, 0, 32, w["b"], keys_out=k_out, values_out=v_out, workspace=ws,
                                 options=opts)
        copy_pair = (k_in.view(torch.uint8), k_out.view(torch.uint8))
    else:
        bits = workloads.matrix_c4(w["rows"], w["cols"]) if w["dtype"] == "fp16" else workloads.matrix_c5(
            w["rows"], w["cols"])
        x = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.float16 if w["dtype"] == "fp16"
                                                                else torch.bfloat16)
        n_keys = w["rows"] * w["cols"]
        vo = torch.empty_like(x)
        io = torch.empty((w["rows"], w["cols"]), dtype=torch.int64, device=dev)
        ws = torch.empty(lrs.segmented_row_sort_workspace_size(w["rows"], w["cols"], w["b"]), dtype=torch.uint8,
                         device=dev)

        def step(opts):
            lrs.segmented_row_sort(x, w["descending"], w["b"], values_out=vo, indices_out=io, workspace=ws,
                                   options=opts)
        scratch = io.view(torch.uint8).reshape(-1)
        half = scratch.numel() // 2 // 16 * 16
        copy_pair = (scratch[:half], scratch[half:2 * half])
    torch.cuda.synchronize()

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step(untimed)
    torch.cuda.synchronize()

    if args.tile_trace:
        # one more sort with every sweep tile's phase record; the clock rate
        # is checked against the sweep time the kernel timer gives
        buf = torch.zeros(max(1, n_keys // 2048) * lrs.KernelTimer.TRACE_WORDS * 8, dtype=torch.int64, device=dev)
        try:
            timer.trace_tiles(buf)
        except lrs.RadixSortArgumentError:
            log("this library records no tile phases: build one with python -m lsd_radix_sort_amd.build "
                "-DLRS_TILE_TRACE=1 --out PATH and pass --lib PATH")
            sys.exit(2)
        with timer as kt:
            step(timed)
            torch.cuda.synchronize()
        used = timer.trace_used()
        timer.trace_tiles(None)
        sweeps = kt.launches["sweep"]
        if used == 0 or sweeps == 0:
            log("no tile records: a library built with -DLRS_TILE_TRACE=1 and a workload sorted by sweeps are needed")
            sys.exit(2)
        rec = buf[:used].view(-1, lrs.KernelTimer.TRACE_WORDS).cpu().numpy()
        if args.tile_trace_out:
            np.save(args.tile_trace_out, rec)
        first, last = rec[:, 0].min(), rec[:, 6].max()
        sweep_ms = kt.ms["sweep"]
        clock_mhz = 100.0
        log(f"records span {(last - first) / clock_mhz:.1f} us at {clock_mhz:g} MHz; the timer's sweeps sum to "
            f"{sweep_ms * 1e3:.1f} us")
        summary = tile_trace_report(rec, sweeps, clock_mhz, sweep_ms)
        print(json.dumps({"metric": "sweep tile phase times", "unit": "us", "workload": name, **summary}),
              flush=True)
        return

    log(f"timing {args.steps} steps")
    with timer as kt:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(timed)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    gkeys = n_keys / (ms_per_step / 1e3) / 1e9

    # The same steps again without the kernel timer, after the timed region:
    # what timing every kernel costs the sort (little for large sorts; for
    # small ones, whose launches the host paces, the events are a large part
    # of each step).  Context only; the line's value is the timed region's.
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        step(untimed)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    ms_per_step_untimed = (t3 - t2) * 1e3 / args.steps

    # Inputs of at most 8192 elements per row are sorted by one whole-row
    # resident launch (one read, one write); longer ones by one sweep per pass.
    resident = kt.launches["resident"] > 0
    kind = "resident" if resident else "sweep"
    dom_launches = max(kt.launches[kind], 1)
    dom_ms_total = kt.ms[kind] / args.steps
    dom_ms = kt.ms[kind] / dom_launches
    hist_ms = kt.ms["histogram"] / max(kt.launches["histogram"], 1)
    clear_ms = kt.ms["clear"] / max(kt.launches["clear"], 1)
    launches_per_sort = dom_launches // args.steps
    bytes_sort = resident_bytes(w) if resident else sweep_bytes(w)
    achieved = bytes_sort / (dom_ms_total / 1e3) / 1e9
    sweep_ms = dom_ms

    # copy yardstick: the library's streaming copy kernel between two resident
    # buffers (the 1 GiB key buffers for the 2^28-pair workloads)
    copy_opts = lrs.SortOptions(timer=timer)
    lrs.copy_probe(copy_pair[0], copy_pair[1])  # untimed: loads the copy kernel's code object
    torch.cuda.synchronize()
    with timer as ct:
        for _ in range(5):
            lrs.copy_probe(copy_pair[0], copy_pair[1], options=copy_opts)
    copy_ms = ct.ms["copy"] / max(ct.launches["copy"], 1)
    copy_gbs = 2 * copy_pair[0].numel() / (copy_ms / 1e3) / 1e9
    log(f"{name}: sort {ms_per_step:.4f} ms/step ({ms_per_step_untimed:.4f} untimed), {gkeys:.3f} Gkeys/s; "
        f"{kind} {sweep_ms:.4f} ms/launch x {launches_per_sort} = {achieved:.0f} GB/s; histogram {hist_ms:.4f} ms; "
        f"clear {clear_ms:.4f} ms; copy {copy_gbs:.0f} GB/s")

    result = {
        "metric": "Gkeys/s and achieved HBM GB/s (% of peak), 2^28 u32 key-value radix sort",
        "value": round(gkeys, 4),
        "unit": "Gkeys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_untimed": round(ms_per_step_untimed, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16" if w["kind"] == "rows" else ("u64" if w.get("key_bytes", 4) == 8 else "u32"),
        "data": "synthetic",
        "config": {"workload": w["desc"], "name": name, "n": n_keys, "digit_bits": w["b"],
                   "passes": launches_per_sort, "scan": args.scan,
                   **({"lib": os.path.basename(args.lib)} if args.lib else {})},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(name) if args.scan == "lookback" and args.lib is None else None,
            "kernel": "resident_sort_kernel (whole row, all passes in LDS)" if resident
                      else "sweep_kernel (one LSD pass)",
            "bytes_per_launch": bytes_sort // max(launches_per_sort, 1),
            "avg_launch_ms": round(sweep_ms, 4),
        },
        "per_kernel_ms": ({"resident_sort": round(sweep_ms, 4)} if resident else
                          {"clear": round(clear_ms, 4), "histogram": round(hist_ms, 4),
                           "sweep_per_pass": round(sweep_ms, 4)}),
        "hbm_gbs_per_pass": round(achieved, 1),
        "copy_probe_gbs": round(copy_gbs, 1),
        "frac_of_copy": round(achieved / copy_gbs, 4),
    }
    del ws, copy_pair
    torch.cuda.empty_cache()
    if name == HEADLINE and not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
