"""Host logic of bench.py (no GPU): the one-GPU refusal, the algorithmic byte
counts the roofline divides by, and the workload table."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_headline_sweep_bytes():
    # 4 passes, each reading and writing a 4-byte key and a 4-byte value per pair
    w = bench.WORKLOADS[bench.HEADLINE]
    assert (w["kind"], w["n"], w["end_bit"], w["b"]) == ("pairs", 1 << 28, 32, 8)
    assert bench.sweep_bytes(w) == 4 * 16 * (1 << 28)


def test_keys_only_sweep_bytes():
    assert bench.sweep_bytes(bench.WORKLOADS["c2_keys_4m_4bit"]) == 8 * 8 * (1 << 22)
    assert bench.sweep_bytes(bench.WORKLOADS["c2_keys_4m_8bit"]) == 4 * 8 * (1 << 22)
    assert bench.sweep_bytes(bench.WORKLOADS["i32_keys_2p28_asc"]) == 4 * 8 * (1 << 28)


def test_wide_key_sweep_bytes():
    # 8-byte keys with a 4-byte value: 24 B per pair per pass, 8 passes of 8 bits
    assert bench.sweep_bytes(bench.WORKLOADS["f64_pairs_2p27_asc"]) == 8 * 24 * (1 << 27)


def test_row_sort_bytes():
    # fp16 rows of 65536, 4 passes, key << 16 | column as one u32 word between
    # passes: 2 in + 4 out, then 4 + 4 twice, then 4 in + 2+8 out = 36 B per element
    w = bench.WORKLOADS["c4_fp16_1024x65536_asc"]
    assert bench.sweep_bytes(w) == 36 * 1024 * 65536
    # longer rows keep the pattern and a u32 index apart: 2 in + 2+4 out, then
    # 6 + 6 twice, then 6 in + 2+8 out = 48 B per element
    assert bench.sweep_bytes(dict(w, rows=1, cols=200_000)) == 48 * 200_000
    # whole-row sort: the pattern in, the pattern and an int64 index out
    assert bench.resident_bytes(bench.WORKLOADS["c5_bf16_4096x4096_desc"]) == 12 * 4096 * 4096
    assert bench.resident_bytes(bench.WORKLOADS["c1_keys_1k_4bit"]) == 8 * 1024


def test_workload_table_is_complete():
    for name, w in bench.WORKLOADS.items():
        assert w["kind"] in ("keys", "pairs", "rows") and w["b"] in (1, 2, 4, 8), name
        assert w["desc"], name
    assert set(bench.MEASURED_TRAFFIC) <= set(bench.WORKLOADS)
    for name, m in bench.MEASURED_TRAFFIC.items():
        assert set(m) >= {"kernel_sha16", "bytes_per_launch", "source"}, name
        assert len(m["kernel_sha16"]) == 16 and m["bytes_per_launch"] > 0, name


def test_traffic_is_tied_to_the_kernel_sources(monkeypatch):
    """A counter figure is reported only for the kernel sources it was taken
    on; after any change to them the line says null until it is re-measured."""
    sha = bench.kernel_sources_sha16()
    monkeypatch.setattr(bench, "MEASURED_TRAFFIC", {"x": {"kernel_sha16": sha, "bytes_per_launch": 123,
                                                          "source": "test"}})
    assert bench.measured_traffic("x") == 123
    assert bench.measured_traffic("y") is None
    monkeypatch.setattr(bench, "MEASURED_TRAFFIC", {"x": {"kernel_sha16": "0" * 16, "bytes_per_launch": 123,
                                                          "source": "test"}})
    assert bench.measured_traffic("x") is None


def test_tile_trace_report_phases_and_placement():
    # two launches of 32 tiles, records built by hand: phase k of every tile
    # lasts k + 1 ticks of the 100 MHz clock (10 ns), launch 1 starts 1000
    # ticks later, tile t of launch 0 ran on XCD (t // 16) % 8 (the dealing of
    # chunks of 16), tile 5 of it on a wrong one
    import numpy as np

    tiles, sweeps = 32, 2
    rec = np.zeros((sweeps * tiles, 12), dtype=np.int64)
    for L in range(sweeps):
        for t in range(tiles):
            r = rec[L * tiles + t]
            r[0] = 1000 * L + t
            for k in range(6):
                r[k + 1] = r[k] + (k + 1)
            r[7] = (t // 16) % 8
            r[8] = (t % 4) << 8 | (t % 2) << 13   # CU, shader engine
            r[9] = 8 * t + (t // 16) % 8           # a workgroup index on that XCD
            r[10] = 3
            r[11] = 0
    rec[5, 7] = 7
    out = bench.tile_trace_report(rec, sweeps, 100.0, 0.5)
    assert out["tiles_per_launch"] == tiles and len(out["launches"]) == sweeps
    for launch in out["launches"]:
        assert launch["phase_median_us"] == [0.01, 0.02, 0.03, 0.04, 0.05, 0.06]
        assert launch["tile_us"] == 0.21
        assert launch["span_us"] == round((31 + 21) / 100.0, 1)
    assert out["tiles_on_dealt_xcd"] == tiles - 1
    # tile 5 reported XCD 7, not its workgroup index mod 8
    assert out["workgroup_xcd_is_index_mod_8"] == tiles - 1
    assert out["lookback_predecessors_median"] == 3.0 and out["lookback_polls_median"] == 0.0
