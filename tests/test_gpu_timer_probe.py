"""GPU: the measurement utilities the library exports beside the sorts.

The kernel timer (radix_sort_timer_*) must count every kernel a timed call
enqueues under its kind, give each a positive time, empty itself on read and
leave the sort's result exact (against the oracle), and be refused (with
nothing enqueued) on a stream that is being captured into a graph.  The copy probe
(radix_sort_copy_probe) must copy exactly the bytes asked for, tails of fewer
than 16 bytes included, write nothing past them, and reject misaligned or
overlapping buffers before launching anything."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

lrs = pytest.importorskip("lsd_radix_sort_amd")


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lrs.load_library()
    return torch.device("cuda:0")


def to_gpu_u32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(a.view(np.int32).copy()).cuda()


def to_np_u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def rows_gpu(bits: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16).copy()).cuda().view(dtype)


def expect_kinds(launches: dict, ms: dict, want: dict):
    """Launch counts per kind exactly as `want` (other kinds 0); a positive
    time for every kind that ran and none for the others."""
    for kind in lrs.KernelTimer.KINDS:
        n = want.get(kind, 0)
        assert launches[kind] == n, f"{kind}: {launches[kind]} launches, expected {n} ({launches})"
        if n:
            assert ms[kind] > 0.0, f"{kind}: no time recorded ({ms})"
        else:
            assert ms[kind] == 0.0, f"{kind}: time without a launch ({ms})"


# ------------------------------------------------------------------ timer

@pytest.mark.parametrize("n,b,want", [
    # several histogram workgroups add into one histogram: a clear first
    ((1 << 20) + 333, 8, {"clear": 1, "histogram": 1, "sweep": 4}),
    # one histogram workgroup stores the counts and clears the look-back words itself
    (16384, 4, {"histogram": 1, "sweep": 8}),
])
def test_timer_counts_lookback_sort(n, b, want):
    log(f"timer: pairs n={n} b={b}")
    keys = workloads.random_u32(7100 + b, n)
    vals = np.arange(n, dtype=np.uint32)
    timer = lrs.KernelTimer()
    try:
        kt, vt = to_gpu_u32(keys), to_gpu_u32(vals)
        with timer:
            ko, vo = lrs.radix_sort_pairs(kt, vt, 0, 32, b, options=lrs.SortOptions(timer=timer))
        expect_kinds(timer.launches, timer.ms, want)
        ek, ev = oracle.radix_sort_pairs(keys, vals, 0, 32, b)
        assert np.array_equal(to_np_u32(ko), ek) and np.array_equal(to_np_u32(vo), ev)
        ms, launches = timer.read()  # emptied by the read at exit
        assert all(v == 0 for v in launches.values()) and all(v == 0.0 for v in ms.values())
    finally:
        timer.close()


def test_timer_counts_reduce_then_scan():
    # per pass one count-and-scan slot (two kernels) and one sweep; no histogram
    # launch and nothing to clear
    n = (1 << 20) + 333
    log(f"timer: reduce-then-scan pairs n={n}")
    keys = workloads.random_u32(7200, n)
    vals = np.arange(n, dtype=np.uint32)
    timer = lrs.KernelTimer()
    try:
        with timer:
            ko, vo = lrs.radix_sort_pairs(to_gpu_u32(keys), to_gpu_u32(vals), 0, 32, 8,
                                          options=lrs.SortOptions(scan="reduce-then-scan", timer=timer))
        expect_kinds(timer.launches, timer.ms, {"histogram": 4, "sweep": 4})
        ek, ev = oracle.radix_sort_pairs(keys, vals, 0, 32, 8)
        assert np.array_equal(to_np_u32(ko), ek) and np.array_equal(to_np_u32(vo), ev)
    finally:
        timer.close()


@pytest.mark.parametrize("what", ["keys_1024", "bf16_rows_8x1024", "bf16_rows_64x4096"])
def test_timer_one_launch_sorts(what):
    # whole sorts in one launch: small ones have their launch bracketed by
    # recorded events, larger ones stamped by the dispatch; one resident launch
    # either way, and the result unchanged
    log(f"timer: one-launch sort {what}")
    timer = lrs.KernelTimer()
    try:
        opts = lrs.SortOptions(timer=timer)
        if what == "keys_1024":
            keys = workloads.keys_c1(1024)
            with timer:
                out = lrs.radix_sort_keys(to_gpu_u32(keys), 0, 12, 4, options=opts)
            assert np.array_equal(to_np_u32(out), oracle.radix_sort_keys(keys, 0, 12, 4))
        else:
            rows, cols = (8, 1024) if what == "bf16_rows_8x1024" else (64, 4096)
            bits = workloads.bf16_64level_bits(7300 + rows, rows * cols).reshape(rows, cols)
            with timer:
                vo, io = lrs.segmented_row_sort(rows_gpu(bits, torch.bfloat16), descending=True, digit_bits=8,
                                                options=opts)
            ev, ei = oracle.segmented_row_sort(bits, descending=True, digit_bits=8)
            assert np.array_equal(vo.view(torch.int16).cpu().numpy().view(np.uint16), ev)
            assert np.array_equal(io.cpu().numpy(), ei)
        expect_kinds(timer.launches, timer.ms, {"resident": 1})
    finally:
        timer.close()


def test_timer_accumulates_calls_until_read():
    n = 50000
    keys = workloads.random_u32(7400, n)
    timer = lrs.KernelTimer()
    try:
        opts = lrs.SortOptions(timer=timer)
        timer.read()
        outs = [lrs.radix_sort_keys(to_gpu_u32(keys), 0, 32, 8, options=opts) for _ in range(3)]
        ms, launches = timer.read()
        per_sort = {"histogram": 1, "sweep": 4}
        # a clear only where several histogram workgroups share the count
        assert launches["clear"] in (0, 3)
        for kind, k in per_sort.items():
            assert launches[kind] == 3 * k, (kind, launches)
        expect = oracle.radix_sort_keys(keys, 0, 32, 8)
        for out in outs:
            assert np.array_equal(to_np_u32(out), expect)
    finally:
        timer.close()


# ------------------------------------------------------------- copy probe

@pytest.mark.parametrize("nbytes", [1, 15, 16, 17, 4096 + 7, 3 * (1 << 20) + 5])
def test_copy_probe_copies_exactly(nbytes):
    log(f"copy probe: {nbytes} bytes")
    rng = np.random.default_rng(7500 + nbytes)
    data = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    src = torch.from_numpy(data).cuda()
    dst = torch.full((nbytes + 64,), 0xA5, dtype=torch.uint8, device=src.device)
    timer = lrs.KernelTimer()
    try:
        with timer:
            lrs.copy_probe(src, dst, options=lrs.SortOptions(timer=timer))
        expect_kinds(timer.launches, timer.ms, {"copy": 1})
    finally:
        timer.close()
    got = dst.cpu().numpy()
    assert np.array_equal(got[:nbytes], data)
    assert np.all(got[nbytes:] == 0xA5), "bytes past the copy were written"


def test_copy_probe_rejects_bad_buffers():
    buf = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    dst = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(lrs.RadixSortArgumentError):
        lrs.copy_probe(buf[4:1028], dst)           # source not 16-byte aligned
    with pytest.raises(lrs.RadixSortArgumentError):
        lrs.copy_probe(buf[:1024], dst[4:1028])    # destination not 16-byte aligned
    with pytest.raises(lrs.RadixSortArgumentError):
        lrs.copy_probe(buf[:2048], buf[1024:])     # overlapping
    with pytest.raises(lrs.RadixSortArgumentError):
        lrs.copy_probe(buf[:2048], dst[:1024])     # destination too small
    torch.cuda.synchronize()
    assert int(dst.sum()) == 0, "a rejected copy wrote"


def test_timed_call_refused_during_graph_capture():
    # a timer's events are for eager calls: under capture the timed call is
    # refused before it enqueues anything, while the same call untimed is
    # captured and its replays sort correctly
    n = 100000
    keys = workloads.random_u32(7600, n)
    kin = to_gpu_u32(keys)
    kout = torch.empty_like(kin)
    ws = torch.empty(lrs.radix_sort_workspace_size(n, 0, 32, 8), dtype=torch.uint8, device=kin.device)
    timer = lrs.KernelTimer()
    try:
        lrs.radix_sort_keys(kin, 0, 32, 8, out=kout, workspace=ws)  # eager call before capture
        torch.cuda.synchronize()
        kout.zero_()
        refused = None
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            try:
                lrs.radix_sort_keys(kin, 0, 32, 8, out=kout, workspace=ws, options=lrs.SortOptions(timer=timer))
            except lrs.RadixSortArgumentError as e:
                refused = e
            lrs.radix_sort_keys(kin, 0, 32, 8, out=kout, workspace=ws)
        torch.cuda.synchronize()
        assert refused is not None and refused.status == 10, f"timed call under capture: {refused!r}"
        ms, launches = timer.read()
        assert all(v == 0 for v in launches.values()), "the refused call recorded launches"
        expect = oracle.radix_sort_keys(keys, 0, 32, 8)
        for rep in range(3):
            kout.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(to_np_u32(kout), expect), f"replay {rep}"
        # and the timer still works eagerly afterwards
        with timer:
            lrs.radix_sort_keys(kin, 0, 32, 8, out=kout, workspace=ws, options=lrs.SortOptions(timer=timer))
        assert timer.launches["sweep"] == 4
        assert np.array_equal(to_np_u32(kout), expect)
    finally:
        timer.close()
