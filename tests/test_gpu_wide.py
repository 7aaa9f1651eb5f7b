"""GPU parity of the wide sweep (64-bit look-back words and 64-bit store
addresses) against the CPU oracle, element for element, tolerance 0.

A row takes the wide sweep by itself from 2^30 four-byte keys and from 2^29
eight-byte keys or row-sort elements.  The `wide_from` option sends shorter
rows there too, so every wide instantiation a caller can reach -- each key
kind, payload kind, digit width and scan strategy -- is compared with the
oracle at small sizes that still span several tiles and a ragged last tile.
Two sorts then run the wide sweep at its real size: 2^29 + 12,345 fp64 keys
with a u32 payload, and one fp16 row of 2^29 + 12,345 elements with its int64
column index (the 2^30 + 12,345 u32 pairs are in test_gpu_parity.py)."""
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


def assert_same(got, exp, what):
    if not np.array_equal(got, exp):
        bad = np.nonzero(got != exp)[0]
        raise AssertionError(f"{what}: {bad.size} mismatches, first at {bad[0]}: got {got[bad[0]]}, "
                             f"expected {exp[bad[0]]}")


def u32_gpu(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(a.view(np.int32).copy()).cuda()


def u32_np(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


def wide(**kw):
    return lrs.SortOptions(wide_from=1, **kw)


# ---------------------------------------------------- 32-bit keys, forced

@pytest.mark.parametrize("scan", ["lookback", "reduce-then-scan"])
@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_wide_u32_keys_and_pairs(b, scan):
    n = 40_003  # three 15,360-key tiles, the last one ragged
    keys = workloads.random_u32(12_000 + b, n)
    keys[::4] &= np.uint32(0x0F0F0F0F)  # ties in every digit
    vals = workloads.random_u32(12_100 + b, n)
    log(f"wide u32 n={n} b={b} {scan}")
    opt = wide(scan=scan)
    ek, ev = oracle.radix_sort_pairs(keys, vals, 0, 32, b)
    ko, vo = lrs.radix_sort_pairs(u32_gpu(keys), u32_gpu(vals), 0, 32, b, options=opt)
    assert_same(u32_np(ko), ek, "pairs keys")
    assert_same(u32_np(vo), ev, "pairs values")
    assert_same(u32_np(lrs.radix_sort_keys(u32_gpu(keys), 0, 32, b, options=opt)), ek, "keys only")


@pytest.mark.parametrize("scan", ["lookback", "reduce-then-scan"])
@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_wide_x32_keys_and_pairs(b, scan):
    # signed, float and descending keys: the two-mask key transform
    n = 33_337
    x = workloads.normal_f64(12_200 + b, n).astype(np.float32)
    x[::3] = np.round(x[::3])
    bits = x.view(np.uint32).copy()
    vals = np.arange(n, dtype=np.uint32)
    opt = wide(scan=scan)
    for key_type, desc in (("f32", False), ("i32", True), ("u32", True)):
        log(f"wide {key_type} desc={desc} n={n} b={b} {scan}")
        kt = u32_gpu(bits)
        if key_type == "f32":
            kt = kt.view(torch.float32)
        ek, ev = oracle.radix_sort_typed(bits, vals, key_type, desc, 0, 32, b)
        ko, vo = lrs.radix_sort_pairs_typed(kt, u32_gpu(vals), desc, key_type, 0, 32, b, options=opt)
        assert_same(u32_np(ko), ek, f"{key_type} pairs keys")
        assert_same(u32_np(vo), ev, f"{key_type} pairs values")
        ko = lrs.radix_sort_keys_typed(kt, desc, key_type, 0, 32, b, options=opt)
        assert_same(u32_np(ko), ek, f"{key_type} keys only")


def test_wide_prefix_from_keys_and_windows():
    """The wide kernel's fallback that counts a tile's prefix from the keys,
    and narrower bit windows."""
    n = 61_441  # four full tiles and one of a single key
    keys = workloads.random_u32(12_300, n) & workloads.random_u32(12_301, n)
    vals = np.arange(n, dtype=np.uint32)
    for begin, end, b, opt in ((0, 32, 8, wide(prefix_from_keys=True)), (3, 30, 4, wide(spin_limit=1)),
                               (5, 17, 2, wide(prefix_from_keys=True))):
        log(f"wide fallback n={n} [{begin},{end}) b={b}")
        ek, ev = oracle.radix_sort_pairs(keys, vals, begin, end, b)
        ko, vo = lrs.radix_sort_pairs(u32_gpu(keys), u32_gpu(vals), begin, end, b, options=opt)
        assert_same(u32_np(ko), ek, "keys")
        assert_same(u32_np(vo), ev, "values")


# ---------------------------------------------------- 64-bit keys, forced

@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_wide_64bit_keys_and_pairs(b):
    n = 20_011  # three 8,192-key tiles, the last one ragged
    hi = workloads.random_u32(12_400 + b, n).astype(np.uint64)
    lo = workloads.random_u32(12_500 + b, n).astype(np.uint64)
    bits = (hi << np.uint64(32)) | lo
    bits[1::3] %= np.uint64(97)  # ties
    vals = np.arange(n, dtype=np.uint32) * np.uint32(2654435761)
    vt = u32_gpu(vals)
    for key_type, desc in (("u64", False), ("i64", True), ("f64", False), ("u64", True)):
        kt = torch.from_numpy(bits.view(np.int64).copy()).cuda()
        if key_type == "f64":
            kt = kt.view(torch.float64)
        log(f"wide {key_type} desc={desc} n={n} b={b}")
        ek, ev = oracle.radix_sort_typed(bits, vals, key_type, desc, 0, 64, b)
        ko, vo = lrs.radix_sort_pairs_typed(kt, vt, desc, key_type, 0, 64, b, options=wide())
        assert_same(ko.view(torch.int64).cpu().numpy().view(np.uint64), ek, f"{key_type} pairs keys")
        assert_same(u32_np(vo), ev, f"{key_type} pairs values")
        ko = lrs.radix_sort_keys_typed(kt, desc, key_type, 0, 64, b, options=wide())
        assert_same(ko.view(torch.int64).cpu().numpy().view(np.uint64), ek, f"{key_type} keys only")


# --------------------------------------------------------- row sorts, forced

@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_wide_rows(b):
    rows, n = 3, 20_011
    bits = workloads.fp16_normal_bits(12_600 + b, rows * n).reshape(rows, n)
    bits[:, ::7] = np.uint16(0x3C00)  # ties (1.0)
    bits[:, 5::31] = np.uint16(0x8000)  # -0
    payload = workloads.random_u32(12_700 + b, rows * n).reshape(rows, n)
    for dtype, desc in (("fp16", False), ("bf16", True)):
        log(f"wide rows {rows}x{n} {dtype} desc={desc} b={b}")
        x = torch.from_numpy(bits.view(np.int16).copy()).cuda().view(
            torch.float16 if dtype == "fp16" else torch.bfloat16)
        ev, ei = oracle.segmented_row_sort(bits, desc, b)
        vo, io = lrs.segmented_row_sort(x, desc, b, options=wide())
        assert_same(vo.view(torch.int16).cpu().numpy().view(np.uint16).ravel(), ev.ravel(), "values")
        assert_same(io.cpu().numpy().ravel(), ei.ravel(), "indices")
        vo, po = lrs.segmented_row_sort_pairs(x, u32_gpu(payload.ravel()).reshape(rows, n), desc, b,
                                              options=wide())
        assert_same(vo.view(torch.int16).cpu().numpy().view(np.uint16).ravel(), ev.ravel(), "pair values")
        assert_same(u32_np(po).ravel(), np.take_along_axis(payload, ei, axis=1).ravel(), "payload")


# ------------------------------------------------------------- real sizes

@pytest.mark.timeout(900)
def test_wide_f64_pairs_past_2p29():
    """2^29 + 12,345 fp64 keys: byte offsets of the keys pass 2^32, so the
    row takes the wide sweep without any option."""
    n = (1 << 29) + 12_345
    log(f"f64 pairs n={n}: generating")
    block = workloads.normal_f64(12_800, 1 << 20)
    block[::5] = np.round(block[::5] * 8) / 8  # ties
    x = np.tile(block, n // block.size + 1)[:n]
    x *= 1.0 + (np.arange(n) % 4099) * 2.0 ** -40  # copies differ in their low bits
    bits = x.view(np.uint64)
    vals = np.arange(n, dtype=np.uint32)
    kt = torch.from_numpy(x).cuda()
    vt = u32_gpu(vals)
    log("f64 pairs: sorting on the GPU")
    ko, vo = lrs.radix_sort_pairs_typed(kt, vt, False)
    torch.cuda.synchronize()
    gk = ko.view(torch.int64).cpu().numpy().view(np.uint64)
    gv = u32_np(vo)
    del kt, vt, ko, vo
    torch.cuda.empty_cache()
    log("f64 pairs: oracle")
    ek, ev = oracle.radix_sort_typed(bits, vals, "f64", False, 0, 64, 8)
    assert_same(gk, ek, "keys")
    assert_same(gv, ev, "values")


@pytest.mark.timeout(900)
def test_wide_fp16_row_past_2p29():
    """One fp16 row of 2^29 + 12,345 elements, 4-bit digits: its int64 index
    passes 2^32 bytes, so every pass (index made, u32 index, int64 index out)
    takes the wide sweep without any option."""
    n = (1 << 29) + 12_345
    log(f"fp16 row n={n}: generating")
    block = workloads.fp16_normal_bits(12_900, 1 << 20)
    bits = np.tile(block, n // block.size + 1)[:n].reshape(1, n)
    x = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.float16)
    log("fp16 row: sorting on the GPU")
    vo, io = lrs.segmented_row_sort(x, False, 4)
    torch.cuda.synchronize()
    gv = vo.view(torch.int16).cpu().numpy().view(np.uint16)
    gi = io.cpu().numpy()
    del x, vo, io
    torch.cuda.empty_cache()
    log("fp16 row: oracle")
    ev, ei = oracle.segmented_row_sort(bits, False, 4)
    assert_same(gv.ravel(), ev.ravel(), "values")
    assert_same(gi.ravel(), ei.ravel(), "indices")
