"""GPU parity: the HIP library against the CPU oracle, element for element,
tolerance 0 (keys, payloads and indices), on the seeded inputs of the five
workloads and on edge cases.  At the 2^28-pair size the result is checked by
the properties that characterise the unique stable sort (sorted, a permutation
carried by the index payload, ties in input order) computed on the GPU with
torch, plus oracle positions of sampled elements computed one by one."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import window

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


def to_gpu(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32).copy()).cuda()
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).cuda()
    return torch.from_numpy(a.copy()).cuda()


def to_np_u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def gpu_keys(keys, begin, end, b, options=None):
    kt = to_gpu(keys)
    out = lrs.radix_sort_keys(kt, begin, end, b, options=options)
    torch.cuda.synchronize()
    assert np.array_equal(to_np_u32(kt), keys), "input was written"
    return to_np_u32(out)


def gpu_pairs(keys, vals, begin, end, b, options=None):
    kt, vt = to_gpu(keys), to_gpu(vals)
    ko, vo = lrs.radix_sort_pairs(kt, vt, begin, end, b, options=options)
    torch.cuda.synchronize()
    assert np.array_equal(to_np_u32(kt), keys) and np.array_equal(to_np_u32(vt), vals), "input was written"
    return to_np_u32(ko), to_np_u32(vo)


def assert_same(got, exp, what):
    if not np.array_equal(got, exp):
        bad = np.nonzero(got != exp)[0]
        raise AssertionError(f"{what}: {bad.size} mismatches, first at {bad[0]}: got {got[bad[0]]}, "
                             f"expected {exp[bad[0]]}")


# ----------------------------------------------------------------- u32 keys

@pytest.mark.parametrize("b", [4, 1, 2, 8])
def test_c1_1024_keys_12_bits(b):
    keys = workloads.keys_c1()
    log(f"c1 b={b}")
    exp = oracle.radix_sort_keys(keys, 0, 12, b)
    assert_same(gpu_keys(keys, 0, 12, b), exp, f"c1 b={b}")


@pytest.mark.parametrize("b", [4, 8])
def test_c2_4m_keys(b):
    keys = workloads.keys_c2()
    log(f"c2 b={b}")
    exp = oracle.radix_sort_keys(keys, 0, 32, b)
    assert_same(exp, np.sort(keys), "oracle vs np.sort")
    assert_same(gpu_keys(keys, 0, 32, b), exp, f"c2 b={b}")


@pytest.mark.parametrize("dist", ["uniform", "and3"])
def test_c3_pairs_reduced_size(dist):
    n = 1 << 22
    keys, vals = workloads.pairs_c3(n, dist)
    log(f"c3 reduced n={n} {dist}")
    ek, ev = oracle.radix_sort_pairs(keys, vals, 0, 32, 8)
    gk, gv = gpu_pairs(keys, vals, 0, 32, 8)
    assert_same(gk, ek, "keys")
    assert_same(gv, ev, "values")


@pytest.mark.parametrize("b,dist", [(8, "uniform"), (4, "and3")])
def test_large_tile_configuration(b, dist):
    # enough elements for the largest sweep tile (at least 256 tiles of 15360)
    n = 15_000_007
    keys = workloads.random_u32(4000 + b, n)
    if dist == "and3":
        keys &= workloads.random_u32(4100, n) & workloads.random_u32(4200, n)
    vals = np.arange(n, dtype=np.uint32)
    log(f"large tiles n={n} b={b} {dist}")
    ek, ev = oracle.radix_sort_pairs(keys, vals, 0, 32, b)
    gk, gv = gpu_pairs(keys, vals, 0, 32, b)
    assert_same(gk, ek, "keys")
    assert_same(gv, ev, "values")
    assert_same(gpu_keys(keys, 0, 32, b), ek, "keys only")


@pytest.mark.parametrize("b,dist", [(8, "and3"), (4, "uniform")])
def test_mid_tile_configuration(b, dist):
    # too few elements for 256 tiles of 15360, enough for 256 of 8192
    n = 3_000_017
    keys = workloads.random_u32(4300 + b, n)
    if dist == "and3":
        keys &= workloads.random_u32(4400, n) & workloads.random_u32(4500, n)
    vals = np.arange(n, dtype=np.uint32)
    log(f"mid tiles n={n} b={b} {dist}")
    ek, ev = oracle.radix_sort_pairs(keys, vals, 0, 32, b)
    gk, gv = gpu_pairs(keys, vals, 0, 32, b)
    assert_same(gk, ek, "keys")
    assert_same(gv, ev, "values")
    assert_same(gpu_keys(keys, 0, 32, b), ek, "keys only")


@pytest.mark.parametrize("n", [15_360 * 260, 15_360 * 260 + 1, 8_192 * 300, 8_192 * 300 + 1])
def test_exact_tile_multiples(n):
    # every tile full (each tile takes the copy of the loops without bounds
    # tests), and the same plus a last tile holding one element
    keys = workloads.random_u32(4600 + n % 7, n)
    keys[::3] &= 0xFF00FF00  # ties in alternate digits
    vals = workloads.random_u32(4700, n)
    log(f"exact tile multiple n={n}")
    ek, ev = oracle.radix_sort_pairs(keys, vals, 0, 32, 8)
    gk, gv = gpu_pairs(keys, vals, 0, 32, 8)
    assert_same(gk, ek, "keys")
    assert_same(gv, ev, "values")
    assert_same(gpu_keys(keys, 0, 32, 8), ek, "keys only")
    ek4 = oracle.radix_sort_keys(keys, 4, 28, 4)
    assert_same(gpu_keys(keys, 4, 28, 4), ek4, "keys only, bits 4-27, b=4")
    ei, _ = oracle.radix_sort_typed(keys, None, "i32", False)
    gi = lrs.radix_sort_keys_typed(to_gpu(keys))  # int32 tensor: signed keys
    torch.cuda.synchronize()
    assert_same(to_np_u32(gi), ei, "int32 keys only")


@pytest.mark.parametrize("b", [4, 8])
def test_keys_at_unaligned_addresses(b):
    """Keys and rows that start off a 16-byte boundary: the per-thread runs of
    narrow-digit sweeps are then read one element at a time, not as vectors."""
    n = 3_000_017
    keys = workloads.random_u32(4800 + b, n + 3)
    base = to_gpu(keys)
    for off in (1, 2, 3):
        log(f"unaligned keys offset={off} b={b}")
        kt = base[off:]
        assert kt.data_ptr() % 16 != 0
        out = lrs.radix_sort_keys(kt, 0, 32, b)
        torch.cuda.synchronize()
        assert_same(to_np_u32(out), oracle.radix_sort_keys(keys[off:], 0, 32, b), f"offset {off}")
    rows, m = 3, 40_000
    bits = workloads.fp16_normal_bits(4900 + b, rows * m + 5)
    t = to_gpu(bits).view(torch.float16)
    for off in (1, 3, 5):
        x = t[off:off + rows * m].view(rows, m)
        assert x.data_ptr() % 16 != 0
        ev, ei = oracle.segmented_row_sort(bits[off:off + rows * m].reshape(rows, m), False, b)
        vo, io = lrs.segmented_row_sort(x, False, b)
        torch.cuda.synchronize()
        assert_same(vo.view(torch.int16).cpu().numpy().view(np.uint16).ravel(), ev.ravel(), f"rows offset {off}")
        assert_same(io.cpu().numpy().ravel(), ei.ravel(), f"rows offset {off} idx")


def test_pass_by_pass_states():
    # the state after p passes is the stable sort by the low p*b bits of the window
    n = 300_001
    keys = workloads.random_u32(31, n) & workloads.random_u32(32, n)
    vals = np.arange(n, dtype=np.uint32)
    for b, begin in ((8, 0), (4, 3), (1, 20), (2, 5)):
        P = oracle.num_passes(begin, 32, b)
        for p in range(1, P + 1):
            end = min(32, begin + p * b)
            ek, ev = oracle.radix_sort_pairs(keys, vals, begin, end, b)
            gk, gv = gpu_pairs(keys, vals, begin, end, b)
            assert_same(gk, ek, f"b={b} begin={begin} passes={p} keys")
            assert_same(gv, ev, f"b={b} begin={begin} passes={p} values")


def test_fuzz_sizes_windows_widths():
    rng = np.random.default_rng(2024)
    sizes = [1, 2, 63, 64, 65, 255, 4095, 4096, 4097, 8191, 8192, 8193, 12289, 65537, 100_003]
    for trial, n in enumerate(sizes + [int(x) for x in rng.integers(1, 200_000, 10)]):
        keys = workloads.random_u32(700 + trial, n)
        if trial % 2:
            keys &= workloads.random_u32(900 + trial, n)
        begin = int(rng.integers(0, 31))
        end = int(rng.integers(begin + 1, 33))
        b = int(rng.choice([1, 2, 4, 8]))
        vals = workloads.random_u32(1100 + trial, n)
        ek, ev = oracle.radix_sort_pairs(keys, vals, begin, end, b)
        gk, gv = gpu_pairs(keys, vals, begin, end, b)
        assert_same(gk, ek, f"n={n} [{begin},{end}) b={b} keys")
        assert_same(gv, ev, f"n={n} [{begin},{end}) b={b} values")
        assert_same(gpu_keys(keys, begin, end, b), ek, f"n={n} keys-only")


def test_degenerate_inputs():
    n = 50_000
    cases = {
        "all_equal": np.full(n, 0xDEADBEEF, dtype=np.uint32),
        "all_max": np.full(n, 0xFFFFFFFF, dtype=np.uint32),
        "all_zero": np.zeros(n, dtype=np.uint32),
        "sorted": np.arange(n, dtype=np.uint32) * np.uint32(977),
        "reversed": (np.arange(n, dtype=np.uint32) * np.uint32(977))[::-1].copy(),
        "two_values": np.where(workloads.random_u32(5, n) & 1, 0xFFFFFFFF, 0).astype(np.uint32),
    }
    vals = np.arange(n, dtype=np.uint32)
    for name, keys in cases.items():
        for b in (1, 8):
            ek, ev = oracle.radix_sort_pairs(keys, vals, 0, 32, b)
            gk, gv = gpu_pairs(keys, vals, 0, 32, b)
            assert_same(gk, ek, f"{name} b={b}")
            assert_same(gv, ev, f"{name} b={b} values")


def test_empty_input():
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    assert lrs.radix_sort_keys(e).numel() == 0
    k, v = lrs.radix_sort_pairs(e, e.clone())
    assert k.numel() == 0 and v.numel() == 0
    x = torch.empty(0, 16, dtype=torch.float16, device="cuda")
    vs, ix = lrs.segmented_row_sort(x)
    assert vs.shape == (0, 16) and ix.shape == (0, 16)


def test_digit_histograms():
    keys = workloads.pairs_c3(1 << 20, "and3")[0]
    kt = to_gpu(keys)
    for begin, end, b in ((0, 32, 8), (0, 32, 4), (0, 12, 4), (3, 30, 1), (5, 17, 2), (1, 30, 4), (7, 32, 2)):
        h = lrs.radix_sort_digit_histograms(kt, begin, end, b)
        torch.cuda.synchronize()
        exp = oracle.all_pass_histograms(keys, begin, end, b)
        assert np.array_equal(h.cpu().numpy().astype(np.uint64), exp), (begin, end, b)


def test_validation_with_real_buffers():
    n = 100_000
    k = torch.zeros(n, dtype=torch.int32, device="cuda")
    o = torch.empty_like(k)
    with pytest.raises(ValueError):
        lrs.radix_sort_keys(k, 0, 32, 3)
    with pytest.raises(ValueError):
        lrs.radix_sort_keys(k, 0, 33, 8)
    with pytest.raises(ValueError):
        lrs.radix_sort_keys(k, out=k)
    ws = torch.empty(lrs.radix_sort_workspace_size(n, 0, 32, 8), dtype=torch.uint8, device="cuda")
    lib = lrs.load_library()
    st = lib.radix_sort_keys(k.data_ptr(), o.data_ptr(), n, 0, 32, 8, ws.data_ptr(), ws.numel() - 1, None, None)
    assert st == 6
    bad = lrs._Options(9, 0, 0, 0, None)
    st = lib.radix_sort_keys(k.data_ptr(), o.data_ptr(), n, 0, 32, 8, ws.data_ptr(), ws.numel(), None,
                             __import__("ctypes").byref(bad))
    assert st == 10
    with pytest.raises(ValueError):  # a workspace one byte short, caught by the binding
        lrs.radix_sort_keys(k, workspace=ws[:-1])
    with pytest.raises(ValueError):  # an output of the wrong length
        lrs.radix_sort_keys(k, out=o[:-1])
    x = torch.zeros(4, 64, dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        lrs.segmented_row_sort(x, digit_bits=5)


# -------------------------------------------------------------- full size

def _u32_to_i64(t):
    return t.view(torch.int32).to(torch.int64) & 0xFFFFFFFF


@pytest.mark.timeout(600)
@pytest.mark.parametrize("n,strategy", [((1 << 29) + 12_345, "lookback"), ((1 << 29) + 12_345, "reduce-then-scan"),
                                        ((1 << 30) + 12_345, "lookback")])
def test_rows_past_2p29_and_2p30_elements(n, strategy):
    """Beyond 2^29 u32 pairs the byte offsets of the 32-bit sweep pass 2^31
    (with either scan strategy); from 2^30 the row takes 64-bit look-back
    words and 64-bit store addresses.  Compared element for element with the
    oracle."""
    log(f"long row n={n}: generating")
    # a seeded 2^20-key block repeated, each copy scrambled by its index
    block = workloads.random_u32(4800, 1 << 20)
    keys = np.tile(block, n // block.size + 1)[:n]
    keys ^= np.arange(n, dtype=np.uint32) * np.uint32(0x9E3779B1)
    keys[1::2] &= np.uint32(0xF0F0F0F0)  # half the keys: ties in every digit
    vals = np.arange(n, dtype=np.uint32)
    kt, vt = to_gpu(keys), to_gpu(vals)
    log(f"long row: sorting on the GPU ({strategy})")
    ko, vo = lrs.radix_sort_pairs(kt, vt, 0, 32, 8, options=lrs.SortOptions(scan=strategy))
    torch.cuda.synchronize()
    del kt, vt
    gk, gv = to_np_u32(ko), to_np_u32(vo)
    del ko, vo
    torch.cuda.empty_cache()
    log("long row: oracle")
    ek, ev = oracle.radix_sort_pairs(keys, vals, 0, 32, 8)
    assert_same(gk, ek, "keys")
    assert_same(gv, ev, "values")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dist", ["uniform", "and3"])
def test_c3_full_size_against_oracle(dist):
    """The 2^28-pair workloads on their seeded inputs, in the launch
    configuration the benchmark times: every key and value equal to the
    oracle's, plus the properties that characterise the stable sort (checked
    on the GPU first, so a failure names what broke)."""
    n = 1 << 28
    log(f"c3 full n={n} {dist}: generating")
    keys, vals = workloads.pairs_c3(n, dist)
    kt, vt = to_gpu(keys), to_gpu(vals)
    log("c3 full: sorting")
    ko, vo = lrs.radix_sort_pairs(kt, vt, 0, 32, 8)
    torch.cuda.synchronize()
    log("c3 full: checking properties")
    k64 = _u32_to_i64(ko)
    idx = _u32_to_i64(vo)
    assert bool((k64[1:] >= k64[:-1]).all()), "not sorted"
    seen = torch.zeros(n, dtype=torch.bool, device="cuda")
    seen[idx] = True
    assert bool(seen.all()), "values are not a permutation"
    del seen
    assert bool((_u32_to_i64(kt)[idx] == k64).all()), "key/value mismatch"
    ties = k64[1:] == k64[:-1]
    assert bool(((idx[1:] > idx[:-1]) | ~ties).all()), "unstable"
    del ties, k64
    gk, gv = to_np_u32(ko), to_np_u32(vo)
    assert np.array_equal(to_np_u32(kt), keys), "input was written"
    del kt, vt, ko, vo
    torch.cuda.empty_cache()
    log("c3 full: oracle")
    ek, ev = oracle.radix_sort_pairs(keys, vals, 0, 32, 8)
    assert_same(gk, ek, "keys")
    assert_same(gv, ev, "values")


# -------------------------------------------------------------- segmented

def gpu_rows(bits: np.ndarray, dtype: str, descending: bool, b: int, options=None):
    t = to_gpu(bits).view(torch.float16 if dtype == "fp16" else torch.bfloat16)
    vo, io = lrs.segmented_row_sort(t, descending, b, options=options)
    torch.cuda.synchronize()
    assert np.array_equal(t.view(torch.int16).cpu().numpy().view(np.uint16), bits), "input was written"
    return vo.view(torch.int16).cpu().numpy().view(np.uint16), io.cpu().numpy()


def test_c4_fp16_1024x65536_ascending():
    bits = workloads.matrix_c4()
    log("c4 oracle")
    ev, ei = oracle.segmented_row_sort(bits, False, 4)
    log("c4 gpu")
    gv, gi = gpu_rows(bits, "fp16", False, 4)
    assert_same(gv.ravel(), ev.ravel(), "c4 values")
    assert_same(gi.ravel(), ei.ravel(), "c4 indices")


def test_c5_bf16_4096x4096_descending():
    bits = workloads.matrix_c5()
    log("c5 oracle")
    ev, ei = oracle.segmented_row_sort(bits, True, 8)
    log("c5 gpu")
    gv, gi = gpu_rows(bits, "bf16", True, 8)
    assert_same(gv.ravel(), ev.ravel(), "c5 values")
    assert_same(gi.ravel(), ei.ravel(), "c5 indices")


@pytest.mark.parametrize("rows,n", [(1, 1), (3, 7), (4, 1000), (2, 2048), (5, 4095), (2, 4097), (3, 8192),
                                     (3, 8193), (7, 12345), (3, 65535), (2, 65536), (2, 65537), (1, 70000),
                                     (300, 33), (2, 200_000)])
@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_rows_ragged_shapes(rows, n, b):
    bits = workloads.fp16_normal_bits(rows * 131 + n, rows * n).reshape(rows, n)
    bits[:, ::17] = np.uint16(0x8000)  # -0
    bits[:, 5::19] = np.uint16(0x0000)  # +0
    bits[:, 3::23] = np.uint16(0x7E00)  # NaN
    bits[:, 7::29] = np.uint16(0xFC00)  # -inf
    for desc in (False, True):
        ev, ei = oracle.segmented_row_sort(bits, desc, b)
        for dtype in ("fp16", "bf16"):
            gv, gi = gpu_rows(bits, dtype, desc, b)
            assert_same(gv.ravel(), ev.ravel(), f"rows={rows} n={n} b={b} desc={desc} {dtype}")
            assert_same(gi.ravel(), ei.ravel(), f"rows={rows} n={n} b={b} desc={desc} {dtype} idx")


@pytest.mark.parametrize("rows,n", [(3, 7), (5, 4095), (3, 8192), (3, 8193), (7, 12345), (2, 200_000),
                                     (64, 65536)])
@pytest.mark.parametrize("b", [4, 8])
def test_rows_with_caller_payload(rows, n, b):
    # the payload must land where the oracle's column index says its element went
    bits = workloads.fp16_normal_bits(rows * 977 + n, rows * n).reshape(rows, n)
    bits[:, ::13] = np.uint16(0x8000)
    payload = (workloads.random_u32(rows + 3 * n, rows * n)).reshape(rows, n)
    for desc in (False, True):
        ev, ei = oracle.segmented_row_sort(bits, desc, b)
        expected_pay = np.take_along_axis(payload, ei, axis=1)
        for dtype in ("fp16", "bf16"):
            t = to_gpu(bits).view(torch.float16 if dtype == "fp16" else torch.bfloat16).reshape(rows, n)
            pt = to_gpu(payload.ravel()).reshape(rows, n)
            vo, po = lrs.segmented_row_sort_pairs(t, pt, desc, b)
            torch.cuda.synchronize()
            gv = vo.view(torch.int16).cpu().numpy().view(np.uint16)
            gp = po.cpu().numpy().view(np.uint32)
            assert_same(gv.ravel(), ev.ravel(), f"rows={rows} n={n} b={b} desc={desc} {dtype} values")
            assert_same(gp.ravel(), expected_pay.ravel(), f"rows={rows} n={n} b={b} desc={desc} {dtype} payload")


# ------------------------------------------------ bounded look-back waits

def _wait_options(limit):
    # 0: no waiting at all, every tile counts its prefix from the keys
    return lrs.SortOptions(prefix_from_keys=True) if limit == 0 else lrs.SortOptions(spin_limit=limit)


@pytest.mark.parametrize("limit", [0, 1])
def test_prefix_counted_from_keys(limit):
    """With the look-back wait bounded to `limit` polls (0: no look-back at
    all), tiles count their prefix over the earlier tiles' keys; the sort must
    not change."""
    opt = _wait_options(limit)
    n = 300_001
    keys = workloads.random_u32(9100, n) & workloads.random_u32(9101, n)
    vals = np.arange(n, dtype=np.uint32)
    for b, begin, end in ((8, 0, 32), (4, 3, 30), (1, 0, 5), (2, 7, 18)):
        log(f"limit={limit} n={n} b={b} bits [{begin},{end})")
        ek, ev = oracle.radix_sort_pairs(keys, vals, begin, end, b)
        gk, gv = gpu_pairs(keys, vals, begin, end, b, opt)
        assert_same(gk, ek, "keys")
        assert_same(gv, ev, "values")
        assert_same(gpu_keys(keys, begin, end, b, opt), ek, "keys only")
    rows, m = 5, 20001
    bits = workloads.fp16_normal_bits(9200, rows * m).reshape(rows, m)
    for desc, dtype, b in ((False, "fp16", 4), (True, "bf16", 8)):
        log(f"limit={limit} rows {rows}x{m} {dtype} desc={desc} b={b}")
        ev, ei = oracle.segmented_row_sort(bits, desc, b)
        gv, gi = gpu_rows(bits, dtype, desc, b, opt)
        assert_same(gv.ravel(), ev.ravel(), "row values")
        assert_same(gi.ravel(), ei.ravel(), "row indices")


def test_prefix_counted_from_keys_large_tiles():
    # the largest tile shape, every tile counting its prefix from the keys
    opt = _wait_options(0)
    n = 15_000_007
    keys = workloads.random_u32(9300, n)
    vals = np.arange(n, dtype=np.uint32)
    log(f"limit=0 large tiles n={n}")
    ek, ev = oracle.radix_sort_pairs(keys, vals, 0, 32, 8)
    gk, gv = gpu_pairs(keys, vals, 0, 32, 8, opt)
    assert_same(gk, ek, "keys")
    assert_same(gv, ev, "values")


# ------------------------------------------------ reduce-then-scan strategy

@pytest.fixture
def reduce_then_scan():
    return lrs.SortOptions(scan="reduce-then-scan")


@pytest.mark.parametrize("n", [8193, 300_001, 3_000_017, 15_000_007])
def test_reduce_then_scan_strategy(n, reduce_then_scan):
    # every tile shape; partitions of one tile (small n) and of several (15M)
    keys = workloads.random_u32(9400 + n % 1000, n)
    if n == 3_000_017:
        keys &= workloads.random_u32(9401, n) & workloads.random_u32(9402, n)
    vals = np.arange(n, dtype=np.uint32)
    for b, begin, end in ((8, 0, 32), (4, 0, 32)) if n > 300_001 else ((8, 0, 32), (4, 3, 30), (1, 0, 5), (2, 7, 18)):
        log(f"reduce-then-scan n={n} b={b} bits [{begin},{end})")
        ek, ev = oracle.radix_sort_pairs(keys, vals, begin, end, b)
        gk, gv = gpu_pairs(keys, vals, begin, end, b, reduce_then_scan)
        assert_same(gk, ek, "keys")
        assert_same(gv, ev, "values")
        assert_same(gpu_keys(keys, begin, end, b, reduce_then_scan), ek, "keys only")


def test_reduce_then_scan_typed_keys(reduce_then_scan):
    n = 1_000_003
    bits = workloads.normal_f64(9500, n).astype(np.float32)
    bits[::7] = np.round(bits[::7])
    kt = torch.from_numpy(bits.copy()).cuda()
    vals = np.arange(n, dtype=np.uint32)
    vt = to_gpu(vals)
    for desc in (False, True):
        ko, vo = lrs.radix_sort_pairs_typed(kt, vt, desc, options=reduce_then_scan)
        torch.cuda.synchronize()
        ek, ev = oracle.radix_sort_typed(bits.view(np.uint32), vals, "f32", desc)
        assert_same(ko.view(torch.int32).cpu().numpy().view(np.uint32), ek, f"f32 desc={desc} keys")
        assert_same(to_np_u32(vo), ev, f"f32 desc={desc} values")


def test_scan_strategy_rejects_unknown():
    with pytest.raises(ValueError):
        lrs.SortOptions(scan="bogus")
    k = torch.zeros(100_000, dtype=torch.int32, device="cuda")
    o = torch.empty_like(k)
    ws = torch.empty(lrs.radix_sort_workspace_size(k.numel()), dtype=torch.uint8, device="cuda")
    bad = lrs._Options(3, 0, 0, 0, None)
    lib = lrs.load_library()
    assert lib.radix_sort_keys(k.data_ptr(), o.data_ptr(), k.numel(), 0, 32, 8, ws.data_ptr(), ws.numel(), None,
                               __import__("ctypes").byref(bad)) == 10


def test_two_sorts_in_flight_on_two_streams():
    # independent workspaces: tickets, look-back words and histograms never mix
    n = 3_000_017
    a = workloads.random_u32(9600, n)
    b = workloads.random_u32(9601, n) & workloads.random_u32(9602, n)
    va = np.arange(n, dtype=np.uint32)
    ka, kb, vt = to_gpu(a), to_gpu(b), to_gpu(va)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for rep in range(3):
        with torch.cuda.stream(s1):
            oa = lrs.radix_sort_pairs(ka, vt, 0, 32, 8)
        with torch.cuda.stream(s2):
            ob = lrs.radix_sort_pairs(kb, vt, 0, 32, 4)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    ea = oracle.radix_sort_pairs(a, va, 0, 32, 8)
    eb = oracle.radix_sort_pairs(b, va, 0, 32, 4)
    for (oa, ob) in outs:
        assert_same(to_np_u32(oa[0]), ea[0], "stream 1 keys")
        assert_same(to_np_u32(oa[1]), ea[1], "stream 1 values")
        assert_same(to_np_u32(ob[0]), eb[0], "stream 2 keys")
        assert_same(to_np_u32(ob[1]), eb[1], "stream 2 values")


# ------------------------------------------------------------- graph capture

@pytest.mark.parametrize("n", [1000, 300_000])
def test_hip_graph_capture_and_replay(n):
    """The whole sort (one resident launch, or clear + histogram + sweeps) is
    captured once into a graph and replayed on new inputs copied into the
    captured input buffers; every replay must equal the oracle and eager."""
    kin = torch.empty(n, dtype=torch.int32, device="cuda")
    vin = torch.empty_like(kin)
    kout = torch.empty_like(kin)
    vout = torch.empty_like(kin)
    ws = torch.empty(max(1, lrs.radix_sort_workspace_size(n, 0, 32, 8, True)), dtype=torch.uint8, device="cuda")
    first = workloads.random_u32(8800, n)
    kin.copy_(to_gpu(first))
    vin.copy_(to_gpu(np.arange(n, dtype=np.uint32)))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on the capture stream
        lrs.radix_sort_pairs(kin, vin, 0, 32, 8, keys_out=kout, values_out=vout, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lrs.radix_sort_pairs(kin, vin, 0, 32, 8, keys_out=kout, values_out=vout, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        keys = workloads.random_u32(8801 + rep, n)
        if rep == 1:
            keys &= workloads.random_u32(8900, n) & workloads.random_u32(8901, n)
        vals = workloads.random_u32(8950 + rep, n)
        kin.copy_(to_gpu(keys))
        vin.copy_(to_gpu(vals))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ek, ev = oracle.radix_sort_pairs(keys, vals, 0, 32, 8)
        assert_same(to_np_u32(kout), ek, f"replay {rep} keys")
        assert_same(to_np_u32(vout), ev, f"replay {rep} values")
        # eager call between replays, same buffers
        ko2, vo2 = lrs.radix_sort_pairs(kin, vin, 0, 32, 8)
        torch.cuda.synchronize()
        assert_same(to_np_u32(ko2), ek, f"eager {rep} keys")
        assert_same(to_np_u32(vo2), ev, f"eager {rep} values")


def _replay_checked(make_inputs, load, run, expect, compare, reps=3):
    """Capture run() once, then for each rep: load fresh inputs into the captured
    buffers, replay, compare with the oracle, and run the same call eagerly
    (with its own outputs) between replays."""
    load(make_inputs(0))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = run()
    torch.cuda.synchronize()
    for rep in range(reps):
        inputs = make_inputs(rep + 1)
        load(inputs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        exp = expect(inputs)
        compare(captured, exp, f"replay {rep}")
        eager = run(fresh=True)
        torch.cuda.synchronize()
        compare(eager, exp, f"eager {rep}")


def test_hip_graph_segmented_rows_multi_tile():
    """Rows longer than one workgroup's tile take the histogram + look-back
    launches; the captured chain must replay correctly on new rows."""
    rows, n = 6, 20_011
    x = torch.empty((rows, n), dtype=torch.float16, device="cuda")
    vo = torch.empty_like(x)
    io = torch.empty((rows, n), dtype=torch.int64, device="cuda")
    ws = torch.empty(max(1, lrs.segmented_row_sort_workspace_size(rows, n, 4)), dtype=torch.uint8, device="cuda")

    def make_inputs(rep):
        v = workloads.normal_f64(9700 + rep, rows * n).astype(np.float16)
        v[:: 3 + rep] = np.round(v[:: 3 + rep])  # ties
        return v.view(np.uint16).reshape(rows, n)

    def load(u):
        x.copy_(torch.from_numpy(u.view(np.int16).copy()).cuda().view(torch.float16))

    def run(fresh=False):
        if fresh:
            return lrs.segmented_row_sort(x, True, 4)
        return lrs.segmented_row_sort(x, True, 4, values_out=vo, indices_out=io, workspace=ws)

    def compare(got, exp, what):
        gv = got[0].view(torch.int16).cpu().numpy().view(np.uint16)
        gi = got[1].cpu().numpy()
        assert np.array_equal(gv, exp[0]), f"{what}: values differ"
        assert np.array_equal(gi, exp[1]), f"{what}: indices differ"

    _replay_checked(make_inputs, load, run, lambda u: oracle.segmented_row_sort(u, True, 4), compare)


def test_hip_graph_typed_f64_pairs():
    """64-bit keys (eight 8-bit passes through the 64-bit sweep) in a graph."""
    n = 1_200_007
    k = torch.empty(n, dtype=torch.float64, device="cuda")
    v = torch.empty(n, dtype=torch.int32, device="cuda")
    ko, vo = torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(1, lrs.radix_sort_typed_workspace_size(n, "f64", 0, 64, 8, True)),
                     dtype=torch.uint8, device="cuda")

    def make_inputs(rep):
        x = workloads.normal_f64(9800 + rep, n)
        x[:: 5 + rep] = np.round(x[:: 5 + rep])
        return x.view(np.uint64).copy(), workloads.random_u32(9850 + rep, n)

    def load(inp):
        k.copy_(torch.from_numpy(inp[0].view(np.float64)).cuda())
        v.copy_(to_gpu(inp[1]))

    def run(fresh=False):
        if fresh:
            return lrs.radix_sort_pairs_typed(k, v, False)
        return lrs.radix_sort_pairs_typed(k, v, False, keys_out=ko, values_out=vo, workspace=ws)

    def compare(got, exp, what):
        gk = got[0].view(torch.int64).cpu().numpy().view(np.uint64)
        assert np.array_equal(gk, exp[0]), f"{what}: keys differ"
        assert_same(to_np_u32(got[1]), exp[1], f"{what}: values")

    _replay_checked(make_inputs, load, run,
                    lambda inp: oracle.radix_sort_typed(inp[0], inp[1], "f64", False, 0, 64, 8), compare)


def test_hip_graph_reduce_then_scan():
    """The reduce-then-scan launches (clear, histogram, and per pass count, scan
    and sweep) captured while that strategy is selected."""
    n = 2_000_003
    kin = torch.empty(n, dtype=torch.int32, device="cuda")
    vin, kout, vout = torch.empty_like(kin), torch.empty_like(kin), torch.empty_like(kin)
    ws = torch.empty(max(1, lrs.radix_sort_workspace_size(n, 0, 32, 4, True, options=lrs.SortOptions(
        scan="reduce-then-scan"))), dtype=torch.uint8, device="cuda")

    def make_inputs(rep):
        keys = workloads.random_u32(9900 + rep, n)
        if rep == 2:
            keys &= workloads.random_u32(9950, n) & workloads.random_u32(9951, n)
        return keys, np.arange(n, dtype=np.uint32)

    def load(inp):
        kin.copy_(to_gpu(inp[0]))
        vin.copy_(to_gpu(inp[1]))

    opt = lrs.SortOptions(scan="reduce-then-scan")

    def run(fresh=False):
        if fresh:
            return lrs.radix_sort_pairs(kin, vin, 0, 32, 4, options=opt)
        return lrs.radix_sort_pairs(kin, vin, 0, 32, 4, keys_out=kout, values_out=vout, workspace=ws, options=opt)

    def compare(got, exp, what):
        assert_same(to_np_u32(got[0]), exp[0], f"{what} keys")
        assert_same(to_np_u32(got[1]), exp[1], f"{what} values")

    _replay_checked(make_inputs, load, run, lambda inp: oracle.radix_sort_pairs(inp[0], inp[1], 0, 32, 4),
                    compare)
