"""GPU parity of the typed 32-bit sorts (signed integers, binary32 floats and
descending u32) against the CPU oracle, element for element with tolerance 0,
keys-only and with a payload, across the whole-row, 4096-, 8192- and
15360-key tile shapes, with special float patterns mixed in."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

lrs = pytest.importorskip("lsd_radix_sort_amd")

SPECIAL_F32 = np.array([0xFFC00000, 0xFF800000, 0xFF7FFFFF, 0xBF800000, 0x80000001, 0x80000000, 0x00000000,
                        0x00000001, 0x3F800000, 0x7F7FFFFF, 0x7F800000, 0x7FC00000, 0x7FC00001, 0xFFFFFFFF],
                       dtype=np.uint32)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lrs.load_library()


def make_keys(key_type: str, n: int, seed: int) -> np.ndarray:
    """Bit patterns (uint32) of n keys of the type, with ties and special values."""
    if key_type == "f32":
        x = workloads.normal_f64(seed, n).astype(np.float32)
        x[::5] = np.round(x[::5] * 4) / 4  # ties
        bits = x.view(np.uint32).copy()
        bits[3::97] = SPECIAL_F32[np.arange(bits[3::97].size) % SPECIAL_F32.size]
        return bits
    bits = workloads.random_u32(seed, n)
    bits[1::3] = bits[1::3] % 64  # ties; for i32 also small positives
    if key_type == "i32":
        small_negative = -(bits[2::11] % 64).astype(np.int64) - 1  # -1 .. -64
        bits[2::11] = small_negative.astype(np.int32).view(np.uint32)
    return bits


def gpu_typed(bits: np.ndarray, key_type: str, descending: bool, b: int, with_vals: bool,
              begin: int = 0, end: int = 32, options=None):
    kt = torch.from_numpy(bits.view(np.int32).copy()).cuda()
    if key_type == "f32":
        kt = kt.view(torch.float32)
    vals = np.arange(bits.size, dtype=np.uint32) * np.uint32(2654435761)
    if with_vals:
        vt = torch.from_numpy(vals.view(np.int32).copy()).cuda()
        ko, vo = lrs.radix_sort_pairs_typed(kt, vt, descending, key_type, begin, end, b, options=options)
        torch.cuda.synchronize()
        return ko.view(torch.int32).cpu().numpy().view(np.uint32), vo.cpu().numpy().view(np.uint32), vals
    ko = lrs.radix_sort_keys_typed(kt, descending, key_type, begin, end, b, options=options)
    torch.cuda.synchronize()
    return ko.view(torch.int32).cpu().numpy().view(np.uint32), None, vals


def check(bits, key_type, descending, b, begin=0, end=32, options=None):
    for with_vals in (False, True):
        gk, gv, vals = gpu_typed(bits, key_type, descending, b, with_vals, begin, end, options)
        ek, ev = oracle.radix_sort_typed(bits, vals if with_vals else None, key_type, descending, begin, end, b)
        bad = np.flatnonzero(gk != ek)
        assert bad.size == 0, f"{key_type} desc={descending} b={b} keys differ at {bad[:5]} (of {bad.size})"
        if with_vals:
            bad = np.flatnonzero(gv != ev)
            assert bad.size == 0, f"{key_type} desc={descending} b={b} values differ at {bad[:5]} (of {bad.size})"


@pytest.mark.parametrize("key_type", ["i32", "f32", "u32"])
@pytest.mark.parametrize("n", [1, 1000, 8192, 8193, 300_001, 3_000_017])
def test_typed_sizes(key_type, n):
    bits = make_keys(key_type, n, 5100 + n)
    for descending in (False, True):
        if key_type == "u32" and not descending and n > 8193:
            continue  # ascending u32 is the plain sort, tested elsewhere
        log(f"{key_type} n={n} desc={descending}")
        check(bits, key_type, descending, 8)


@pytest.mark.parametrize("key_type", ["i32", "f32"])
@pytest.mark.parametrize("b", [1, 2, 4])
def test_typed_digit_widths(key_type, b):
    bits = make_keys(key_type, 50_003, 5200 + b)
    for descending in (False, True):
        log(f"{key_type} b={b} desc={descending}")
        check(bits, key_type, descending, b)


def test_typed_bit_window():
    # sort f32 keys by the top 12 bits of their image only: ties beyond keep input order
    bits = make_keys("f32", 100_000, 5300)
    check(bits, "f32", False, 4, 20, 32)
    check(bits, "f32", True, 8, 16, 32)


@pytest.mark.parametrize("key_type", ["i32", "u32"])
def test_typed_one_xor_kinds(key_type):
    # int32 keys (either direction) and descending u32 keys map to their image
    # by one XOR with a constant: bit windows, narrow digits, the
    # reduce-then-scan sweeps and the largest tile of that key kind
    bits = make_keys(key_type, 200_003, 5500)
    for descending in ((False, True) if key_type == "i32" else (True,)):
        log(f"{key_type} desc={descending} windows")
        check(bits, key_type, descending, 4, 20, 32)
        check(bits, key_type, descending, 8, 8, 31)
        log(f"{key_type} desc={descending} reduce-then-scan")
        check(bits, key_type, descending, 8, options=lrs.SortOptions(scan="reduce-then-scan"))
    for b in (1, 2):
        check(bits[:50_003], key_type, True, b)
    big = make_keys(key_type, 15_000_007, 5600)
    log(f"{key_type} n=15000007 desc")
    check(big, key_type, True, 8)


def test_typed_largest_tile():
    bits = make_keys("f32", 15_000_007, 5400)
    log("f32 n=15000007 asc")
    check(bits, "f32", False, 8)


def test_typed_rejects_unknown_key_type():
    k = torch.zeros(16, dtype=torch.int32, device="cuda")
    o = torch.empty_like(k)
    ws = torch.empty(1, dtype=torch.uint8, device="cuda")
    lib = lrs.load_library()
    st = lib.radix_sort_keys_typed(k.data_ptr(), o.data_ptr(), 16, 7, 0, 0, 32, 8, ws.data_ptr(), 1,
                                   torch.cuda.current_stream().cuda_stream, None)
    assert st == 7  # LRS_ERR_DTYPE


# ------------------------------------------------------------- 64-bit keys

SPECIAL_F64 = np.array([0xFFF8000000000000, 0xFFF0000000000000, 0xFFEFFFFFFFFFFFFF, 0xBFF0000000000000,
                        0x8000000000000001, 0x8000000000000000, 0x0000000000000000, 0x0000000000000001,
                        0x3FF0000000000000, 0x7FEFFFFFFFFFFFFF, 0x7FF0000000000000, 0x7FF8000000000000,
                        0x7FF8000000000001, 0xFFFFFFFFFFFFFFFF], dtype=np.uint64)


def make_keys64(key_type: str, n: int, seed: int) -> np.ndarray:
    """Bit patterns (uint64) of n keys of the type, with ties and special values."""
    if key_type == "f64":
        x = workloads.normal_f64(seed, n)
        x[::5] = np.round(x[::5] * 4) / 4
        bits = x.view(np.uint64).copy()
        bits[3::97] = SPECIAL_F64[np.arange(bits[3::97].size) % SPECIAL_F64.size]
        return bits
    hi = workloads.random_u32(seed, n).astype(np.uint64)
    lo = workloads.random_u32(seed + 7, n).astype(np.uint64)
    bits = (hi << np.uint64(32)) | lo
    bits[1::3] = bits[1::3] % np.uint64(64)  # ties, small positives
    if key_type == "i64":
        small_negative = -(bits[2::11] % np.uint64(64)).astype(np.int64) - 1
        bits[2::11] = small_negative.view(np.uint64)
    return bits


def check64(bits, key_type, descending, b, begin=0, end=64):
    kt = torch.from_numpy(bits.view(np.int64).copy()).cuda()
    if key_type == "f64":
        kt = kt.view(torch.float64)
    vals = np.arange(bits.size, dtype=np.uint32) * np.uint32(2654435761)
    vt = torch.from_numpy(vals.view(np.int32).copy()).cuda()
    for with_vals in (False, True):
        if with_vals:
            ko, vo = lrs.radix_sort_pairs_typed(kt, vt, descending, key_type, begin, end, b)
        else:
            ko, vo = lrs.radix_sort_keys_typed(kt, descending, key_type, begin, end, b), None
        torch.cuda.synchronize()
        gk = ko.view(torch.int64).cpu().numpy().view(np.uint64)
        ek, ev = oracle.radix_sort_typed(bits, vals if with_vals else None, key_type, descending, begin, end, b)
        bad = np.flatnonzero(gk != ek)
        assert bad.size == 0, f"{key_type} desc={descending} b={b} keys differ at {bad[:5]} (of {bad.size})"
        if with_vals:
            gv = vo.cpu().numpy().view(np.uint32)
            bad = np.flatnonzero(gv != ev)
            assert bad.size == 0, f"{key_type} desc={descending} b={b} values differ at {bad[:5]} (of {bad.size})"


@pytest.mark.parametrize("key_type", ["i64", "f64", "u64"])
@pytest.mark.parametrize("n", [1, 1000, 8193, 300_001, 1_200_007, 2_500_003])
def test_typed64_sizes(key_type, n):
    # 2048-, 4096- and 8192-key tile shapes of 64-bit keys
    bits = make_keys64(key_type, n, 6100 + n % 1000)
    for descending in (False, True):
        log(f"{key_type} n={n} desc={descending}")
        check64(bits, key_type, descending, 8)


@pytest.mark.parametrize("key_type", ["i64", "f64"])
@pytest.mark.parametrize("b", [2, 4])
def test_typed64_digit_widths(key_type, b):
    bits = make_keys64(key_type, 40_003, 6200 + b)
    for descending in (False, True):
        log(f"{key_type} b={b} desc={descending}")
        check64(bits, key_type, descending, b)


def test_typed64_one_bit_digits_and_windows():
    bits = make_keys64("i64", 5003, 6300)
    check64(bits, "i64", False, 1)            # 64 one-bit passes
    check64(bits, "i64", True, 4, 16, 48)     # a middle window of the image
    check64(make_keys64("u64", 70_001, 6301), "u64", False, 8, 0, 40)
