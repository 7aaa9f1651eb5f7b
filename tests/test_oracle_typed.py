"""Pins of the oracle's typed 32- and 64-bit sorts (signed integers, binary32
and binary64 floats, descending order) against numpy's stable sort, the plain definition of a
descending stable order, the real-number order of floats, and a hand-ordered
list of special float patterns (Day 35 "Pitfalls": floats and signed integers
sort as unsigned integers after an order-preserving map)."""
import struct

import numpy as np
import pytest

import oracle
import workloads

SPECIAL_F32_IN_ORDER = [  # ascending order under the reading: -NaN first, +NaN last, -0 before +0
    0xFFC00000,  # -NaN (quiet)
    0xFF800000,  # -inf
    0xFF7FFFFF,  # -max
    0xBF800000,  # -1
    0x80800000,  # -smallest normal
    0x80000001,  # -smallest subnormal
    0x80000000,  # -0
    0x00000000,  # +0
    0x00000001,  # +smallest subnormal
    0x00800000,  # +smallest normal
    0x3F800000,  # +1
    0x7F7FFFFF,  # +max
    0x7F800000,  # +inf
    0x7FC00000,  # +NaN (quiet)
]


def _perm(keys, key_type, descending, b=8, begin=0, end=32):
    n = len(keys)
    _, idx = oracle.radix_sort_typed(keys, np.arange(n, dtype=np.uint32), key_type, descending, begin, end, b)
    return idx.astype(np.int64)


def _desc_stable(values):
    # plain definition: larger first, equal values in input order
    return np.array(sorted(range(len(values)), key=lambda i: (-values[i], i)), dtype=np.int64)


@pytest.mark.parametrize("n", [1, 2, 17, 1000, 20000])
def test_i32_against_numpy_and_definition(n):
    x = workloads.random_u32(600 + n, n).view(np.int32).copy()
    if n >= 4:
        x[:4] = [np.iinfo(np.int32).min, np.iinfo(np.int32).max, 0, -1]
    x[n // 2:] = x[n // 2:] % 97 - 48  # many ties
    asc = _perm(x, "i32", False)
    assert np.array_equal(asc, np.argsort(x, kind="stable"))
    desc = _perm(x, "i32", True)
    assert np.array_equal(desc, _desc_stable([int(v) for v in x]))


@pytest.mark.parametrize("n", [3, 1000, 20000])
def test_f32_against_numpy_and_definition(n):
    x = workloads.normal_f64(700 + n, n).astype(np.float32)
    x[::7] = np.round(x[::7])  # ties, including +0 (never -0: numpy ranks -0 == +0)
    x[x == 0] = np.float32(0.0)
    asc = _perm(x, "f32", False)
    assert np.array_equal(asc, np.argsort(x, kind="stable"))
    desc = _perm(x, "f32", True)
    assert np.array_equal(desc, _desc_stable([float(v) for v in x]))


def test_f32_special_values_order():
    order = np.array(SPECIAL_F32_IN_ORDER, dtype=np.uint32)
    rng = np.random.default_rng(5)
    for _ in range(20):
        shuffled = order[rng.permutation(order.size)]
        keys, _ = oracle.radix_sort_typed(shuffled, None, "f32", False)
        assert np.array_equal(keys, order)
        keys, _ = oracle.radix_sort_typed(shuffled, None, "f32", True)
        assert np.array_equal(keys, order[::-1])


def test_f32_image_is_monotone_in_real_value():
    a = workloads.random_u32(801, 20000)
    b = workloads.random_u32(802, 20000)
    checked = 0
    for x, y in zip(a.tolist(), b.tolist()):
        fx = struct.unpack("<f", struct.pack("<I", x))[0]
        fy = struct.unpack("<f", struct.pack("<I", y))[0]
        if fx != fx or fy != fy or fx == fy:  # NaNs and equal values (incl. -0 == +0)
            continue
        checked += 1
        assert (oracle.key32(x, "f32") < oracle.key32(y, "f32")) == (fx < fy)
        assert (oracle.key32(x, "f32", True) < oracle.key32(y, "f32", True)) == (fx > fy)
    assert checked > 19000


def test_i32_image_is_monotone():
    vals = [-2**31, -2**31 + 1, -65536, -2, -1, 0, 1, 2, 65535, 2**31 - 2, 2**31 - 1]
    images = [oracle.key32(v & 0xFFFFFFFF, "i32") for v in vals]
    assert images == sorted(images) and len(set(images)) == len(images)
    assert images[0] == 0 and images[-1] == 0xFFFFFFFF


def test_u32_typed_matches_plain_sort_and_descending_definition():
    x = workloads.random_u32(900, 5000) % 1000
    k, _ = oracle.radix_sort_typed(x, None, "u32", False)
    assert np.array_equal(k, oracle.radix_sort_keys(x))
    desc = _perm(x, "u32", True)
    assert np.array_equal(desc, _desc_stable([int(v) for v in x]))


@pytest.mark.parametrize("key_type", ["i32", "f32"])
def test_digit_widths_agree(key_type):
    x = workloads.random_u32(950, 4000)
    if key_type == "f32":
        x = workloads.normal_f64(951, 4000).astype(np.float32).view(np.uint32)
    vals = np.arange(x.size, dtype=np.uint32)
    ref = oracle.radix_sort_typed(x, vals, key_type, True, 0, 32, 8)
    for b in (1, 2, 4):
        got = oracle.radix_sort_typed(x, vals, key_type, True, 0, 32, b)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


# ------------------------------------------------------------- 64-bit keys

SPECIAL_F64_IN_ORDER = [
    0xFFF8000000000000,  # -NaN
    0xFFF0000000000000,  # -inf
    0xFFEFFFFFFFFFFFFF,  # -max
    0xBFF0000000000000,  # -1
    0x8000000000000001,  # -smallest subnormal
    0x8000000000000000,  # -0
    0x0000000000000000,  # +0
    0x0000000000000001,  # +smallest subnormal
    0x3FF0000000000000,  # +1
    0x7FEFFFFFFFFFFFFF,  # +max
    0x7FF0000000000000,  # +inf
    0x7FF8000000000000,  # +NaN
]


def _i64(n, seed):
    hi = workloads.random_u32(seed, n).astype(np.uint64)
    lo = workloads.random_u32(seed + 1, n).astype(np.uint64)
    return ((hi << np.uint64(32)) | lo).view(np.int64).copy()


@pytest.mark.parametrize("n", [1, 17, 5000])
def test_i64_against_numpy_and_definition(n):
    x = _i64(n, 1100 + n)
    if n >= 4:
        x[:4] = [np.iinfo(np.int64).min, np.iinfo(np.int64).max, 0, -1]
    x[n // 2:] = x[n // 2:] % 97 - 48
    asc = _perm64(x, "i64", False)
    assert np.array_equal(asc, np.argsort(x, kind="stable"))
    assert np.array_equal(_perm64(x, "i64", True), _desc_stable([int(v) for v in x]))


def _perm64(keys, key_type, descending, b=8, begin=0, end=64):
    n = len(keys)
    _, idx = oracle.radix_sort_typed(keys, np.arange(n, dtype=np.uint32), key_type, descending, begin, end, b)
    return idx.astype(np.int64)


@pytest.mark.parametrize("n", [3, 5000])
def test_f64_against_numpy_and_definition(n):
    x = workloads.normal_f64(1200 + n, n)
    x[::7] = np.round(x[::7])
    x[x == 0] = 0.0
    assert np.array_equal(_perm64(x, "f64", False), np.argsort(x, kind="stable"))
    assert np.array_equal(_perm64(x, "f64", True), _desc_stable([float(v) for v in x]))


def test_f64_special_values_order():
    order = np.array(SPECIAL_F64_IN_ORDER, dtype=np.uint64)
    rng = np.random.default_rng(6)
    for _ in range(20):
        shuffled = order[rng.permutation(order.size)]
        assert np.array_equal(oracle.radix_sort_typed(shuffled, None, "f64", False, 0, 64)[0], order)
        assert np.array_equal(oracle.radix_sort_typed(shuffled, None, "f64", True, 0, 64)[0], order[::-1])


def test_u64_descending_definition_and_window():
    x = _i64(3000, 1300).view(np.uint64) % np.uint64(10 ** 12)
    assert np.array_equal(_perm64(x, "u64", True), _desc_stable([int(v) for v in x]))
    # the top 16 bits of the i64 image order like the arithmetic shift of the value by 48
    y = _i64(3000, 1310)
    assert np.array_equal(_perm64(y, "i64", False, 4, 48, 64), np.argsort(y >> 48, kind="stable"))


@pytest.mark.parametrize("key_type", ["i64", "f64"])
def test_digit_widths_agree_64(key_type):
    x = _i64(2000, 1400) if key_type == "i64" else workloads.normal_f64(1401, 2000)
    vals = np.arange(x.size, dtype=np.uint32)
    ref = oracle.radix_sort_typed(x, vals, key_type, False, 0, 64, 8)
    for b in (2, 4):
        got = oracle.radix_sort_typed(x, vals, key_type, False, 0, 64, b)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
