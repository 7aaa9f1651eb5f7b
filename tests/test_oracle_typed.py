"""Pins of the oracle's typed 32-bit sort (signed integers, binary32 floats,
descending order) against numpy's stable sort, the plain definition of a
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
