"""Pins of the order-preserving 16-bit float key and the segmented row sort.

The key map is checked exhaustively over all 2^16 patterns against the real
numbers they encode (numpy float16; bf16 as the top half of a float32); the row
sort is checked against torch.sort(stable=True) on the CPU for inputs with no
NaN and no signed zero (where the two definitions coincide), and against the
stable-sort invariants for inputs with heavy duplicates.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import check_stable_sort_by_index

ALL = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


@pytest.fixture(scope="module")
def keys_asc():
    return oracle.float16_keys(ALL, False)


@pytest.fixture(scope="module")
def keys_desc():
    return oracle.float16_keys(ALL, True)


def _real(bits, dtype):
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def test_bijection(keys_asc, keys_desc):
    assert np.unique(keys_asc).size == 1 << 16
    assert np.unique(keys_desc).size == 1 << 16
    assert np.array_equal(keys_desc, (~keys_asc).astype(np.uint16))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_order_matches_real_values(keys_asc, keys_desc, dtype):
    x = _real(ALL, dtype)
    ok = ~np.isnan(x)
    xs, ka, kd = x[ok], keys_asc[ok].astype(np.int64), keys_desc[ok].astype(np.int64)
    order = np.argsort(ka, kind="stable")
    assert np.all(np.diff(xs[order]) >= 0)
    # strict: different reals give different keys in the same order
    o = np.argsort(xs, kind="stable")
    dx = np.diff(xs[o])
    dk = np.diff(ka[o])
    assert np.all(dk[dx > 0] > 0)
    # only the two zeros tie as reals, and -0 sorts immediately before +0
    assert np.count_nonzero(dx == 0) == 1
    assert oracle.float16_key(0x8000) + 1 == oracle.float16_key(0x0000)
    # descending reverses the order of distinct reals
    assert np.all(np.diff(kd[o])[dx > 0] < 0)
    # infinities are the extreme non-NaN keys
    inf = 0x7C00 if dtype == "fp16" else 0x7F80
    assert oracle.float16_key(inf) == ka.max()
    assert oracle.float16_key(inf | 0x8000) == ka.min()


def _torch_rows(bits, dtype, descending):
    t = torch.from_numpy(bits.astype(np.int16)).view(torch.float16 if dtype == "fp16" else torch.bfloat16)
    v, i = torch.sort(t, dim=-1, descending=descending, stable=True)
    return v.view(torch.int16).numpy().view(np.uint16), i.numpy()


@pytest.mark.parametrize("dtype,descending,b", [("fp16", False, 4), ("fp16", True, 8),
                                                 ("bf16", True, 8), ("bf16", False, 2)])
def test_rows_match_torch_stable_sort(dtype, descending, b):
    rows, n = 6, 777
    if dtype == "fp16":
        bits = workloads.fp16_normal_bits(4242, rows * n).reshape(rows, n)
    else:
        bits = workloads.bf16_64level_bits(4243, rows * n).reshape(rows, n)
    zero = (bits & np.uint16(0x7FFF)) == 0
    bits[zero] = np.uint16(0x3C00 if dtype == "fp16" else 0x3F80)  # no signed zeros
    vo, io = oracle.segmented_row_sort(bits, descending, b)
    tv, ti = _torch_rows(bits, dtype, descending)
    assert np.array_equal(vo, tv)
    assert np.array_equal(io, ti)


def test_descending_ties_keep_input_order():
    rows, n = 3, 4096
    bits = workloads.bf16_64level_bits(99, rows * n).reshape(rows, n)
    vo, io = oracle.segmented_row_sort(bits, True, 8)
    for r in range(rows):
        kd = oracle.float16_keys(vo[r], True)
        check_stable_sort_by_index(bits[r], vo[r], io[r], kd)
        x = _real(vo[r], "bf16")
        assert np.all(np.diff(x) <= 0)


def test_widths_agree_on_rows():
    bits = workloads.fp16_normal_bits(7, 4 * 1000).reshape(4, 1000)
    ref = oracle.segmented_row_sort(bits, False, 1)
    for b in (2, 4, 8):
        v, i = oracle.segmented_row_sort(bits, False, b)
        assert np.array_equal(v, ref[0]) and np.array_equal(i, ref[1])


def test_row_stable_position():
    bits = workloads.bf16_64level_bits(3, 2000)
    vo, io = oracle.segmented_row_sort(bits.reshape(1, -1), True, 8)
    where = np.empty(2000, dtype=np.int64)
    where[io[0]] = np.arange(2000)
    for j in (0, 5, 999, 1999):
        assert oracle.row_stable_position(bits, True, j) == where[j]


def test_segmented_histograms():
    bits = workloads.fp16_normal_bits(8, 3 * 500).reshape(3, 500)
    h = oracle.segmented_histograms(bits, False, 4)
    assert h.shape == (3, 4, 16)
    k = oracle.float16_keys(bits, False).astype(np.int64)
    for r in range(3):
        for p in range(4):
            assert np.array_equal(h[r, p], np.bincount((k[r] >> (4 * p)) & 15, minlength=16))


def test_workload_generators():
    # SplitMix64: draw 0 of seed 0 is the published first output 0xE220A8397B1DCDAF
    assert int(workloads.splitmix64(0, 1)[0]) == 0xE220A8397B1DCDAF
    k = workloads.keys_c1()
    assert k.size == 1024 and k.max() < 4096
    b = workloads.matrix_c5(8, 4096)
    x = _real(b.ravel(), "bf16")
    assert np.unique(x).size <= 64 and x.min() >= -4.0 and x.max() <= 3.875
    assert not np.any(b == np.uint16(0x8000))
    f = workloads.matrix_c4(2, 4096)
    assert np.all(np.isfinite(f.view(np.float16)))
