"""Oracle vs textbook/library stable sorts, invariants and cross-width agreement.

Python's sorted() and numpy's argsort(kind="stable") are stable comparison sorts,
independent of the oracle's counting passes.  The exhaustive cases cover every
sequence of up to 5 keys over 4 bits for each digit width that divides the
window; the random cases cover windows that do not start at 0 or divide evenly.
"""
import itertools

import numpy as np
import pytest

import oracle
import workloads
from helpers import check_stable_sort_by_index, window


def _expected(keys, begin, end):
    w = window(keys, begin, end)
    order = np.argsort(w, kind="stable")
    return keys[order], order.astype(np.uint32)


@pytest.mark.parametrize("b", [1, 2, 4])
def test_exhaustive_small_sequences(b):
    for n in range(0, 5):
        for seq in itertools.product(range(16), repeat=n):
            keys = np.array(seq, dtype=np.uint32)
            ko, vo = oracle.radix_sort_pairs(keys, np.arange(n, dtype=np.uint32), 0, 4, b)
            order = sorted(range(n), key=lambda i: seq[i])
            assert vo.tolist() == order, (seq, b)
            assert ko.tolist() == [seq[i] for i in order]


@pytest.mark.parametrize("b", [1, 2, 4, 8])
@pytest.mark.parametrize("descending", [False, True])
def test_exhaustive_five_key_sequences(b, descending):
    """Every sequence of 5 keys over 4 bits (16^5 = 1,048,576 of them), each
    sorted on its own by the oracle's LSD passes: the sequences are the rows of
    a matrix whose entries are fp16 patterns 0x3C00 + v (1 + v/1024, ordered
    like v), and the row sort runs the counting-pass sort per row over the
    16-bit key.  numpy's stable argsort along each row is the reference."""
    m = 16 ** 5
    seq = ((np.arange(m)[:, None] >> (4 * np.arange(4, -1, -1))[None, :]) & 15).astype(np.int64)
    bits = (0x3C00 + seq).astype(np.uint16)
    vals, idx = oracle.segmented_row_sort(bits, descending, b)
    order = np.argsort(-seq if descending else seq, axis=1, kind="stable")
    assert np.array_equal(idx, order), f"b={b} descending={descending}: an index order differs"
    assert np.array_equal(vals, np.take_along_axis(bits, order, axis=1))


def test_random_windows_all_widths():
    rng = np.random.default_rng(1234)
    for trial in range(300):
        n = int(rng.integers(0, 301))
        keys = workloads.random_u32(900 + trial, n)
        if trial % 3 == 0:
            keys &= workloads.random_u32(5000 + trial, n)  # duplicates / skew
        begin = int(rng.integers(0, 32))
        end = int(rng.integers(begin + 1, 33))
        b = int(rng.choice([1, 2, 4, 8]))
        vals = np.arange(n, dtype=np.uint32)
        ko, vo = oracle.radix_sort_pairs(keys, vals, begin, end, b)
        ek, ev = _expected(keys, begin, end)
        assert np.array_equal(ko, ek) and np.array_equal(vo, ev), (trial, n, begin, end, b)
        kb, vb = oracle.radix_sort_pairs(keys, vals, begin, end, b, backward=True)
        assert np.array_equal(kb, ko) and np.array_equal(vb, vo)
        check_stable_sort_by_index(keys, ko, vo, window(ko, begin, end))


def test_widths_agree_and_invariants():
    n = 50000
    keys = workloads.random_u32(77, n) & workloads.random_u32(78, n)
    vals = np.arange(n, dtype=np.uint32)
    ref = None
    for b in (1, 2, 4, 8):
        ko, vo = oracle.radix_sort_pairs(keys, vals, 0, 32, b)
        check_stable_sort_by_index(keys, ko, vo)
        if ref is None:
            ref = (ko, vo)
        assert np.array_equal(ko, ref[0]) and np.array_equal(vo, ref[1]), b
    assert np.array_equal(ref[0], np.sort(keys))


def test_all_pass_histograms_match_bincount():
    keys = workloads.random_u32(5, 20000) & workloads.random_u32(6, 20000)
    for begin, end, b in ((0, 32, 8), (0, 32, 4), (3, 29, 8), (0, 12, 4), (7, 10, 1)):
        h = oracle.all_pass_histograms(keys, begin, end, b)
        P = oracle.num_passes(begin, end, b)
        assert h.shape == (P, 1 << b)
        for p in range(P):
            shift = begin + p * b
            width = min(b, end - shift)
            d = window(keys, shift, shift + width)
            assert np.array_equal(h[p], np.bincount(d.astype(np.int64), minlength=1 << b)), (p, b)


def test_stable_position_is_the_sort_destination():
    n = 3000
    keys = workloads.random_u32(11, n) & np.uint32(0x3F0F)
    for begin, end in ((0, 32), (4, 12), (8, 14)):
        ko, vo = oracle.radix_sort_pairs(keys, np.arange(n, dtype=np.uint32), begin, end, 4)
        where = np.empty(n, dtype=np.int64)
        where[vo.astype(np.int64)] = np.arange(n)
        for i in (0, 1, 17, 1234, n - 1):
            assert oracle.stable_position(keys, begin, end, i) == where[i]


def test_bits_outside_window_are_carried_and_tie():
    keys = np.array([0xF0000001, 0x00000001, 0x70000000, 0x10000001], dtype=np.uint32)
    ko, vo = oracle.radix_sort_pairs(keys, np.arange(4, dtype=np.uint32), 0, 4, 2)
    assert vo.tolist() == [2, 0, 1, 3]
    assert ko.tolist() == [0x70000000, 0xF0000001, 0x00000001, 0x10000001]


def test_invalid_arguments():
    keys = np.arange(4, dtype=np.uint32)
    for begin, end, b in ((0, 32, 3), (4, 4, 4), (0, 33, 8), (-1, 8, 4), (9, 8, 4)):
        with pytest.raises(ValueError):
            oracle.radix_sort_keys(keys, begin, end, b)
