"""Pins of the CPU oracle against values the pages print and facts they state.

- DSA CUDA from first principles, ch.13: the base-10 worked example (digit
  counts and offsets of section 13.1, the stable pass of section 13.2, the
  per-element ranks and the digit-3 indicator scan, and the two-pass LSD sort
  of section 13.3).
- 100 Days of GPU, Day 35: the 16-key one-bit split (9 clear keys, last scan
  cell + last flag = 9, 16 distinct stable destinations) checked against the
  split formula the page quotes (t = i - f + totalFalses for a set key, f for a
  clear key), which is a different algorithm from the oracle's counting pass.
"""
import numpy as np

import oracle
from helpers import ints, read_fixture, tagged

EX = read_fixture("dsa_ch13_worked_example.txt")
SPLIT = read_fixture("day35_onebit_split16.txt")


def _digits_place(values, place, base=10):
    return [oracle.digit_place(v, place, base) for v in values]


def test_section_13_1_digits_counts_offsets():
    a = ints(EX["input"])
    d = _digits_place(a, 1)
    assert d == ints(EX["digits_place1"])
    count, offset, _ = oracle.counting_pass(d, 10)
    assert count.tolist() == ints(EX["count_place1"])
    assert offset.tolist() == ints(EX["offset_place1"])
    assert int(count.sum()) == len(a)


def _apply(dest, *arrays):
    outs = []
    for arr in arrays:
        o = [None] * len(arr)
        for i, di in enumerate(dest):
            o[int(di)] = arr[i]
        outs.append(o)
    return outs


def test_section_13_2_one_stable_pass():
    a = ints(EX["input"])
    tags = list(range(len(a)))
    _, _, dest = oracle.counting_pass(_digits_place(a, 1), 10)
    vals, tg = _apply(dest, a, tags)
    ev, et = tagged(EX["pass1_tagged"])
    assert vals == ev and tg == et
    # the two 13s keep @1 before @6
    assert [t for v, t in zip(vals, tg) if v == 13] == [1, 6]


def test_section_13_2_ranks_and_indicator_scan():
    a = ints(EX["input"])
    d = _digits_place(a, 1)
    rank = oracle.rank_within_digit(d)
    assert rank.tolist() == ints(EX["rank_within_digit"])
    # the printed digit-3 indicator and its exclusive scan
    ind = [1 if x == 3 else 0 for x in d]
    assert ind == ints(EX["indicator_digit3"])
    scan = ints(EX["indicator_digit3_exclusive_scan"])
    for i in range(len(a)):
        if d[i] == 3:
            assert rank[i] == scan[i]
    # destination = offset[digit] + rank, the same as the counting pass
    count, offset, dest = oracle.counting_pass(d, 10)
    assert [int(offset[d[i]] + rank[i]) for i in range(len(a))] == dest.tolist()


def test_section_13_3_two_pass_lsd():
    a = ints(EX["input"])
    tags = list(range(len(a)))
    assert int(EX["passes_needed"][0]) == 2
    vals, tg = a, tags
    for place, key in ((1, "pass1_tagged"), (10, "pass2_tagged")):
        _, _, dest = oracle.counting_pass(_digits_place(vals, place), 10)
        vals, tg = _apply(dest, vals, tg)
        ev, et = tagged(EX[key])
        assert vals == ev and tg == et, key


def test_backward_walk_agrees_on_worked_example():
    a = ints(EX["input"])
    d = _digits_place(a, 1)
    _, _, fwd = oracle.counting_pass(d, 10)
    assert oracle.counting_pass_backward(d, 10).tolist() == fwd.tolist()


def test_one_bit_split_16_keys():
    bits = ints(SPLIT["bits"])
    n = int(SPLIT["keys_total"][0])
    F_expected = int(SPLIT["clear_count"][0])
    assert len(bits) == n
    # the page's construction: flag 1 under clear keys, exclusive scan, formula
    flag = [1 - b for b in bits]
    f = [sum(flag[:i]) for i in range(n)]
    total_falses = f[-1] + flag[-1]
    assert total_falses == F_expected == 9
    formula = [(total_falses + i - f[i]) if bits[i] else f[i] for i in range(n)]
    # 16 distinct destinations, each group in input order
    assert sorted(formula) == list(range(n))
    clear_dst = [formula[i] for i in range(n) if not bits[i]]
    set_dst = [formula[i] for i in range(n) if bits[i]]
    assert clear_dst == list(range(9)) and set_dst == list(range(9, 16))
    # the oracle's radix-2 counting pass reaches the same destinations
    count, offset, dest = oracle.counting_pass(bits, 2)
    assert dest.tolist() == formula
    assert count.tolist() == [9, 7] and offset.tolist() == [0, 9]
    # and so does the 1-bit LSD sort over that single bit, as a permutation
    keys = np.array(bits, dtype=np.uint32) << np.uint32(5)
    ko, vo = oracle.radix_sort_pairs(keys, np.arange(n, dtype=np.uint32), 5, 6, 1)
    inv = np.empty(n, dtype=np.int64)
    inv[vo.astype(np.int64)] = np.arange(n)
    assert inv.tolist() == formula


def test_digit_bits_and_pass_count():
    assert oracle.digit_bits(0xABCD1234, 0, 4) == 0x4
    assert oracle.digit_bits(0xABCD1234, 28, 4) == 0xA
    assert oracle.digit_bits(0xABCD1234, 8, 8) == 0x12
    assert oracle.digit_bits(0xFFFFFFFF, 30, 2) == 3
    assert oracle.digit_bits(0x80000000, 0, 32) == 0x80000000
    # P = ceil(width / b); the radix-16 exercise over keys below 4096 needs 3 passes
    assert oracle.num_passes(0, 12, 4) == 3
    assert oracle.num_passes(0, 32, 8) == 4
    assert oracle.num_passes(0, 32, 4) == 8
    assert oracle.num_passes(0, 32, 1) == 32
    assert oracle.num_passes(3, 13, 4) == 3
    assert oracle.num_passes(0, 16, 8) == 2


def test_radix16_three_passes_low_digit_first():
    # gpu.rocks "The Whole Sort": keys below 4096, radix 16, place 1, 16, 256.
    keys = np.array([0x321, 0x123, 0x213, 0x132, 0x312, 0x231, 0x111, 0x333], dtype=np.uint32)
    ko = oracle.radix_sort_keys(keys, 0, 12, 4)
    assert ko.tolist() == sorted(keys.tolist())
    # after one pass (bits 0..3) the array is ordered by the low hex digit, stably
    k1 = oracle.radix_sort_keys(keys, 0, 4, 4)
    assert k1.tolist() == sorted(keys.tolist(), key=lambda x: x & 0xF)
    # running the passes high digit first instead orders by the low digit: the
    # state after the high pass then the low pass is the one-pass low-digit order
    hi_first = oracle.radix_sort_keys(oracle.radix_sort_keys(keys, 8, 12, 4), 0, 4, 4)
    assert hi_first.tolist() == sorted(sorted(keys.tolist(), key=lambda x: x >> 8), key=lambda x: x & 0xF)
    assert hi_first.tolist() != ko.tolist()
