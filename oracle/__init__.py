"""CPU oracle for LSD radix sort -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (``lsd_radix_sort_amd``) never does and
shares no code with it.  The arithmetic lives in ``lrs_oracle.c`` (plain C,
built with gcc by :func:`build`); this module only marshals numpy arrays.

Sources: CUDA Handbook ch.16 "Radix Sort" (the three per-pass steps and the
host pass/driver listings); DSA CUDA from first principles ch.13 (sections
13.1-13.3); 100 Days of GPU, Day 35 (backward walk, payload exercise,
pitfalls); gpu.rocks "The Whole Sort"; FlagTree PR #1084 (descending flag in
the order-preserving float conversion, int64 column-index payload).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lrs_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblrs_oracle.so")
_CTX_SRC = os.path.join(_HERE, "std_sort_context.cpp")
_CTX_PATH = os.path.join(_HERE, "libstd_sort_context.so")
_lib = None

OK = 0


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/liblrs_oracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-fPIC", "-shared", "-o", tmp, _SRC]
        )
        os.replace(tmp, _LIB_PATH)
    if force or not os.path.exists(_CTX_PATH):
        tmp = _CTX_PATH + ".tmp"
        subprocess.check_call(["g++", "-std=c++17", "-O2", "-Wall", "-fPIC", "-shared", "-o", tmp, _CTX_SRC])
        os.replace(tmp, _CTX_PATH)
    return _LIB_PATH


def std_sort_seconds(keys: np.ndarray) -> float:
    """Seconds std::sort takes on one core to sort a copy of these u32 keys (a
    context figure for the benchmark, not part of the oracle)."""
    if not os.path.exists(_CTX_PATH):
        build(force=True)
    lib = ctypes.CDLL(_CTX_PATH)
    lib.std_sort_u32_seconds.argtypes = [ctypes.c_void_p, ctypes.c_uint64]
    lib.std_sort_u32_seconds.restype = ctypes.c_double
    a = np.ascontiguousarray(keys, dtype=np.uint32).copy()
    secs = lib.std_sort_u32_seconds(a.ctypes.data, a.size)
    assert np.all(a[1:] >= a[:-1]), "std::sort did not sort"
    return float(secs)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    u64, i64, c_int, u32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32
    lib.oracle_digit_bits.argtypes = [u32, c_int, c_int]
    lib.oracle_digit_bits.restype = u32
    lib.oracle_digit_place.argtypes = [u64, u64, u32]
    lib.oracle_digit_place.restype = u32
    lib.oracle_counting_pass.argtypes = [P, u64, u32, P, P, P]
    lib.oracle_counting_pass.restype = c_int
    lib.oracle_counting_pass_backward.argtypes = [P, u64, u32, P]
    lib.oracle_counting_pass_backward.restype = c_int
    lib.oracle_rank_within_digit.argtypes = [P, u64, P]
    lib.oracle_rank_within_digit.restype = None
    lib.oracle_num_passes.argtypes = [c_int, c_int, c_int]
    lib.oracle_num_passes.restype = c_int
    lib.oracle_all_pass_histograms.argtypes = [P, u64, c_int, c_int, c_int, P]
    lib.oracle_all_pass_histograms.restype = c_int
    lib.oracle_radix_sort_pairs.argtypes = [P, P, P, P, u64, c_int, c_int, c_int, c_int]
    lib.oracle_radix_sort_pairs.restype = c_int
    lib.oracle_stable_position.argtypes = [P, u64, c_int, c_int, u64]
    lib.oracle_stable_position.restype = u64
    lib.oracle_float16_key.argtypes = [ctypes.c_uint16, c_int]
    lib.oracle_float16_key.restype = ctypes.c_uint16
    lib.oracle_segmented_row_sort.argtypes = [P, P, P, i64, i64, c_int, c_int]
    lib.oracle_segmented_row_sort.restype = c_int
    lib.oracle_segmented_histograms.argtypes = [P, i64, i64, c_int, c_int, P]
    lib.oracle_segmented_histograms.restype = c_int
    lib.oracle_row_stable_position.argtypes = [P, u64, c_int, u64]
    lib.oracle_row_stable_position.restype = u64
    lib.oracle_key32.argtypes = [u32, c_int, c_int, P]
    lib.oracle_key32.restype = c_int
    lib.oracle_radix_sort_typed.argtypes = [P, P, P, P, u64, c_int, c_int, c_int, c_int, c_int]
    lib.oracle_radix_sort_typed.restype = c_int
    lib.oracle_key64.argtypes = [u64, c_int, c_int, P]
    lib.oracle_key64.restype = c_int
    lib.oracle_radix_sort_typed64.argtypes = [P, P, P, P, u64, c_int, c_int, c_int, c_int, c_int]
    lib.oracle_radix_sort_typed64.restype = c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != OK:
        raise ValueError(f"oracle {what} failed with code {rc}")


def _u32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.uint32))


# ------------------------------------------------------------------ digits

def digit_bits(key: int, shift: int, width: int) -> int:
    return int(_load().oracle_digit_bits(key, shift, width))


def digit_place(value: int, place: int, base: int) -> int:
    return int(_load().oracle_digit_place(value, place, base))


def num_passes(begin_bit: int, end_bit: int, digit_bits: int) -> int:
    return int(_load().oracle_num_passes(begin_bit, end_bit, digit_bits))


# ------------------------------------------------------- one counting pass

def counting_pass(digits, radix: int):
    """Return (count, offset, dest) of one stable counting-sort pass."""
    d = _u32(digits)
    count = np.zeros(radix, dtype=np.uint64)
    offset = np.zeros(radix, dtype=np.uint64)
    dest = np.zeros(d.size, dtype=np.uint64)
    _check(_load().oracle_counting_pass(_ptr(d), d.size, radix, _ptr(count), _ptr(offset), _ptr(dest)),
           "counting_pass")
    return count, offset, dest


def counting_pass_backward(digits, radix: int) -> np.ndarray:
    d = _u32(digits)
    dest = np.zeros(d.size, dtype=np.uint64)
    _check(_load().oracle_counting_pass_backward(_ptr(d), d.size, radix, _ptr(dest)),
           "counting_pass_backward")
    return dest


def rank_within_digit(digits) -> np.ndarray:
    d = _u32(digits)
    rank = np.zeros(d.size, dtype=np.uint64)
    _load().oracle_rank_within_digit(_ptr(d), d.size, _ptr(rank))
    return rank


# ------------------------------------------------------------ u32 sorting

def all_pass_histograms(keys, begin_bit: int, end_bit: int, digit_bits: int) -> np.ndarray:
    k = _u32(keys)
    P = num_passes(begin_bit, end_bit, digit_bits)
    hist = np.zeros((max(P, 0), 1 << digit_bits), dtype=np.uint64)
    _check(_load().oracle_all_pass_histograms(_ptr(k), k.size, begin_bit, end_bit, digit_bits,
                                              _ptr(hist)), "all_pass_histograms")
    return hist


def radix_sort_pairs(keys, vals=None, begin_bit: int = 0, end_bit: int = 32,
                     digit_bits: int = 8, backward: bool = False):
    """Stable LSD sort by bits [begin_bit, end_bit).  Returns (keys, vals-or-None)."""
    k = _u32(keys)
    v = None if vals is None else _u32(vals)
    if v is not None and v.size != k.size:
        raise ValueError("keys and vals differ in length")
    ko = np.empty_like(k)
    vo = None if v is None else np.empty_like(v)
    _check(_load().oracle_radix_sort_pairs(_ptr(k), _ptr(v), _ptr(ko), _ptr(vo), k.size,
                                           begin_bit, end_bit, digit_bits, int(backward)),
           "radix_sort_pairs")
    return ko, vo


def radix_sort_keys(keys, begin_bit: int = 0, end_bit: int = 32, digit_bits: int = 8,
                    backward: bool = False) -> np.ndarray:
    return radix_sort_pairs(keys, None, begin_bit, end_bit, digit_bits, backward)[0]


def stable_position(keys: np.ndarray, begin_bit: int, end_bit: int, i: int) -> int:
    k = _u32(keys)
    return int(_load().oracle_stable_position(_ptr(k), k.size, begin_bit, end_bit, int(i)))


# ------------------------------------------------------ typed 32-bit keys

KEY_TYPES = {"u32": 0, "i32": 1, "f32": 2, "u64": 3, "i64": 4, "f64": 5}


def key64(bits: int, key_type: str, descending: bool = False) -> int:
    """Order-preserving u64 image of one 64-bit pattern of the given type."""
    out = np.zeros(1, dtype=np.uint64)
    _check(_load().oracle_key64(int(bits) & 0xFFFFFFFFFFFFFFFF, KEY_TYPES[key_type], int(descending), _ptr(out)),
           "key64")
    return int(out[0])


def key32(bits: int, key_type: str, descending: bool = False) -> int:
    """Order-preserving u32 image of one 32-bit pattern of the given type."""
    out = np.zeros(1, dtype=np.uint32)
    _check(_load().oracle_key32(int(bits) & 0xFFFFFFFF, KEY_TYPES[key_type], int(descending), _ptr(out)),
           "key32")
    return int(out[0])


def radix_sort_typed(keys, vals=None, key_type: str = "u32", descending: bool = False,
                     begin_bit: int = 0, end_bit: int = 32, digit_bits: int = 8):
    """Stable sort of 32- or 64-bit keys (bit patterns of u32/i32/f32 or u64/i64/f64) by
    their image's bit window; returns (key patterns, vals-or-None) in sorted order."""
    if key_type.endswith("64"):
        k = np.ascontiguousarray(np.asarray(keys).view(np.uint64))
        v = None if vals is None else _u32(vals)
        if v is not None and v.size != k.size:
            raise ValueError("keys and vals differ in length")
        ko = np.empty_like(k)
        vo = None if v is None else np.empty_like(v)
        _check(_load().oracle_radix_sort_typed64(_ptr(k), _ptr(v), _ptr(ko), _ptr(vo), k.size, KEY_TYPES[key_type],
                                                 int(descending), begin_bit, end_bit, digit_bits), "radix_sort_typed64")
        return ko, vo
    k = np.ascontiguousarray(np.asarray(keys).view(np.uint32))
    v = None if vals is None else _u32(vals)
    if v is not None and v.size != k.size:
        raise ValueError("keys and vals differ in length")
    ko = np.empty_like(k)
    vo = None if v is None else np.empty_like(v)
    _check(_load().oracle_radix_sort_typed(_ptr(k), _ptr(v), _ptr(ko), _ptr(vo), k.size, KEY_TYPES[key_type],
                                           int(descending), begin_bit, end_bit, digit_bits), "radix_sort_typed")
    return ko, vo


# ------------------------------------------------------- 16-bit float rows

def float16_key(bits: int, descending: bool = False) -> int:
    return int(_load().oracle_float16_key(bits, int(descending)))


def float16_keys(bits: np.ndarray, descending: bool = False) -> np.ndarray:
    """Vector form of float16_key, one C call per element (small inputs only)."""
    f = _load().oracle_float16_key
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([f(int(b), int(descending)) for b in flat], dtype=np.uint16).reshape(np.shape(bits))


def segmented_row_sort(vals, descending: bool = False, digit_bits: int = 8):
    """Sort every row of a 2-D uint16 array of fp16/bf16 bit patterns.

    Returns (sorted bit patterns uint16[rows, n], int64 column indices [rows, n]).
    """
    u = np.ascontiguousarray(np.asarray(vals, dtype=np.uint16))
    if u.ndim != 2:
        raise ValueError("expected a 2-D array")
    rows, n = u.shape
    vo = np.empty_like(u)
    io = np.empty((rows, n), dtype=np.int64)
    _check(_load().oracle_segmented_row_sort(_ptr(u), _ptr(vo), _ptr(io), rows, n,
                                             int(descending), digit_bits), "segmented_row_sort")
    return vo, io


def segmented_histograms(vals, descending: bool, digit_bits: int) -> np.ndarray:
    u = np.ascontiguousarray(np.asarray(vals, dtype=np.uint16))
    rows, n = u.shape
    P = num_passes(0, 16, digit_bits)
    hist = np.zeros((rows, P, 1 << digit_bits), dtype=np.uint64)
    _check(_load().oracle_segmented_histograms(_ptr(u), rows, n, int(descending), digit_bits,
                                               _ptr(hist)), "segmented_histograms")
    return hist


def row_stable_position(row: np.ndarray, descending: bool, j: int) -> int:
    r = np.ascontiguousarray(np.asarray(row, dtype=np.uint16))
    return int(_load().oracle_row_stable_position(_ptr(r), r.size, int(descending), int(j)))
