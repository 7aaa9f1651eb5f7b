"""Seeded synthetic inputs for the five sort workloads.

This module only draws random numbers; it holds none of the sort's arithmetic.
Both the GPU tests/bench and the CPU oracle take their inputs from here, so both
sides see byte-identical data.

Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), written out from its published
definition: the state advances by the golden-ratio increment 0x9E3779B97F4A7C15
and each output is the state passed through the 64-bit finaliser
    z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27; z *= 0x94D049BB133111EB;
    z ^= z >> 31.
Draw i of a stream seeded with s is therefore mix(s + (i + 1) * 0x9E3779B97F4A7C15),
which vectorises.  A u32 is the high 32 bits of one draw.  A standard normal is
Box-Muller on two draws in float64 (cosine branch only).  fp16 values are the
float64 normal rounded to nearest-even by numpy; bf16 values are built from
exactly representable levels so no rounding is involved.

Workloads (each seeded with 0x5EED0000 + k, k the workload's index):
  0  1,024 u32 keys uniform in [0, 4096); keys only; 4-bit digits over bits 0..11
  1  4,194,304 u32 keys uniform over 32 bits; keys only; 4-bit and 8-bit digits
  2  2^28 u32 keys + u32 values (value = index); 8-bit digits; uniform keys, or
     keys = AND of three independent uniform words (skewed buckets)
  3  fp16 matrix (1024, 65536), N(0,1); rows sorted ascending; 4-bit digits
  4  bf16 matrix (4096, 4096), N(0,1) rounded to 64 levels k/8,
     k = clamp(round_half_even(8x), -32, 31); rows sorted descending; 8-bit digits
"""
from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
SEED_BASE = 0x5EED0000
_CHUNK = 1 << 22


def seed_of(k: int) -> int:
    return SEED_BASE + k


def splitmix64(seed: int, count: int, start: int = 0) -> np.ndarray:
    """Draws start .. start+count-1 of the SplitMix64 stream seeded with `seed`."""
    out = np.empty(count, dtype=np.uint64)
    s = np.uint64(seed & 0xFFFFFFFFFFFFFFFF)
    with np.errstate(over="ignore"):
        for lo in range(0, count, _CHUNK):
            hi = min(count, lo + _CHUNK)
            i = np.arange(start + lo + 1, start + hi + 1, dtype=np.uint64)
            z = s + i * GOLDEN
            z ^= z >> np.uint64(30)
            z *= _M1
            z ^= z >> np.uint64(27)
            z *= _M2
            z ^= z >> np.uint64(31)
            out[lo:hi] = z
    return out


def uniform_u32(seed: int, count: int, start: int = 0) -> np.ndarray:
    out = np.empty(count, dtype=np.uint32)
    for lo in range(0, count, _CHUNK):
        hi = min(count, lo + _CHUNK)
        out[lo:hi] = (splitmix64(seed, hi - lo, start + lo) >> np.uint64(32)).astype(np.uint32)
    return out


def _unit(draws: np.ndarray) -> np.ndarray:
    """Map 64-bit draws to float64 in [0, 1) using their top 53 bits."""
    return (draws >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def normal_f64(seed: int, count: int) -> np.ndarray:
    """Box-Muller: z = sqrt(-2 ln(1 - u1)) cos(2 pi u2) from draws 2i and 2i+1."""
    out = np.empty(count, dtype=np.float64)
    for lo in range(0, count, _CHUNK):
        hi = min(count, lo + _CHUNK)
        d = splitmix64(seed, 2 * (hi - lo), 2 * lo)
        u1 = _unit(d[0::2])
        u2 = _unit(d[1::2])
        out[lo:hi] = np.sqrt(-2.0 * np.log1p(-u1)) * np.cos(2.0 * np.pi * u2)
    return out


def fp16_normal_bits(seed: int, count: int) -> np.ndarray:
    return normal_f64(seed, count).astype(np.float16).view(np.uint16)


def bf16_64level_bits(seed: int, count: int) -> np.ndarray:
    """bf16 patterns of k/8 for k = clamp(rne(8x), -32, 31); all exactly representable."""
    x = normal_f64(seed, count)
    k = np.clip(np.rint(8.0 * x), -32, 31) + 0.0  # + 0.0 turns a rounded -0 into +0
    v = (k / 8.0).astype(np.float32)
    # bf16 = high half of the float32 pattern; exact for these values (<= 5 significant bits)
    bits = (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    assert np.all((v.view(np.uint32) & np.uint32(0xFFFF)) == 0)
    return bits


# -------------------------------------------------------------- workloads

WORKLOADS = {
    "c1_keys_1k_4bit": dict(index=0, kind="keys", n=1024, begin_bit=0, end_bit=12, digit_bits=(4,)),
    "c2_keys_4m": dict(index=1, kind="keys", n=4194304, begin_bit=0, end_bit=32, digit_bits=(4, 8)),
    "c3_pairs_2p28_uniform": dict(index=2, kind="pairs", n=1 << 28, begin_bit=0, end_bit=32,
                                  digit_bits=(8,), dist="uniform"),
    "c3_pairs_2p28_and3": dict(index=2, kind="pairs", n=1 << 28, begin_bit=0, end_bit=32,
                               digit_bits=(8,), dist="and3"),
    "c4_fp16_1024x65536_asc": dict(index=3, kind="segmented", rows=1024, cols=65536,
                                   dtype="fp16", descending=False, digit_bits=(4,)),
    "c5_bf16_4096x4096_desc": dict(index=4, kind="segmented", rows=4096, cols=4096,
                                   dtype="bf16", descending=True, digit_bits=(8,)),
    # typed 32-bit keys (not one of the five configurations; the same sizes as the pair sort)
    "f32_pairs_2p28_desc": dict(index=5, kind="typed_pairs", n=1 << 28, key_type="f32",
                                descending=True, digit_bits=(8,)),
    "i32_keys_2p28_asc": dict(index=6, kind="typed_keys", n=1 << 28, key_type="i32",
                              descending=False, digit_bits=(8,)),
    "f64_pairs_2p27_asc": dict(index=7, kind="typed_pairs", n=1 << 27, key_type="f64",
                               descending=False, digit_bits=(8,)),
}


def keys_c1(n: int = 1024) -> np.ndarray:
    return uniform_u32(seed_of(0), n) & np.uint32(0xFFF)


def keys_c2(n: int = 4194304) -> np.ndarray:
    return uniform_u32(seed_of(1), n)


def pairs_c3(n: int = 1 << 28, dist: str = "uniform"):
    """Keys and values (value = original index) of the 2^28-pair workload.

    Uniform keys are draws 0..n-1 of the stream; AND-3 keys use draws
    0..n-1, n..2n-1 and 2n..3n-1 as the three words.
    """
    seed = seed_of(2)
    if dist == "uniform":
        keys = uniform_u32(seed, n)
    elif dist == "and3":
        keys = uniform_u32(seed, n, 0)
        keys &= uniform_u32(seed, n, n)
        keys &= uniform_u32(seed, n, 2 * n)
    else:
        raise ValueError(dist)
    vals = np.arange(n, dtype=np.uint32)
    return keys, vals


def matrix_c4(rows: int = 1024, cols: int = 65536) -> np.ndarray:
    return fp16_normal_bits(seed_of(3), rows * cols).reshape(rows, cols)


def matrix_c5(rows: int = 4096, cols: int = 4096) -> np.ndarray:
    return bf16_64level_bits(seed_of(4), rows * cols).reshape(rows, cols)


def keys_f32_normal(n: int = 1 << 28) -> np.ndarray:
    """Bit patterns (uint32) of N(0,1) draws (Box-Muller in fp64) rounded to
    binary32; the typed-key workload."""
    return normal_f64(seed_of(5), n).astype(np.float32).view(np.uint32)


def keys_f64_normal(n: int = 1 << 27) -> np.ndarray:
    """Bit patterns (uint64) of N(0,1) draws (Box-Muller in fp64)."""
    return normal_f64(seed_of(7), n).view(np.uint64)


def keys_i32_uniform(n: int = 1 << 28) -> np.ndarray:
    """Bit patterns (uint32) of uniform signed 32-bit integers."""
    return uniform_u32(seed_of(6), n)


def random_u32(seed: int, n: int) -> np.ndarray:
    """Generic seeded u32 keys for fuzz cases."""
    return uniform_u32(seed, n)
