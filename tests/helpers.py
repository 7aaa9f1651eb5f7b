"""Shared test helpers: fixture parsing and the properties that characterise a
stable sort (sorted by the windowed key, a permutation of the input carried by
an index payload, equal keys keeping input order).  Together the three
properties fix the unique stable result, so they also check outputs too large
for the full oracle."""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_fixture(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = v.split()
    return out


def ints(tokens) -> list[int]:
    return [int(t) for t in tokens]


def tagged(tokens) -> tuple[list[int], list[int]]:
    vals, tags = [], []
    for t in tokens:
        v, i = t.split("@")
        vals.append(int(v))
        tags.append(int(i))
    return vals, tags


def window(keys: np.ndarray, begin_bit: int, end_bit: int) -> np.ndarray:
    k = keys.astype(np.uint64)
    mask = np.uint64((1 << (end_bit - begin_bit)) - 1)
    return (k >> np.uint64(begin_bit)) & mask


def check_stable_sort_by_index(keys_in: np.ndarray, keys_out: np.ndarray, idx_out: np.ndarray,
                               wkey_out: np.ndarray | None = None):
    """Invariants of a stable sort whose payload is the original index.

    wkey_out: the windowed (ordering) key of each output element; defaults to keys_out.
    Raises AssertionError naming the first failing index.
    """
    n = keys_in.size
    assert keys_out.size == n and idx_out.size == n
    if n == 0:
        return
    idx = idx_out.astype(np.int64)
    # permutation of [0, n)
    assert idx.min() >= 0 and idx.max() < n, "payload out of range"
    seen = np.zeros(n, dtype=bool)
    seen[idx] = True
    assert seen.all(), f"payload is not a permutation: first missing {int(np.argmin(seen))}"
    # every key travelled with its payload
    bad = np.nonzero(keys_out != keys_in[idx])[0]
    assert bad.size == 0, f"key/payload mismatch at {int(bad[0])}"
    w = keys_out if wkey_out is None else wkey_out
    w = w.astype(np.int64)
    d = np.diff(w)
    bad = np.nonzero(d < 0)[0]
    assert bad.size == 0, f"not sorted at {int(bad[0]) + 1}"
    ties = d == 0
    bad = np.nonzero(ties & (np.diff(idx) <= 0))[0]
    assert bad.size == 0, f"unstable at {int(bad[0]) + 1}: payloads {idx[bad[0]]}, {idx[bad[0] + 1]}"
