"""Relative-attention-bias buckets (oracle; test infrastructure only).

Position buckets: one bucket per relative offset j - p_i, clamped to
+-(max_len-1), so a table holds 2*max_len - 1 entries (the bucket counts of
the pages' workloads: 99, 399, 2047 and 16383 for max_len 50, 200, 1024,
8192). A query's position p_i is its index, except that candidates appended
for M-FALCON-style scoring all sit at position ``hist`` (the first candidate
slot), so they see the history as the first candidate would.

Time buckets: floor(log2(|ts_i - ts_j| + 1)) computed exactly in integers as
bitlen(|dt| + 1) - 1, then clamped to the last bucket.

Parity pins: ``tests/test_oracle_buckets.py`` (special values, brute force
with Python's ``int.bit_length``).
"""
from __future__ import annotations

import numpy as np


def position_buckets(rows: np.ndarray, cols: np.ndarray, hist: int, max_len: int) -> np.ndarray:
    """bp[r, c] for query indices ``rows`` and key indices ``cols`` (int64)."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    p = np.minimum(rows, hist)
    rel = cols[None, :] - p[:, None]
    lim = max_len - 1
    return np.clip(rel, -lim, lim) + lim


def bit_length_u64(x: np.ndarray) -> np.ndarray:
    """Exact bit length of unsigned 64-bit integers (0 -> 0)."""
    y = np.asarray(x, dtype=np.uint64).copy()
    out = np.zeros(y.shape, dtype=np.int64)
    for s in (32, 16, 8, 4, 2, 1):
        big = y >= (np.uint64(1) << np.uint64(s))
        out += np.where(big, s, 0)
        y = np.where(big, y >> np.uint64(s), y)
    out += (y > 0).astype(np.int64)
    return out


def time_buckets(ts_rows: np.ndarray, ts_cols: np.ndarray, n_buckets: int) -> np.ndarray:
    """bt[r, c] = min(bitlen(|ts_rows[r] - ts_cols[c]| + 1) - 1, n_buckets - 1).

    Differences are taken in unsigned 64-bit arithmetic so that no int64
    overflow can occur for any pair of int64 timestamps.
    """
    a = np.asarray(ts_rows, dtype=np.int64)[:, None]
    b = np.asarray(ts_cols, dtype=np.int64)[None, :]
    ua = a.astype(np.uint64)  # two's complement reinterpretation
    ub = b.astype(np.uint64)
    ge = a >= b
    with np.errstate(over="ignore"):
        absdiff = np.where(ge, ua - ub, ub - ua)      # exact modulo 2^64, true value < 2^64
        plus1 = absdiff + np.uint64(1)                 # wraps to 0 only for |dt| = 2^64 - 1
    bl = bit_length_u64(plus1)
    bl = np.where(plus1 == 0, 65, bl)                  # |dt| + 1 = 2^64 has bit length 65
    return np.minimum(bl - 1, n_buckets - 1)
