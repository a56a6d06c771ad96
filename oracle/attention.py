"""Vectorised float64 oracle of jagged HSTU attention (test infrastructure only).

The definition is written out in ``oracle/__init__.py``. This module
evaluates it per sequence and head, a block of query rows at a time so that
8192-long sequences fit in memory; blocking over rows is the only reordering
and each row's sum still runs over all of its keys in one matrix product.

Pins: scalar brute force (``oracle/scalar.py``), closed forms (Q=0 and
zero bias gives 0; K=0 gives SiLU(bias)/N times a prefix sum of V),
the L=1 case, the L/(L+1) rescaling when a token is appended, causality,
batch-order independence, linearity, finite differences and autograd of an
independent torch formulation (``tests/test_oracle_attention.py``).
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .buckets import position_buckets, time_buckets


def silu(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _rab_head(h, rab_pos, rab_time):
    """Row of the rab tables used by head h: 0 when one table is shared."""
    tab = rab_pos if rab_pos is not None else rab_time
    return 0 if tab is None or tab.shape[0] == 1 else h


def _seq_meta(seq_offsets, num_targets, b):
    s = int(seq_offsets[b])
    e = int(seq_offsets[b + 1])
    L = e - s
    nt = 0 if num_targets is None else int(num_targets[b])
    return s, e, L, L - nt


def _mask(rows: np.ndarray, L: int, hist: int) -> np.ndarray:
    cols = np.arange(L)
    return ((cols[None, :] <= rows[:, None]) & (cols[None, :] < hist)) | \
        (cols[None, :] == rows[:, None])


def _bias(rows, L, hist, s, max_len, timestamps, rab_pos, rab_time, hr):
    """Bias block [len(rows), L] for rab head ``hr`` (0 where a table is absent)."""
    bias = np.zeros((len(rows), L))
    cols = np.arange(L)
    if rab_pos is not None:
        bias += rab_pos[hr][position_buckets(rows, cols, hist, max_len)]
    if rab_time is not None:
        ts = timestamps[s:s + L]
        bias += rab_time[hr][time_buckets(ts[rows], ts, rab_time.shape[1])]
    return bias


def _buckets(rows, L, hist, s, max_len, timestamps, rab_pos, rab_time):
    cols = np.arange(L)
    bp = position_buckets(rows, cols, hist, max_len) if rab_pos is not None else None
    bt = None
    if rab_time is not None:
        ts = timestamps[s:s + L]
        bt = time_buckets(ts[rows], ts, rab_time.shape[1])
    return bp, bt


def attention_fwd(q, k, v, u, seq_offsets, max_len, num_targets=None, timestamps=None,
                  rab_pos=None, rab_time=None, chunk_rows: int = 1024):
    """Forward: returns (O, A), both float64 ``[T, H, Dv]``.

    ``u`` None means no gate (O = A). ``rab_pos`` ``[Hr, 2*max_len-1]`` and
    ``rab_time`` ``[Hr, NT]`` may each be None (term absent); Hr is 1 (shared)
    or H.
    """
    q, k, v, u = _f64(q), _f64(k), _f64(v), _f64(u)
    rab_pos, rab_time = _f64(rab_pos), _f64(rab_time)
    T, H, _ = q.shape
    Dv = v.shape[2]
    A = np.zeros((T, H, Dv))
    B = len(seq_offsets) - 1
    for b in range(B):
        s, e, L, hist = _seq_meta(seq_offsets, num_targets, b)
        for r0 in range(0, L, chunk_rows):
            rows = np.arange(r0, min(L, r0 + chunk_rows))
            m = _mask(rows, L, hist)
            for h in range(H):
                hr = _rab_head(h, rab_pos, rab_time)
                S = q[s + rows, h, :] @ k[s:e, h, :].T
                S += _bias(rows, L, hist, s, max_len, timestamps, rab_pos, rab_time, hr)
                P = np.where(m, silu(S), 0.0) / L
                A[s + rows, h, :] = P @ v[s:e, h, :]
    O = A * u if u is not None else A.copy()
    return O, A


def attention_fwd_rows(q, k, v, u, seq_offsets, max_len, token_rows, num_targets=None,
                       timestamps=None, rab_pos=None, rab_time=None):
    """Forward for selected global token rows only: (O, A) of shape [n, H, Dv].

    Same definition as :func:`attention_fwd`; used to check sampled outputs of
    full-size workloads without evaluating every row.
    """
    q, k, v, u = _f64(q), _f64(k), _f64(v), _f64(u)
    rab_pos, rab_time = _f64(rab_pos), _f64(rab_time)
    token_rows = np.asarray(token_rows, dtype=np.int64)
    H = q.shape[1]
    Dv = v.shape[2]
    A = np.zeros((len(token_rows), H, Dv))
    seq_of = np.searchsorted(np.asarray(seq_offsets), token_rows, side="right") - 1
    for n, (t, b) in enumerate(zip(token_rows.tolist(), seq_of.tolist())):
        s, e, L, hist = _seq_meta(seq_offsets, num_targets, b)
        rows = np.array([t - s])
        m = _mask(rows, L, hist)
        for h in range(H):
            hr = _rab_head(h, rab_pos, rab_time)
            S = q[t:t + 1, h, :] @ k[s:e, h, :].T
            S += _bias(rows, L, hist, s, max_len, timestamps, rab_pos, rab_time, hr)
            P = np.where(m, silu(S), 0.0) / L
            A[n, h, :] = (P @ v[s:e, h, :])[0]
    O = A * u[token_rows] if u is not None else A.copy()
    return O, A


def attention_bwd(q, k, v, u, seq_offsets, max_len, d_o, num_targets=None, timestamps=None,
                  rab_pos=None, rab_time=None, chunk_rows: int = 1024):
    """Backward: returns dict dq, dk, dv, du (None without gate), d_rab_pos, d_rab_time.

    Recomputes A from the inputs (the oracle keeps no state between calls).
    """
    q, k, v, u, d_o = _f64(q), _f64(k), _f64(v), _f64(u), _f64(d_o)
    rab_pos, rab_time = _f64(rab_pos), _f64(rab_time)
    T, H, Dq = q.shape
    Dv = v.shape[2]
    _, A = attention_fwd(q, k, v, u, seq_offsets, max_len, num_targets, timestamps,
                         rab_pos, rab_time, chunk_rows)
    dA = d_o * u if u is not None else d_o
    du = d_o * A if u is not None else None
    dq = np.zeros((T, H, Dq))
    dk = np.zeros((T, H, Dq))
    dv = np.zeros((T, H, Dv))
    d_pos = np.zeros_like(rab_pos) if rab_pos is not None else None
    d_time = np.zeros_like(rab_time) if rab_time is not None else None
    B = len(seq_offsets) - 1
    for b in range(B):
        s, e, L, hist = _seq_meta(seq_offsets, num_targets, b)
        for r0 in range(0, L, chunk_rows):
            rows = np.arange(r0, min(L, r0 + chunk_rows))
            m = _mask(rows, L, hist)
            bp, bt = _buckets(rows, L, hist, s, max_len, timestamps, rab_pos, rab_time)
            for h in range(H):
                hr = _rab_head(h, rab_pos, rab_time)
                S = q[s + rows, h, :] @ k[s:e, h, :].T
                S += _bias(rows, L, hist, s, max_len, timestamps, rab_pos, rab_time, hr)
                sig = _sigmoid(S)
                P = np.where(m, S * sig, 0.0) / L
                dAr = dA[s + rows, h, :]
                dv[s:e, h, :] += P.T @ dAr
                dP = dAr @ v[s:e, h, :].T
                dS = np.where(m, dP * sig * (1.0 + S * (1.0 - sig)), 0.0) / L
                dq[s + rows, h, :] = dS @ k[s:e, h, :]
                dk[s:e, h, :] += dS.T @ q[s + rows, h, :]
                if d_pos is not None:
                    d_pos[hr] += np.bincount(bp[m], weights=dS[m], minlength=d_pos.shape[1])
                if d_time is not None:
                    d_time[hr] += np.bincount(bt[m], weights=dS[m], minlength=d_time.shape[1])
    return dict(dq=dq, dk=dk, dv=dv, du=du, d_rab_pos=d_pos, d_rab_time=d_time)


def unmasked_pairs(seq_offsets, num_targets=None) -> int:
    """Number of (i, j) pairs with M[i, j] = 1, summed over sequences."""
    total = 0
    for b in range(len(seq_offsets) - 1):
        _, _, L, hist = _seq_meta(seq_offsets, num_targets, b)
        total += hist * (hist + 1) // 2 + (L - hist) * (hist + 1)
    return total
