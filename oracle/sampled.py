"""Oracle values at sampled places of full-size workloads -- TEST INFRASTRUCTURE ONLY.

The same definition as ``oracle/attention.py`` (written out in
``oracle/__init__.py``), evaluated only where a full-size check looks:

* rows of dQ and dU: for query i, S, P and dS over all of its keys;
* key rows of dK and dV: for key j, S, P and dS over all of its queries;
* sums of dS along one diagonal j - i = delta, over sequences, heads and
  rows. Without candidates, and with every sequence no longer than
  max_len, such a diagonal is exactly the set of pairs that read position
  bucket delta + max_len - 1, so the sum is that entry of d_rab_pos (summed
  over heads when one table is shared);
* the whole rab-table gradients (``rab_gradients``): dS over every unmasked
  pair, added into the bucket each pair reads, without forming dQ, dK or dV.

Each sampled item costs O(L * D) in float64, so 8192-long sequences are
cheap; the rab gradients cost the pairs' S and dP (two matrix products per
block of rows) and may spread the (sequence, head) units over worker
processes, whose per-unit tables are added in unit order.
Pins: the scalar brute force of ``oracle/scalar.py`` on tiny inputs with
candidates and both rab tables (``tests/test_oracle_sampled.py``).
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, _rab_head, _seq_meta, _sigmoid
from .buckets import bit_length_u64, position_buckets, time_buckets


def locate(seq_offsets, token: int):
    """(sequence index, in-sequence index) of a global token row."""
    offs = np.asarray(seq_offsets, dtype=np.int64)
    b = int(np.searchsorted(offs, token, side="right") - 1)
    return b, int(token - offs[b])


def _grid_terms(q, k, v, dA, s, L, hist, max_len, timestamps, rab_pos, rab_time, h, hr, rows, cols):
    """P and dS on the grid rows x cols (in-sequence indices) of one sequence and head."""
    S = q[s + rows, h, :] @ k[s + cols, h, :].T
    if rab_pos is not None:
        S = S + rab_pos[hr][position_buckets(rows, cols, hist, max_len)]
    if rab_time is not None:
        ts = np.asarray(timestamps[s:s + L], dtype=np.int64)
        S = S + rab_time[hr][time_buckets(ts[rows], ts[cols], rab_time.shape[1])]
    m = ((cols[None, :] <= rows[:, None]) & (cols[None, :] < hist)) | (cols[None, :] == rows[:, None])
    sg = _sigmoid(S)
    P = np.where(m, S * sg, 0.0) / L
    dP = dA[s + rows, h, :] @ v[s + cols, h, :].T
    dS = np.where(m, dP * sg * (1.0 + S * (1.0 - sg)), 0.0) / L
    return P, dS


def _prep(q, k, v, u, d_o, rab_pos, rab_time):
    q, k, v, u, d_o = _f64(q), _f64(k), _f64(v), _f64(u), _f64(d_o)
    dA = d_o * u if u is not None else d_o
    return q, k, v, u, d_o, dA, _f64(rab_pos), _f64(rab_time)


def attention_bwd_rows(q, k, v, u, seq_offsets, max_len, d_o, token_rows, num_targets=None,
                       timestamps=None, rab_pos=None, rab_time=None):
    """dQ and dU at the given global query rows: ``(dq [n, H, Dqk], du [n, H, Dv] or None)``."""
    q, k, v, u, d_o, dA, rab_pos, rab_time = _prep(q, k, v, u, d_o, rab_pos, rab_time)
    H = q.shape[1]
    n = len(token_rows)
    dq = np.zeros((n, H, q.shape[2]))
    du = np.zeros((n, H, v.shape[2])) if u is not None else None
    for r, t in enumerate(token_rows):
        b, i = locate(seq_offsets, int(t))
        s, e, L, hist = _seq_meta(seq_offsets, num_targets, b)
        rows, cols = np.array([i]), np.arange(L)
        for h in range(H):
            hr = _rab_head(h, rab_pos, rab_time)
            P, dS = _grid_terms(q, k, v, dA, s, L, hist, max_len, timestamps, rab_pos, rab_time,
                                h, hr, rows, cols)
            dq[r, h] = dS[0] @ k[s:e, h, :]
            if du is not None:
                du[r, h] = d_o[s + i, h] * (P[0] @ v[s:e, h, :])
    return dq, du


def attention_bwd_cols(q, k, v, u, seq_offsets, max_len, d_o, token_cols, num_targets=None,
                       timestamps=None, rab_pos=None, rab_time=None):
    """dK and dV at the given global key rows: ``(dk [n, H, Dqk], dv [n, H, Dv])``."""
    q, k, v, u, d_o, dA, rab_pos, rab_time = _prep(q, k, v, u, d_o, rab_pos, rab_time)
    H = q.shape[1]
    n = len(token_cols)
    dk = np.zeros((n, H, q.shape[2]))
    dv = np.zeros((n, H, v.shape[2]))
    for c, t in enumerate(token_cols):
        b, j = locate(seq_offsets, int(t))
        s, e, L, hist = _seq_meta(seq_offsets, num_targets, b)
        rows, cols = np.arange(L), np.array([j])
        for h in range(H):
            hr = _rab_head(h, rab_pos, rab_time)
            P, dS = _grid_terms(q, k, v, dA, s, L, hist, max_len, timestamps, rab_pos, rab_time,
                                h, hr, rows, cols)
            dk[c, h] = dS[:, 0] @ q[s:e, h, :]
            dv[c, h] = P[:, 0] @ dA[s:e, h, :]
    return dk, dv


def _time_bucket_pairs(ts_a: np.ndarray, ts_b: np.ndarray, n_buckets: int) -> np.ndarray:
    """Element-wise time bucket of the pairs (ts_a[m], ts_b[m])."""
    a = np.asarray(ts_a, dtype=np.int64)
    b = np.asarray(ts_b, dtype=np.int64)
    ua, ub = a.astype(np.uint64), b.astype(np.uint64)
    with np.errstate(over="ignore"):
        plus1 = np.where(a >= b, ua - ub, ub - ua) + np.uint64(1)
    bl = np.where(plus1 == 0, 65, bit_length_u64(plus1))
    return np.minimum(bl - 1, n_buckets - 1)


def diagonal_ds_sums(q, k, v, u, seq_offsets, max_len, d_o, deltas, timestamps=None,
                     rab_pos=None, rab_time=None):
    """For each delta <= 0: sum of dS_ij over all sequences, heads and rows with j = i + delta.

    No candidates (every row a history row). Returns ``[len(deltas)]`` when
    the rab tables are shared by all heads (or absent), else ``[H, len(deltas)]``.
    """
    q, k, v, u, d_o, dA, rab_pos, rab_time = _prep(q, k, v, u, d_o, rab_pos, rab_time)
    H = q.shape[1]
    shared = _rab_head(1, rab_pos, rab_time) == 0
    out = np.zeros((H, len(deltas)))
    for b in range(len(seq_offsets) - 1):
        s, e, L, hist = _seq_meta(seq_offsets, None, b)
        ts = None if timestamps is None else np.asarray(timestamps[s:e], dtype=np.int64)
        for n, delta in enumerate(deltas):
            delta = int(delta)
            assert delta <= 0
            rows = np.arange(-delta, L)
            if rows.size == 0:
                continue
            cols = rows + delta
            for h in range(H):
                hr = _rab_head(h, rab_pos, rab_time)
                S = np.einsum("md,md->m", q[s + rows, h, :], k[s + cols, h, :])
                if rab_pos is not None:
                    lim = max_len - 1
                    S = S + rab_pos[hr][np.clip(cols - np.minimum(rows, hist), -lim, lim) + lim]
                if rab_time is not None:
                    S = S + rab_time[hr][_time_bucket_pairs(ts[rows], ts[cols], rab_time.shape[1])]
                sg = _sigmoid(S)
                dP = np.einsum("md,md->m", dA[s + rows, h, :], v[s + cols, h, :])
                out[h, n] += float(np.sum(dP * sg * (1.0 + S * (1.0 - sg)))) / L
    return out.sum(axis=0) if shared else out


def _one_blas_thread():
    """Worker processes use one BLAS thread each (the processes are the parallelism)."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:  # pragma: no cover
        pass


def _rab_unit(args):
    """d_rab_pos / d_rab_time contributions of one (sequence, head)."""
    (q, k, v, dA, s, L, hist, max_len, ts, rab_pos_row, rab_time_row, n_pos, n_time, rows_per) = args
    gp = np.zeros(n_pos) if rab_pos_row is not None else None
    gt = np.zeros(n_time) if rab_time_row is not None else None
    for r0 in range(0, L, rows_per):
        rows = np.arange(r0, min(L, r0 + rows_per))
        cols = np.arange(rows[-1] + 1)                 # every unmasked pair has j <= i
        S = q[rows] @ k[cols].T
        bp = position_buckets(rows, cols, hist, max_len) if gp is not None else None
        bt = time_buckets(ts[rows], ts[cols], n_time) if gt is not None else None
        if bp is not None:
            S = S + rab_pos_row[bp]
        if bt is not None:
            S = S + rab_time_row[bt]
        m = ((cols[None, :] <= rows[:, None]) & (cols[None, :] < hist)) | (cols[None, :] == rows[:, None])
        sg = _sigmoid(S)
        dP = dA[rows] @ v[cols].T
        dS = np.where(m, dP * sg * (1.0 + S * (1.0 - sg)), 0.0) / L
        if gp is not None:
            gp += np.bincount(bp[m], weights=dS[m], minlength=n_pos)
        if gt is not None:
            gt += np.bincount(bt[m], weights=dS[m], minlength=n_time)
    return gp, gt


def rab_gradients(q, k, v, u, seq_offsets, max_len, d_o, num_targets=None, timestamps=None,
                  rab_pos=None, rab_time=None, workers: int = 1, rows_per: int = 256):
    """The rab-table gradients of the backward: ``(d_rab_pos or None, d_rab_time or None)``.

    Entry p of a table is the sum of dS_ij over the unmasked pairs (b, h, i, j)
    whose bucket is p, over the heads that read that table row. The (sequence,
    head) units run in ``workers`` processes (1: in this one); their tables
    are added in unit order.
    """
    q, k, v, u, d_o, dA, rab_pos, rab_time = _prep(q, k, v, u, d_o, rab_pos, rab_time)
    H = q.shape[1]
    tab = rab_pos if rab_pos is not None else rab_time
    Hr = 1 if tab is None else tab.shape[0]
    n_pos = 2 * max_len - 1
    n_time = rab_time.shape[1] if rab_time is not None else 0
    units, dest = [], []
    for b in range(len(seq_offsets) - 1):
        s, e, L, hist = _seq_meta(seq_offsets, num_targets, b)
        if L == 0:
            continue
        ts = None if timestamps is None else np.asarray(timestamps[s:e], dtype=np.int64)
        for h in range(H):
            hr = _rab_head(h, rab_pos, rab_time)
            units.append((np.ascontiguousarray(q[s:e, h]), np.ascontiguousarray(k[s:e, h]),
                          np.ascontiguousarray(v[s:e, h]), np.ascontiguousarray(dA[s:e, h]), s, L,
                          hist, max_len, ts, None if rab_pos is None else rab_pos[hr],
                          None if rab_time is None else rab_time[hr], n_pos, n_time, rows_per))
            dest.append(hr)
    if workers > 1 and len(units) > 1:
        import multiprocessing as mp
        with mp.get_context("fork").Pool(min(workers, len(units)), initializer=_one_blas_thread) as pool:
            parts = pool.map(_rab_unit, units, chunksize=1)
    else:
        parts = [_rab_unit(a) for a in units]
    gp = np.zeros((Hr, n_pos)) if rab_pos is not None else None
    gt = np.zeros((Hr, n_time)) if rab_time is not None else None
    for hr, (a, c) in zip(dest, parts):
        if gp is not None:
            gp[hr] += a
        if gt is not None:
            gt[hr] += c
    return gp, gt
