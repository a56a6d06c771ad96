"""Pure-Python scalar evaluation of the same definition (tiny inputs only).

Written independently of ``oracle/attention.py`` -- plain loops, Python
floats (IEEE double), ``math.exp`` and ``int.bit_length`` -- so the two
cross-check each other. Test infrastructure only.
"""
from __future__ import annotations

import math


def _sig(x: float) -> float:
    if x < -700.0:
        return 0.0
    return 1.0 / (1.0 + math.exp(-x))


def _pos_bucket(i: int, j: int, hist: int, max_len: int) -> int:
    p = i if i < hist else hist
    rel = j - p
    lim = max_len - 1
    rel = max(-lim, min(lim, rel))
    return rel + lim


def _time_bucket(ti: int, tj: int, nb: int) -> int:
    return min((abs(int(ti) - int(tj)) + 1).bit_length() - 1, nb - 1)


def _rows(x):
    return None if x is None else [[[float(e) for e in hd] for hd in tok] for tok in x]


def _table(x):
    return None if x is None else [[float(e) for e in row] for row in x]


def _pairs(seq_offsets, num_targets):
    """Yields (s, L, hist, i, j) for unmasked pairs, in sequence/row/col order."""
    for b in range(len(seq_offsets) - 1):
        s = int(seq_offsets[b])
        L = int(seq_offsets[b + 1]) - s
        hist = L - (0 if num_targets is None else int(num_targets[b]))
        for i in range(L):
            for j in range(L):
                if (j <= i and j < hist) or j == i:
                    yield s, L, hist, i, j


def _score(q, k, s, h, i, j, hist, max_len, ts, rp, rt):
    acc = 0.0
    for d in range(len(q[s + i][h])):
        acc += q[s + i][h][d] * k[s + j][h][d]
    hr = 0
    tab = rp if rp is not None else rt
    if tab is not None and len(tab) > 1:
        hr = h
    if rp is not None:
        acc += rp[hr][_pos_bucket(i, j, hist, max_len)]
    if rt is not None:
        acc += rt[hr][_time_bucket(ts[s + i], ts[s + j], len(rt[hr]))]
    return acc, hr


def scalar_attention_fwd(q, k, v, u, seq_offsets, max_len, num_targets=None, timestamps=None,
                         rab_pos=None, rab_time=None):
    """Returns (O, A) as nested Python lists [T][H][Dv]."""
    q, k, v, u = _rows(q), _rows(k), _rows(v), _rows(u)
    rp, rt = _table(rab_pos), _table(rab_time)
    ts = None if timestamps is None else [int(t) for t in timestamps]
    T, H, Dv = len(q), len(q[0]) if q else 0, len(v[0][0]) if v else 0
    A = [[[0.0] * Dv for _ in range(H)] for _ in range(T)]
    for s, L, hist, i, j in _pairs(seq_offsets, num_targets):
        for h in range(H):
            sc, _ = _score(q, k, s, h, i, j, hist, max_len, ts, rp, rt)
            p = sc * _sig(sc) / L
            for d in range(Dv):
                A[s + i][h][d] += p * v[s + j][h][d]
    if u is None:
        O = [[list(r) for r in tok] for tok in A]
    else:
        O = [[[A[t][h][d] * u[t][h][d] for d in range(Dv)] for h in range(H)] for t in range(T)]
    return O, A


def scalar_attention_bwd(q, k, v, u, seq_offsets, max_len, d_o, num_targets=None,
                         timestamps=None, rab_pos=None, rab_time=None):
    """Returns dict of nested lists: dq, dk, dv, du, d_rab_pos, d_rab_time."""
    _, A = scalar_attention_fwd(q, k, v, u, seq_offsets, max_len, num_targets, timestamps,
                                rab_pos, rab_time)
    q, k, v, u, d_o = _rows(q), _rows(k), _rows(v), _rows(u), _rows(d_o)
    rp, rt = _table(rab_pos), _table(rab_time)
    ts = None if timestamps is None else [int(t) for t in timestamps]
    T, H = len(q), len(q[0]) if q else 0
    Dq, Dv = (len(q[0][0]) if q else 0), (len(v[0][0]) if v else 0)
    dA = [[[d_o[t][h][d] * (u[t][h][d] if u is not None else 1.0) for d in range(Dv)]
           for h in range(H)] for t in range(T)]
    du = None if u is None else \
        [[[d_o[t][h][d] * A[t][h][d] for d in range(Dv)] for h in range(H)] for t in range(T)]
    dq = [[[0.0] * Dq for _ in range(H)] for _ in range(T)]
    dk = [[[0.0] * Dq for _ in range(H)] for _ in range(T)]
    dv = [[[0.0] * Dv for _ in range(H)] for _ in range(T)]
    dp_tab = None if rp is None else [[0.0] * len(r) for r in rp]
    dt_tab = None if rt is None else [[0.0] * len(r) for r in rt]
    for s, L, hist, i, j in _pairs(seq_offsets, num_targets):
        for h in range(H):
            sc, hr = _score(q, k, s, h, i, j, hist, max_len, ts, rp, rt)
            sg = _sig(sc)
            p = sc * sg / L
            dp = 0.0
            for d in range(Dv):
                dv[s + j][h][d] += p * dA[s + i][h][d]
                dp += dA[s + i][h][d] * v[s + j][h][d]
            ds = dp * sg * (1.0 + sc * (1.0 - sg)) / L
            for d in range(Dq):
                dq[s + i][h][d] += ds * k[s + j][h][d]
                dk[s + j][h][d] += ds * q[s + i][h][d]
            if dp_tab is not None:
                dp_tab[hr][_pos_bucket(i, j, hist, max_len)] += ds
            if dt_tab is not None:
                dt_tab[hr][_time_bucket(ts[s + i], ts[s + j], len(rt[hr]))] += ds
    return dict(dq=dq, dk=dk, dv=dv, du=du, d_rab_pos=dp_tab, d_rab_time=dt_tab)
