"""Float64 oracle of one HSTU layer forward around the attention (test infrastructure only).

The Generative Recommenders README ("HSTU Ultra attention benchmark" and "FP8
linear reference and benchmark") lists a layer's steps: a UVQK projection
(``hstu_compute_uqvk``), the attention, then output normalisation, gating and
the output projection (``hstu_compute_output``). The plainest reading taken
here, for the M-FALCON-style inference layer workload:

    UVQK = SiLU(X W1 + b1)                      [T, 4*H*D]
    U, V, Q, K = column blocks of UVQK, in that order; head h of each block
                 occupies columns [h*D, (h+1)*D)
    A    = attention(Q, K, V; no gate, no rab, candidates masked)   [T, H*D]
    Y    = (LayerNorm(A) * U) W2 + b2,  LayerNorm over the H*D features of a
           token, eps 1e-5, unit scale, zero shift.

Pins: LayerNorm moments, brute-force GEMMs, and the attention oracle's own
pins (``tests/test_oracle_layer.py``).
"""
from __future__ import annotations

import numpy as np

from .attention import attention_fwd, attention_fwd_rows, silu

LN_EPS = 1e-5


def layernorm(a: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    mu = a.mean(axis=-1, keepdims=True)
    var = ((a - mu) ** 2).mean(axis=-1, keepdims=True)
    return (a - mu) / np.sqrt(var + eps)


def split_uvqk(uvqk: np.ndarray, heads: int, head_dim: int):
    T = uvqk.shape[0]
    w = heads * head_dim
    blocks = [uvqk[:, n * w:(n + 1) * w].reshape(T, heads, head_dim) for n in range(4)]
    return tuple(blocks)  # U, V, Q, K


def layer_fwd(x, w1, b1, w2, b2, seq_offsets, num_targets, heads, head_dim,
              chunk_rows: int = 1024):
    """Returns dict with uvqk, a (attention output, [T, H*D]) and y ([T, d_model])."""
    x = np.asarray(x, dtype=np.float64)
    uvqk = silu(x @ np.asarray(w1, np.float64) + np.asarray(b1, np.float64))
    u, v, q, k = split_uvqk(uvqk, heads, head_dim)
    max_len = int(np.max(np.diff(np.asarray(seq_offsets)))) if len(seq_offsets) > 1 else 1
    _, a = attention_fwd(q, k, v, None, seq_offsets, max(max_len, 1), num_targets,
                         None, None, None, chunk_rows)
    T = x.shape[0]
    a2 = a.reshape(T, heads * head_dim)
    y = (layernorm(a2) * u.reshape(T, heads * head_dim)) @ np.asarray(w2, np.float64) \
        + np.asarray(b2, np.float64)
    return dict(uvqk=uvqk, a=a2, y=y)


def layer_fwd_rows(x, w1, b1, w2, b2, seq_offsets, num_targets, heads, head_dim, token_rows):
    """uvqk, a and y of :func:`layer_fwd` at selected global rows only.

    The projection is evaluated for the sequences that hold those rows (a
    row's attention reads its whole sequence), the attention and the output
    steps for the rows themselves.
    """
    x = np.asarray(x, dtype=np.float64)
    w1 = np.asarray(w1, np.float64)
    w2 = np.asarray(w2, np.float64)
    offs = np.asarray(seq_offsets, dtype=np.int64)
    token_rows = np.asarray(token_rows, dtype=np.int64)
    n, HD = len(token_rows), heads * head_dim
    out = dict(uvqk=np.zeros((n, 4 * HD)), a=np.zeros((n, HD)), y=np.zeros((n, w2.shape[1])))
    seqs = np.searchsorted(offs, token_rows, side="right") - 1
    for b in np.unique(seqs):
        s, e = int(offs[b]), int(offs[b + 1])
        uvqk = silu(x[s:e] @ w1 + np.asarray(b1, np.float64))
        u, v, q, k = split_uvqk(uvqk, heads, head_dim)
        sel = np.nonzero(seqs == b)[0]
        rows = token_rows[sel] - s
        nt = None if num_targets is None else np.array([int(num_targets[b])])
        _, a = attention_fwd_rows(q, k, v, None, np.array([0, e - s]), max(e - s, 1), rows, nt)
        a2 = a.reshape(len(rows), HD)
        out["uvqk"][sel] = uvqk[rows]
        out["a"][sel] = a2
        out["y"][sel] = (layernorm(a2) * u[rows].reshape(len(rows), HD)) @ w2 \
            + np.asarray(b2, np.float64)
    return out
