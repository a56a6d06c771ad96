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
pins (``tests/test_oracle_layer.py``). The layer's backward (:func:`layer_bwd`)
is the chain rule of these steps, pinned by central finite differences of
:func:`layer_fwd` on small shapes.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_bwd, attention_fwd, attention_fwd_rows, silu

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


def layernorm_bwd(a: np.ndarray, d_ln: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    """dA of LayerNorm over the last axis (unit scale, zero shift) from dLN:
    with xh = (a - mu) / sigma, dA = (dLN - mean(dLN) - xh * mean(dLN * xh)) / sigma."""
    a = np.asarray(a, dtype=np.float64)
    d_ln = np.asarray(d_ln, dtype=np.float64)
    mu = a.mean(axis=-1, keepdims=True)
    sigma = np.sqrt(((a - mu) ** 2).mean(axis=-1, keepdims=True) + eps)
    xh = (a - mu) / sigma
    return (d_ln - d_ln.mean(axis=-1, keepdims=True)
            - xh * (d_ln * xh).mean(axis=-1, keepdims=True)) / sigma


def layer_bwd(x, w1, b1, w2, b2, seq_offsets, num_targets, heads, head_dim, dy):
    """Gradients of sum(Y * dy) for :func:`layer_fwd`: dict dx, dw1, db1, dw2, db2.

    The chain rule of the forward's steps, in reverse:
        Z = LayerNorm(A) * U:  dW2 = Z^T dY, db2 = sum_rows dY, dZ = dY W2^T
        dU = dZ * LayerNorm(A),  dA = LayerNorm'(A)^T (dZ * U)
        dQ, dK, dV = attention backward with dO = dA (no gate, no rab)
        dPre = [dU, dV, dQ, dK] * SiLU'(Pre),  Pre = X W1 + b1,
               SiLU'(z) = s(z) (1 + z (1 - s(z))), s the logistic sigmoid
        dW1 = X^T dPre,  db1 = sum_rows dPre,  dX = dPre W1^T
    """
    x = np.asarray(x, dtype=np.float64)
    w1 = np.asarray(w1, np.float64)
    w2 = np.asarray(w2, np.float64)
    dy = np.asarray(dy, np.float64)
    T = x.shape[0]
    HD = heads * head_dim
    pre = x @ w1 + np.asarray(b1, np.float64)
    uvqk = silu(pre)
    u, v, q, k = split_uvqk(uvqk, heads, head_dim)
    max_len = int(np.max(np.diff(np.asarray(seq_offsets)))) if len(seq_offsets) > 1 else 1
    max_len = max(max_len, 1)
    _, a = attention_fwd(q, k, v, None, seq_offsets, max_len, num_targets)
    a2 = a.reshape(T, HD)
    ln = layernorm(a2)
    u2 = u.reshape(T, HD)
    z = ln * u2
    dw2 = z.T @ dy
    db2 = dy.sum(axis=0)
    dz = dy @ w2.T
    du = dz * ln
    da = layernorm_bwd(a2, dz * u2)
    g = attention_bwd(q, k, v, None, seq_offsets, max_len, da.reshape(T, heads, head_dim),
                      num_targets)
    d_uvqk = np.concatenate([du, g["dv"].reshape(T, HD), g["dq"].reshape(T, HD),
                             g["dk"].reshape(T, HD)], axis=1)
    sig = 1.0 / (1.0 + np.exp(-pre))
    d_pre = d_uvqk * sig * (1.0 + pre * (1.0 - sig))
    return dict(dx=d_pre @ w1.T, dw1=x.T @ d_pre, db1=d_pre.sum(axis=0), dw2=dw2, db2=db2)
