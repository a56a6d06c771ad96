"""Autograd entry point and the HSTU layer forward built on the C ABI."""
from __future__ import annotations

import torch

from . import ops


class _HstuAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, u, rab_pos, rab_time, seq_offsets, max_len, num_targets, timestamps):
        o, a = ops.attn_fwd(q, k, v, u, seq_offsets, max_len, num_targets=num_targets,
                            timestamps=timestamps, rab_pos=rab_pos, rab_time=rab_time,
                            save_a=u is not None)
        ctx.save_for_backward(q, k, v, u, rab_pos, rab_time, seq_offsets, num_targets,
                              timestamps, a)
        ctx.max_len = max_len
        return o

    @staticmethod
    def backward(ctx, d_o):
        q, k, v, u, rab_pos, rab_time, seq_offsets, num_targets, timestamps, a = ctx.saved_tensors
        g = ops.attn_bwd(q, k, v, u, seq_offsets, ctx.max_len, a, d_o, num_targets=num_targets,
                         timestamps=timestamps, rab_pos=rab_pos, rab_time=rab_time)
        return (g["dq"], g["dk"], g["dv"], g["du"], g["d_rab_pos"], g["d_rab_time"],
                None, None, None, None)


def hstu_attention(q, k, v, u, seq_offsets, max_len, *, num_targets=None, timestamps=None,
                   rab_pos=None, rab_time=None):
    """Jagged causal HSTU pointwise attention, differentiable in q, k, v, u and the rab tables.

    q, k: [T, H, D]; v, u: [T, H, D] (u may be None: no gate); seq_offsets int64
    [B+1] on the device; rab_pos [Hr, 2*max_len-1], rab_time [Hr, NT] fp32 with
    int64 timestamps [T]; num_targets int64 [B] marks appended candidates.
    """
    return _HstuAttention.apply(q, k, v, u, rab_pos, rab_time, seq_offsets, max_len,
                                num_targets, timestamps)


def hstu_layer_fwd(x, w1, b1, w2, b2, seq_offsets, num_targets, heads: int, head_dim: int,
                   eps: float = 1e-5):
    """One HSTU layer forward: Y = (LayerNorm(A) * U) W2 + b2 with A the attention of
    the SiLU'd UVQK projection (column blocks U, V, Q, K; head h at [h*D, (h+1)*D)).

    Returns (y [T, d_model] bf16, a [T, H*D] fp32, uvqk [T, 4*H*D] bf16).
    """
    T = x.shape[0]
    HD = heads * head_dim
    uvqk = ops.linear(x, w1, b1, silu=True)
    u, v, q, k = (uvqk[:, n * HD:(n + 1) * HD].view(T, heads, head_dim) for n in range(4))
    _, a = ops.attn_fwd(q, k, v, None, seq_offsets, 1, num_targets=num_targets, save_a=True)
    a2 = a.view(T, HD)
    g = ops.layernorm_gate(a2, uvqk[:, 0:HD], eps)
    y = ops.linear(g, w2, b2, silu=False)
    return y, a2, uvqk


def hstu_layer_bwd(x, w1, b1, w2, seq_offsets, num_targets, heads: int, head_dim: int, uvqk, a,
                   dy, eps: float = 1e-5):
    """Gradients of :func:`hstu_layer_fwd` from dY: dict dx, dw1, db1, dw2, db2
    (uvqk and a as the forward returned them)."""
    return ops.layer_bwd(x, w1, b1, w2, seq_offsets, num_targets, heads, head_dim, uvqk, a, dy,
                         eps)
