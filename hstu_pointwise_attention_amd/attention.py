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


def prepare_fp8_weights(w1, w2):
    """E4M3 codes and per-output-feature scales of the layer's two projection
    weights (w1 [d_model, 4*H*D], w2 [H*D, d_model]), computed once and kept."""
    w1q, w1s = ops.fp8_prepare_weight(w1)
    w2q, w2s = ops.fp8_prepare_weight(w2)
    return dict(w1q=w1q, w1s=w1s, w2q=w2q, w2s=w2s)


def hstu_layer_fwd_fp8(x, fp8_weights, b1, b2, seq_offsets, num_targets, heads: int,
                       head_dim: int, eps: float = 1e-5):
    """:func:`hstu_layer_fwd` with both projections in FP8: X quantised row-wise,
    UVQK = SiLU(FP8 GEMM with the prepared W1 + b1), the attention, LayerNorm(A) * U
    quantised row-wise in the same kernel, Y = FP8 GEMM with the prepared W2 + b2.

    Returns (y [T, d_model] bf16, a [T, H*D] fp32, uvqk [T, 4*H*D] bf16).
    """
    T = x.shape[0]
    HD = heads * head_dim
    w = fp8_weights
    xq, xs = ops.fp8_quantize_rows(x)
    uvqk = ops.fp8_linear(xq, xs, w["w1q"], w["w1s"], b1, silu=True)
    u, v, q, k = (uvqk[:, n * HD:(n + 1) * HD].view(T, heads, head_dim) for n in range(4))
    _, a = ops.attn_fwd(q, k, v, None, seq_offsets, 1, num_targets=num_targets, save_a=True)
    a2 = a.view(T, HD)
    zq, zs = ops.layernorm_gate_fp8(a2, uvqk[:, 0:HD], eps)
    y = ops.fp8_linear(zq, zs, w["w2q"], w["w2s"], b2, silu=False)
    return y, a2, uvqk


def hstu_layer_bwd(x, w1, b1, w2, seq_offsets, num_targets, heads: int, head_dim: int, uvqk, a,
                   dy, eps: float = 1e-5, max_len: int = 0):
    """Gradients of :func:`hstu_layer_fwd` from dY: dict dx, dw1, db1, dw2, db2
    (uvqk and a as the forward returned them; max_len, when given, bounds the
    sequence lengths and lets the attention backward export dS)."""
    return ops.layer_bwd(x, w1, b1, w2, seq_offsets, num_targets, heads, head_dim, uvqk, a, dy,
                         eps, max_len)
