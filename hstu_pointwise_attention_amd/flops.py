"""Host-side work accounting: unmasked pairs and algorithmic FLOPs.

FLOPs are counted over unmasked (sequence, head, i, j) pairs only: the
forward does 2*Dqk (Q K^T) + 2*Dv (P V) per pair; the backward recomputes
Q K^T and does dA' V^T, s^T dA', dS^T Q and dS K, i.e. 6*Dqk + 4*Dv (the
FlashAttention convention: backward = 2.5 x forward).
"""
from __future__ import annotations


def unmasked_pairs_host(lengths, num_targets=None) -> int:
    total = 0
    for b, L in enumerate(lengths):
        L = int(L)
        nt = 0 if num_targets is None else min(max(int(num_targets[b]), 0), L)
        hist = L - nt
        total += hist * (hist + 1) // 2 + nt * (hist + 1)
    return total


def attention_flops(lengths, heads: int, d_qk: int, d_v: int, num_targets=None) -> dict:
    """Algorithmic FLOPs of the step and of each attention kernel.

    The backward's algorithmic work is split over two kernels: the
    key-block kernel ("bwd") does Q K^T, dA' V^T, s^T dA' and dS^T Q
    (4*Dqk + 4*Dv per pair); the query-block kernel ("dq") owns dS K
    (2*Dqk). The latter also recomputes Q K^T and dA' V^T, which is not
    counted.
    """
    pairs = unmasked_pairs_host(lengths, num_targets) * heads
    fwd = pairs * (2 * d_qk + 2 * d_v)
    bwd = pairs * (6 * d_qk + 4 * d_v)
    kernels = {"fwd": fwd, "bwd": pairs * (4 * d_qk + 4 * d_v), "dq": pairs * 2 * d_qk}
    return dict(pair_heads=pairs, fwd=fwd, bwd=bwd, total=fwd + bwd, kernels=kernels)
