"""CPU oracle for jagged HSTU pointwise attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product path (the HIP library and its Python
binding) never calls it and shares no code with it.

What it computes
----------------
The pages name the method -- HSTU, a sequential transducer for large-vocabulary,
drifting streams of user actions (Abstract of "Actions Speak Louder than Words:
Trillion-Parameter Sequential Transducers for Generative Recommendations"), its
target-aware full causal self-attention and M-FALCON
(Generative Recommenders README, "HSTU Ultra attention benchmark" and the
introduction) -- but print none of its equations. The oracle is the plain
definition of the pointwise attention those passages name, per sequence b of
length L and head h, over in-sequence indices 0 <= i, j < L:

    mask   M[i,j]  = (j <= i and j < hist) or j == i,  hist = L - num_targets
    bias   B[i,j]  = rab_pos[hr, bp(i,j)] + rab_time[hr, bt(i,j)]
    score  S[i,j]  = sum_d Q[i,d] K[j,d] + B[i,j]
    prob   P[i,j]  = M[i,j] * SiLU(S[i,j]) / L,   SiLU(x) = x / (1 + exp(-x))
    out    A[i]    = sum_j P[i,j] V[j];  O[i] = A[i] * U[i]  (gate on) or A[i]

    bp(i,j) = clamp(j - p_i, -(max_len-1), max_len-1) + (max_len-1),
              p_i = min(i, hist)
    bt(i,j) = min(bitlen(|ts_i - ts_j| + 1) - 1, n_time_buckets - 1)

Backward from dO: dA = dO*U, dU = dO*A, dP = dA V^T,
dS = M * dP * SiLU'(S) / L with SiLU'(x) = s(x)(1 + x(1 - s(x))), s the
logistic sigmoid; dQ = dS K, dK = dS^T Q, dV = P^T dA, and each rab table's
gradient is the sum of dS over the unmasked pairs that read that entry
(summed over heads when one table is shared by all heads).

Every step is float64 (bf16 inputs are taken as the exact values they hold),
except FP8 quantisation (``oracle.fp8``), whose codes are integers decided in
float32, the kernel's precision.
Which checks pin these functions is stated in each function's docstring and
in ``tests/test_oracle_*.py``.
"""
from .buckets import position_buckets, time_buckets, bit_length_u64
from .attention import attention_fwd, attention_bwd, attention_fwd_rows, silu
from .scalar import scalar_attention_fwd, scalar_attention_bwd
from .layer import layer_fwd, layernorm
from . import fp8

__all__ = [
    "position_buckets", "time_buckets", "bit_length_u64",
    "attention_fwd", "attention_bwd", "attention_fwd_rows", "silu",
    "scalar_attention_fwd", "scalar_attention_bwd", "layer_fwd", "layernorm",
]
