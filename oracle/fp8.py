"""Oracle of the FP8 (E4M3) row-wise quantised projection -- TEST INFRASTRUCTURE ONLY.

The Generative Recommenders README ("FP8 linear reference and benchmark", and
the HSTU Ultra stack description before it) names the steps: row-wise E4M3
quantisation, an FP8 addmm whose weights may be quantised once and cached,
and LayerNorm / output-normalisation-and-gating steps fused with the
quantisation of their output. It gives no formulas. Readings taken (the
plainest that the rest supports):

  * E4M3 is the OCP 8-bit float E4M3FN: sign, 4 exponent bits with bias 7,
    3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6; no
    infinities; codes 0x7F and 0xFF are NaN; the largest finite magnitude is
    1.75 * 2^8 = 448 and the smallest positive one 2^-9. Values round to the
    nearest code, ties to the even mantissa, and saturate at +-448.
  * Row-wise quantisation of a row r: scale s_r = amax_r / 448 (s_r = 1 for a
    row of zeros) and codes E4M3(x / s_r). The codes are integers decided by
    floating point, so the scale and the quotient are taken in float32, the
    kernel's precision (numpy float32 arithmetic rounds as IEEE does).
  * A weight W [K, N] of y = x W is quantised per output feature n (per row
    of W^T) and kept as codes [N, K] with scales [N].
  * FP8 addmm: y[m, n] = s_x[m] s_w[n] sum_k x_q[m, k] w_q[n, k] + bias[n],
    exact here (float64), then the projection's activation (SiLU for UVQK).
  * LayerNorm-and-gate to FP8: z = LayerNorm(a) * u per row as in
    oracle.layer, rounded to float32, then row-wise quantisation of z.

Pins: tests/test_oracle_fp8.py (torch's CPU float8_e4m3fn conversion, the
format's closed-form values, exact cases and the error bound).
"""
from __future__ import annotations

import numpy as np

from .attention import attention_fwd, silu
from .layer import layernorm, split_uvqk

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6          # smallest normal binade: 2^-6
_MANT_BITS = 3


def e4m3_round(v) -> np.ndarray:
    """Nearest E4M3FN value of each element (ties to even), saturating at +-448."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)                      # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, _MIN_NORMAL_EXP)  # binade exponent; subnormals share 2^-6's spacing
    ulp = np.ldexp(1.0, e - _MANT_BITS)
    q = np.round(a / ulp) * ulp              # np.round: half to even; a / ulp is exact
    q = np.minimum(q, E4M3_MAX)
    return np.where(np.signbit(v), -q, q)


def e4m3_encode(v) -> np.ndarray:
    """Codes (uint8) of values already on the E4M3 grid (e.g. e4m3_round's output)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    sign = np.signbit(v).astype(np.uint8) << 7
    _, ex = np.frexp(a)
    normal = a >= 2.0 ** _MIN_NORMAL_EXP
    e = np.where(normal, ex - 1, _MIN_NORMAL_EXP)
    field = np.where(normal, e + 7, 0)
    mant = np.where(normal, a / np.ldexp(1.0, e) - 1.0, a / 2.0 ** _MIN_NORMAL_EXP) * 8
    assert np.all(mant == np.round(mant)), "value not on the E4M3 grid"
    return (sign | (field.astype(np.uint8) << 3) | mant.astype(np.uint8)).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """Values (float64) of E4M3FN codes; NaN for 0x7F and 0xFF."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    field = (c >> 3) & 0xF
    mant = c & 0x7
    val = np.where(field == 0, mant / 8.0 * 2.0 ** _MIN_NORMAL_EXP,
                   (1.0 + mant / 8.0) * np.ldexp(1.0, field - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


def quantize_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Row-wise E4M3 quantisation of x [M, K]: codes uint8 [M, K], scales float32 [M]."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    quotient = (x / scale[:, None]).astype(np.float32)
    return e4m3_encode(e4m3_round(quotient)), scale


def quantize_weight(w) -> tuple[np.ndarray, np.ndarray]:
    """Weight W [K, N] quantised per output feature: codes [N, K], scales [N]."""
    return quantize_rows(np.asarray(w, dtype=np.float32).T)


def fp8_addmm(xq, x_scale, wq, w_scale, bias=None) -> np.ndarray:
    """y = s_x s_w (x_q w_q^T) + bias in float64, wq stored [N, K]."""
    y = e4m3_decode(xq) @ e4m3_decode(wq).T
    y = y * np.asarray(x_scale, np.float64)[:, None] * np.asarray(w_scale, np.float64)[None, :]
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    return y


def fp8_linear(xq, x_scale, wq, w_scale, bias=None, apply_silu: bool = False) -> np.ndarray:
    y = fp8_addmm(xq, x_scale, wq, w_scale, bias)
    return silu(y) if apply_silu else y


def layernorm_gate_fp8(a, u, eps: float = 1e-5) -> tuple[np.ndarray, np.ndarray]:
    """Codes and scales of the row-wise quantisation of LayerNorm(a) * u."""
    z = (layernorm(a, eps) * np.asarray(u, np.float64)).astype(np.float32)
    return quantize_rows(z)


def layer_fwd_fp8(x, w1, b1, w2, b2, seq_offsets, num_targets, heads, head_dim,
                  eps: float = 1e-5):
    """oracle.layer.layer_fwd with both projections in FP8 (the README's
    fp8_addmm_fwd layer): X quantised row-wise, UVQK = SiLU(FP8 addmm with the
    prepared W1), attention as before, LayerNorm(A) * U quantised row-wise in
    the same step, Y = FP8 addmm with the prepared W2. Returns dict uvqk, a, y."""
    xq, xs = quantize_rows(x)
    w1q, w1s = quantize_weight(w1)
    uvqk = fp8_linear(xq, xs, w1q, w1s, b1, apply_silu=True)
    u, v, q, k = split_uvqk(uvqk, heads, head_dim)
    offs = np.asarray(seq_offsets)
    max_len = max(int(np.max(np.diff(offs))) if len(offs) > 1 else 1, 1)
    _, a = attention_fwd(q, k, v, None, offs, max_len, num_targets)
    T = uvqk.shape[0]
    a2 = a.reshape(T, heads * head_dim)
    zq, zs = layernorm_gate_fp8(a2, u.reshape(T, heads * head_dim), eps)
    w2q, w2s = quantize_weight(w2)
    return dict(uvqk=uvqk, a=a2, y=fp8_addmm(zq, zs, w2q, w2s, b2))
