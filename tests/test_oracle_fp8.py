"""Pins of oracle.fp8 to things other than itself: torch's CPU float8_e4m3fn
conversion (a library routine for the same format), the format's closed-form
values, exact cases where quantisation loses nothing, and the error bound of
3-bit-mantissa rounding."""
import numpy as np
import pytest

from oracle import fp8 as F
from oracle.layer import layernorm


def _torch_e4m3(v):
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch has no float8_e4m3fn")
    t = torch.from_numpy(np.asarray(v, np.float32))
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_closed_form_values():
    """Facts of the E4M3FN format: 1.0 is 0x38, the largest finite value 448 is
    0x7E, the smallest normal 2^-6 is 0x08, the smallest subnormal 2^-9 is 0x01,
    0x7F / 0xFF are NaN, and the sign is the top bit."""
    d = F.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert d[0x38] == 1.0 and d[0x7E] == 448.0 and d[0x08] == 2.0 ** -6 and d[0x01] == 2.0 ** -9
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert np.all(d[0x80:0xFF][~np.isnan(d[0x80:0xFF])] == -d[0x00:0x7F][~np.isnan(d[0x00:0x7F])])
    finite = d[~np.isnan(d)]
    assert finite.size == 254 and np.max(finite) == 448.0
    # positive finite codes decode to increasing values
    assert np.all(np.diff(d[0x00:0x7F]) > 0)


def test_round_matches_torch_cast():
    """Nearest-even rounding agrees with torch's float8_e4m3fn cast on random
    magnitudes over the whole range, subnormals included, and on every
    midpoint between adjacent codes (ties)."""
    rng = np.random.default_rng(0)
    mags = np.exp2(rng.uniform(-12, np.log2(460), 20000))
    v = (mags * rng.choice([-1, 1], mags.size)).astype(np.float32)
    assert np.array_equal(F.e4m3_round(v), _torch_e4m3(v))
    grid = F.e4m3_decode(np.arange(0x00, 0x7F, dtype=np.uint8))
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
    assert np.array_equal(F.e4m3_round(mids), _torch_e4m3(mids))
    assert np.array_equal(F.e4m3_round(-mids), _torch_e4m3(-mids))


def test_ties_to_even_and_saturation():
    # between 1.0 (0x38, mantissa 0) and 1.125 (0x39) the tie goes to 1.0;
    # between 1.125 and 1.25 (mantissa 2) it goes to 1.25
    assert F.e4m3_round(1.0625) == 1.0
    assert F.e4m3_round(1.1875) == 1.25
    assert F.e4m3_round(2.0 ** -10) == 0.0            # half the smallest subnormal: tie to 0
    assert F.e4m3_round(3 * 2.0 ** -10) == 2.0 ** -8   # 1.5 subnormal steps: tie to 2 steps
    assert F.e4m3_round(463.9) == 448.0 and F.e4m3_round(1e6) == 448.0
    assert F.e4m3_round(-1e6) == -448.0


def test_encode_decode_round_trip():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = F.e4m3_decode(codes)
    assert np.array_equal(F.e4m3_encode(vals), codes)
    assert np.array_equal(F.e4m3_round(vals), vals)


def test_quantize_rows_exact_when_on_grid():
    """Rows built as E4M3 values times a power of two, each holding +-448 times
    that power, quantise without loss: scale = the power, codes = the values."""
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, size=(6, 40)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C
    codes[:, 7] = 0x7E
    codes[2, 7] = 0xFE                                 # -448 as the row's extreme
    p = np.exp2(np.array([-8, -3, 0, 2, 5, 9], np.float64))
    x = F.e4m3_decode(codes) * p[:, None]
    q, s = F.quantize_rows(x)
    assert np.array_equal(s.astype(np.float64), p)
    assert np.array_equal(F.e4m3_decode(q), F.e4m3_decode(codes))


def test_quantize_zero_row_and_scales_per_row():
    x = np.zeros((3, 16), np.float32)
    x[1, 3] = -2.0
    x[2] = np.linspace(-1, 4, 16)
    q, s = F.quantize_rows(x)
    assert s[0] == 1.0 and np.all(q[0] == 0)
    assert s[1] == np.float32(2.0) / np.float32(448.0)
    assert F.e4m3_decode(q[1, 3]) == -448.0
    assert F.e4m3_decode(q[2, -1]) == 448.0


def test_addmm_exact_on_grid():
    """With on-grid inputs, different scales per row and per output feature, the
    FP8 addmm equals x w + b exactly (a transposed operand or scale would not)."""
    rng = np.random.default_rng(2)
    M, K, N = 5, 24, 7
    cx = rng.integers(0, 0x77, size=(M, K)).astype(np.uint8) | (rng.integers(0, 2, (M, K)) << 7).astype(np.uint8)
    cw = rng.integers(0, 0x77, size=(K, N)).astype(np.uint8)
    cx[:, 0] = 0x7E
    cw[0, :] = 0x7E
    px = np.exp2(rng.integers(-4, 5, M).astype(np.float64))
    pw = np.exp2(rng.integers(-4, 5, N).astype(np.float64))
    x = F.e4m3_decode(cx) * px[:, None]
    w = F.e4m3_decode(cw) * pw[None, :]
    b = rng.standard_normal(N)
    xq, xs = F.quantize_rows(x)
    wq, ws = F.quantize_weight(w)
    assert wq.shape == (N, K)
    y = F.fp8_addmm(xq, xs, wq, ws, b)
    assert np.array_equal(y, x @ w + b)
    assert np.allclose(F.fp8_linear(xq, xs, wq, ws, b, apply_silu=True),
                       (x @ w + b) / (1 + np.exp(-(x @ w + b))), rtol=1e-15, atol=0)


def test_addmm_error_bound():
    """Each quantised element is within a relative 2^-4 of its value (3
    mantissa bits, nearest rounding) or within half the smallest subnormal
    step times the scale, so |y_q - x w| <= sum_k |x||w| (2 * 2^-4 + 2^-8) + tiny."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((32, 64)).astype(np.float32)
    w = (rng.standard_normal((64, 48)) / 8).astype(np.float32)
    xq, xs = F.quantize_rows(x)
    wq, ws = F.quantize_weight(w)
    y = F.fp8_addmm(xq, xs, wq, ws)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    bound = np.abs(x).astype(np.float64) @ np.abs(w).astype(np.float64) * (2 * 2.0 ** -4 + 2.0 ** -8)
    sub = 2.0 ** -10 * (np.abs(x).max() * np.abs(ws).max() * 448 + np.abs(w).max() * np.abs(xs).max() * 448) * 64
    assert np.all(np.abs(y - ref) <= bound + sub)
    # and quantisation is not the identity: a real error is present
    assert np.max(np.abs(y - ref)) > 0


def test_layernorm_gate_fp8_dequantises_to_layernorm_times_gate():
    rng = np.random.default_rng(4)
    a = rng.standard_normal((10, 128)) * 3 + 1
    u = rng.standard_normal((10, 128))
    q, s = F.layernorm_gate_fp8(a, u)
    z = layernorm(a) * u
    deq = F.e4m3_decode(q) * s[:, None].astype(np.float64)
    amax = np.max(np.abs(z), axis=1, keepdims=True)
    assert np.all(np.abs(deq - z) <= 2.0 ** -4 * np.abs(z) + 2.0 ** -10 * amax / 448 * 2)
    assert np.allclose(np.max(np.abs(deq), axis=1), amax[:, 0], rtol=1e-6)


def test_layer_fwd_fp8_close_to_layer_fwd():
    """The FP8 layer stays within FP8 rounding of the unquantised layer
    (rel-L2 of Y below 2^-3), and is not the unquantised layer itself."""
    from oracle.layer import layer_fwd
    rng = np.random.default_rng(5)
    offs = np.array([0, 40, 97], np.int64)
    nt = np.array([8, 5], np.int64)
    x = rng.standard_normal((97, 64))
    w1 = rng.standard_normal((64, 4 * 64)) / 8
    w2 = rng.standard_normal((64, 64)) / 8
    b1, b2 = 0.1 * rng.standard_normal(256), 0.1 * rng.standard_normal(64)
    ref = layer_fwd(x, w1, b1, w2, b2, offs, nt, 2, 32)
    got = F.layer_fwd_fp8(x, w1, b1, w2, b2, offs, nt, 2, 32)
    e = np.linalg.norm(got["y"] - ref["y"]) / np.linalg.norm(ref["y"])
    assert 1e-4 < e < 2.0 ** -3, e
