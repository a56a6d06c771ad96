"""Pins of the layer oracle (CPU only)."""
import numpy as np

import oracle
from oracle.layer import layer_fwd_rows, split_uvqk


def test_layernorm_moments():
    rng = np.random.default_rng(0)
    a = 5.0 + 3.0 * rng.standard_normal((7, 512))
    y = oracle.layernorm(a)
    var = a.var(axis=1)
    assert np.allclose(y.mean(axis=1), 0.0, atol=1e-12)
    assert np.allclose(y.var(axis=1), var / (var + 1e-5), rtol=1e-12)


def test_layer_bruteforce_tiny():
    """GEMMs, SiLU, split order and LN of the layer against scalar loops."""
    import math
    rng = np.random.default_rng(1)
    H, D, dm = 2, 3, 4
    offs = np.array([0, 4, 7])
    nt = np.array([1, 2])
    T = 7
    x = rng.standard_normal((T, dm))
    w1 = 0.5 * rng.standard_normal((dm, 4 * H * D))
    b1 = 0.1 * rng.standard_normal(4 * H * D)
    w2 = 0.5 * rng.standard_normal((H * D, dm))
    b2 = 0.1 * rng.standard_normal(dm)
    r = oracle.layer_fwd(x, w1, b1, w2, b2, offs, nt, H, D)
    # projection, by loops
    uvqk = np.zeros((T, 4 * H * D))
    for t in range(T):
        for c in range(4 * H * D):
            z = b1[c] + sum(x[t, m] * w1[m, c] for m in range(dm))
            uvqk[t, c] = z / (1.0 + math.exp(-z))
    assert np.max(np.abs(uvqk - r["uvqk"])) < 1e-12
    u, v, q, k = split_uvqk(uvqk, H, D)
    assert np.array_equal(u[:, 1, :], uvqk[:, D:2 * D])
    assert np.array_equal(k[:, 0, :], uvqk[:, 3 * H * D:3 * H * D + D])
    So, Sa = oracle.scalar_attention_fwd(q, k, v, None, offs, 4, nt)
    a = np.array(Sa).reshape(T, H * D)
    assert np.max(np.abs(a - r["a"])) < 1e-12
    y = np.zeros((T, dm))
    for t in range(T):
        mu = sum(a[t]) / (H * D)
        var = sum((e - mu) ** 2 for e in a[t]) / (H * D)
        ln = [(e - mu) / math.sqrt(var + 1e-5) for e in a[t]]
        g = [ln[c] * u.reshape(T, H * D)[t, c] for c in range(H * D)]
        for n in range(dm):
            y[t, n] = b2[n] + sum(g[c] * w2[c, n] for c in range(H * D))
    assert np.max(np.abs(y - r["y"])) < 1e-12


def test_layer_rows_match_full():
    """The sampled-rows form used by the full-size layer check agrees with the full layer."""
    rng = np.random.default_rng(2)
    H, D, dm = 2, 4, 6
    offs = np.array([0, 9, 9, 16])
    nt = np.array([3, 0, 2])
    T = 16
    x = rng.standard_normal((T, dm))
    w1 = 0.5 * rng.standard_normal((dm, 4 * H * D))
    b1 = 0.1 * rng.standard_normal(4 * H * D)
    w2 = 0.5 * rng.standard_normal((H * D, dm))
    b2 = 0.1 * rng.standard_normal(dm)
    full = oracle.layer_fwd(x, w1, b1, w2, b2, offs, nt, H, D)
    rows = np.array([0, 5, 8, 9, 15, 12])
    part = layer_fwd_rows(x, w1, b1, w2, b2, offs, nt, H, D, rows)
    for key in ("uvqk", "a", "y"):
        want = full[key][rows]
        assert np.max(np.abs(part[key] - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def test_layer_bwd_finite_differences():
    """Every gradient of the layer oracle against central differences of its
    forward (directional derivatives along random directions, plus single
    entries), so a dropped term, a transposed operand or a wrong sign in the
    chain rule fails here."""
    from oracle.layer import layer_bwd, layer_fwd
    rng = np.random.default_rng(3)
    H, D, dm = 2, 3, 5
    offs = np.array([0, 5, 9])
    nt = np.array([2, 1])
    T = 9
    x = 0.7 * rng.standard_normal((T, dm))
    w1 = 0.6 * rng.standard_normal((dm, 4 * H * D))
    b1 = 0.2 * rng.standard_normal(4 * H * D)
    w2 = 0.6 * rng.standard_normal((H * D, dm))
    b2 = 0.2 * rng.standard_normal(dm)
    dy = rng.standard_normal((T, dm))
    g = layer_bwd(x, w1, b1, w2, b2, offs, nt, H, D, dy)
    params = dict(x=x, w1=w1, b1=b1, w2=w2, b2=b2)

    def loss(**kw):
        p = dict(params, **kw)
        return float(np.sum(layer_fwd(p["x"], p["w1"], p["b1"], p["w2"], p["b2"], offs, nt, H, D)["y"] * dy))

    h = 1e-5
    for name, grad in (("x", "dx"), ("w1", "dw1"), ("b1", "db1"), ("w2", "dw2"), ("b2", "db2")):
        base = params[name]
        for trial in range(3):
            d = rng.standard_normal(base.shape)
            num = (loss(**{name: base + h * d}) - loss(**{name: base - h * d})) / (2 * h)
            ana = float(np.sum(g[grad] * d))
            assert abs(num - ana) <= 1e-6 * max(1.0, abs(num)), (name, trial, num, ana)
        idx = tuple(int(rng.integers(n)) for n in base.shape)
        e = np.zeros_like(base)
        e[idx] = 1.0
        num = (loss(**{name: base + h * e}) - loss(**{name: base - h * e})) / (2 * h)
        assert abs(num - g[grad][idx]) <= 1e-6 * max(1.0, abs(num)), (name, idx, num, g[grad][idx])


def test_layernorm_bwd_finite_differences():
    from oracle.layer import layernorm_bwd
    rng = np.random.default_rng(4)
    a = 2.0 + rng.standard_normal((3, 16))
    d_ln = rng.standard_normal((3, 16))
    got = layernorm_bwd(a, d_ln)
    h = 1e-6
    for trial in range(4):
        d = rng.standard_normal(a.shape)
        num = (np.sum(oracle.layernorm(a + h * d) * d_ln) - np.sum(oracle.layernorm(a - h * d) * d_ln)) / (2 * h)
        assert abs(num - np.sum(got * d)) <= 1e-7 * max(1.0, abs(num))
