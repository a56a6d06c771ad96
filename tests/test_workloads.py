"""Host-side checks of the seeded input generators (CPU only)."""
import numpy as np
import torch

import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]   # ties
    ours = W.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_shapes_and_determinism():
    a = W.make_attention_inputs(W.TINY)
    b = W.make_attention_inputs(W.TINY)
    assert list(a["lengths"]) == [7, 13, 32, 50]
    assert a["q"].shape == (102, 2, 32)
    assert a["rab_pos"].shape == (1, 99) and a["rab_time"].shape == (1, 64)
    for key in ("q", "k", "v", "u", "d_o", "rab_pos", "rab_time", "timestamps"):
        assert np.array_equal(a[key], b[key])
    ts = a["timestamps"]
    offs = a["seq_offsets"]
    for s in range(4):
        seg = ts[offs[s]:offs[s + 1]]
        assert seg[0] == W.T0_SECONDS and np.all(np.diff(seg) >= 0)


def test_length_distributions():
    rng = np.random.default_rng(5)
    L = W.draw_lengths(rng, "powerlaw", (64, 1024, 1.2), 200000)
    assert L.min() >= 64 and L.max() <= 1024
    assert abs(L.mean() - 307.0) < 3.0       # discrete mean of the truncated power law
    L = W.draw_lengths(rng, "uniform", (4096, 8192), 100000)
    assert L.min() == 4096 and L.max() == 8192 and abs(L.mean() - 6144) < 20


def test_bf16_workload_values_are_bf16():
    a = W.make_attention_inputs(W.PUBLIC)
    q = a["q"]
    assert np.array_equal(q, W.round_to_bf16(q))
    assert len(a["lengths"]) == 128 and a["lengths"].min() >= 20 and a["lengths"].max() <= 200
