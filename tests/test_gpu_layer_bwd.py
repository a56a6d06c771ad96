"""Parity of the HSTU layer backward (hstu_layer_bwd, through the C ABI) with
oracle.layer.layer_bwd, the chain rule pinned by finite differences in
tests/test_oracle_layer.py (needs a gfx950 GPU).

The HIP path stores its intermediates (Pre, Z, dZ, dA, dU, dQ, dK, dV, dPre)
in bf16, as the forward stores UVQK, so the bar is the bf16 one: rel-L2 <= 1e-2
for every gradient.
"""
import numpy as np
import pytest

from oracle.layer import layer_bwd as oracle_layer_bwd
from tests import parity as P
from workloads import round_to

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hstu_pointwise_attention_amd import _lib
    _lib.load()


def _case(lengths, n_targets, d_model, heads, head_dim, seed):
    import torch
    from hstu_pointwise_attention_amd.attention import hstu_layer_bwd, hstu_layer_fwd
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, np.int64)
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    nt = np.asarray(n_targets, np.int64)
    M = int(offs[-1])
    HD = heads * head_dim
    x = round_to(rng.standard_normal((M, d_model)), "bf16")
    w1 = round_to(rng.standard_normal((d_model, 4 * HD)) / np.sqrt(d_model), "bf16")
    b1 = (0.1 * rng.standard_normal(4 * HD)).astype(np.float32)
    w2 = round_to(rng.standard_normal((HD, d_model)) / np.sqrt(HD), "bf16")
    b2 = (0.1 * rng.standard_normal(d_model)).astype(np.float32)
    dy = round_to(rng.standard_normal((M, d_model)), "bf16")
    dev = "cuda"
    bf = lambda t: torch.from_numpy(np.ascontiguousarray(t)).to(dev, torch.bfloat16)
    f32 = lambda t: torch.from_numpy(np.ascontiguousarray(t)).to(dev, torch.float32)
    i64 = lambda t: torch.from_numpy(t).to(dev)
    tx, tw1, tw2, tdy = bf(x), bf(w1), bf(w2), bf(dy)
    tb1, tb2 = f32(b1), f32(b2)
    y, a, uvqk = hstu_layer_fwd(tx, tw1, tb1, tw2, tb2, i64(offs), i64(nt), heads, head_dim)
    want = oracle_layer_bwd(x, w1, b1, w2, b2, offs, nt, heads, head_dim, dy)
    # max_len 0: the attention backward recomputes dS for dQ; the longest
    # length: it exports dS tiles instead
    for max_len in (0, int(lengths.max()) if len(lengths) else 0):
        g = hstu_layer_bwd(tx, tw1, tb1, tw2, i64(offs), i64(nt), heads, head_dim, uvqk, a, tdy,
                           max_len=max_len)
        torch.cuda.synchronize()
        tag = (f"lengths {list(lengths)} targets {list(nt)} d_model {d_model} H{heads} D{head_dim}"
               f" max_len {max_len}")
        print(tag, flush=True)
        for key in ("dx", "dw1", "db1", "dw2", "db2"):
            e = P.rel_l2(P.host(g[key]), want[key])
            assert e <= P.BF16_REL, (tag, key, e)


def test_layer_bwd_small():
    """Token count not a multiple of 32 (padded rows of the weight GEMMs), candidates."""
    _case([96 + 32, 70 + 10, 5], [32, 10, 2], d_model=128, heads=2, head_dim=64, seed=1)


def test_layer_bwd_head_dims():
    _case([40, 65], [8, 0], d_model=256, heads=4, head_dim=32, seed=2)
    _case([130, 33], [30, 3], d_model=128, heads=1, head_dim=128, seed=3)


def test_layer_bwd_medium():
    """Two users with 1000 history rows and 200 candidates, d_model 256, H 2, D 128."""
    _case([1200, 1200], [200, 200], d_model=256, heads=2, head_dim=128, seed=4)


def test_layer_bwd_no_tokens():
    import torch
    from hstu_pointwise_attention_amd import ops
    dev = "cuda"
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device=dev)
    w1 = torch.ones((128, 512), dtype=torch.bfloat16, device=dev)
    w2 = torch.ones((128, 128), dtype=torch.bfloat16, device=dev)
    offs = torch.zeros(2, dtype=torch.int64, device=dev)
    g = ops.layer_bwd(x, w1, torch.zeros(512, device=dev), w2, offs, None, 2, 64,
                      torch.zeros((0, 512), dtype=torch.bfloat16, device=dev),
                      torch.zeros((0, 128), dtype=torch.float32, device=dev),
                      torch.zeros((0, 128), dtype=torch.bfloat16, device=dev))
    torch.cuda.synchronize()
    for key in ("dw1", "db1", "dw2", "db2"):
        assert float(g[key].abs().max()) == 0.0, key
