"""The layer's GEMM (hstu_linear, through the C ABI) on small ragged shapes
(needs a gfx950 GPU).

The expected value is the definition y = act(x w + b) in float64 on the
bf16-rounded operands (act = SiLU, z * sigmoid(z), or identity), the
projection step of oracle.layer; tolerance: rel-L2 <= 1e-2 and max-abs
within bf16 output rounding.
"""
import numpy as np
import pytest

from oracle.attention import silu
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


@pytest.mark.parametrize("M,K,N,ldx,act,bias", [
    (1, 32, 128, 32, False, False),        # one row, one stage shorter than the stage depth
    (77, 96, 384, 96, True, True),         # ragged rows, reduction not a multiple of 64
    (300, 512, 256, 520, True, True),      # strided x, several row tiles with a tail
    (1024, 160, 128, 160, False, True),    # row tiles a multiple of 8 (XCD grouping on)
])
def test_linear(M, K, N, ldx, act, bias):
    import torch
    from hstu_pointwise_attention_amd import ops
    rng = np.random.default_rng(M * 7 + K)
    xs = round_to(rng.standard_normal((M, ldx)), "bf16")
    w = round_to(rng.standard_normal((K, N)) / np.sqrt(K), "bf16")
    b = (0.3 * rng.standard_normal(N)).astype(np.float32) if bias else None
    dev = "cuda"
    tx = torch.from_numpy(xs).to(dev, torch.bfloat16)[:, :K]
    tw = torch.from_numpy(w).to(dev, torch.bfloat16)
    tb = torch.from_numpy(b).to(dev) if bias else None
    y = P.host(ops.linear(tx, tw, tb, silu=act))
    torch.cuda.synchronize()
    z = xs[:, :K].astype(np.float64) @ w.astype(np.float64)
    if bias:
        z = z + b.astype(np.float64)
    want = silu(z) if act else z
    assert P.rel_l2(y, want) <= P.BF16_REL
    assert float(np.max(np.abs(y - want))) <= 1e-2 * max(1.0, float(np.max(np.abs(want))))
