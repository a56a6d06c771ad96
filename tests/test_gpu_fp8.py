"""FP8 (E4M3FN) projection path through the C ABI against oracle.fp8 (needs a
gfx950 GPU).

Codes are integers decided in fp32 on both sides (the scale amax / 448 and the
quotient x / scale are IEEE fp32 divisions), so row quantisation and weight
preparation must match the oracle byte for byte, scales bit for bit. The FP8
GEMM then runs on identical codes: what remains is fp32 summation order and
the bf16 output rounding (rel-L2 <= 1e-2, max-abs <= 2^-7 of the largest
output). LayerNorm-and-gate forms z in fp32 in its own order, so a code may
differ where z sits within an ulp of a rounding boundary: at most 0.1% of the
codes may differ, each by one step.
"""
import numpy as np
import pytest

from oracle import fp8 as F
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


def _bf16_rows(rng, M, K):
    """bf16 values with per-row magnitudes over 2^-20 .. 2^6, a zero row, and
    entries far below their row's amax (subnormal codes)."""
    x = rng.standard_normal((M, K)) * np.exp2(rng.integers(-20, 7, size=(M, 1)))
    if M > 3:
        x[2] = 0.0
        x[3, : K // 2] *= 2.0 ** -9
    return round_to(x, "bf16")


def _dev(a, dt):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dt)


@pytest.mark.parametrize("M,K,ldx", [(1, 16, 16), (77, 96, 104), (300, 512, 512), (1030, 2048, 2048)])
def test_quantize_rows_bit_exact(M, K, ldx):
    import torch
    from hstu_pointwise_attention_amd import ops
    rng = np.random.default_rng(M + K)
    xs = _bf16_rows(rng, M, ldx)
    q, s = ops.fp8_quantize_rows(_dev(xs, torch.bfloat16)[:, :K])
    wq, ws = F.quantize_rows(xs[:, :K])
    q, s = P.host(q).astype(np.uint8), P.host(s).astype(np.float32)
    assert np.array_equal(s.view(np.uint32), ws.view(np.uint32)), "scales"
    bad = np.argwhere(q != wq)
    assert bad.size == 0, (bad[:5], q[tuple(bad[0])], wq[tuple(bad[0])])


@pytest.mark.parametrize("K,N", [(16, 1), (64, 130), (512, 2048)])
def test_prepare_weight_bit_exact(K, N):
    import torch
    from hstu_pointwise_attention_amd import ops
    rng = np.random.default_rng(K * 3 + N)
    w = round_to(rng.standard_normal((K, N)) / np.sqrt(K), "bf16")
    q, s = ops.fp8_prepare_weight(_dev(w, torch.bfloat16))
    wq, ws = F.quantize_weight(w)
    assert np.array_equal(P.host(s).astype(np.float32).view(np.uint32), ws.view(np.uint32))
    assert np.array_equal(P.host(q).astype(np.uint8), wq)


@pytest.mark.parametrize("M,K,N,act,bias", [
    (1, 16, 1, False, False),
    (77, 96, 200, True, True),          # ragged rows and columns, K shorter than a stage
    (300, 512, 512, False, True),
    (4096, 512, 512, False, True),      # the pages' FP8 addmm benchmark shape
    (1024, 2048, 384, True, True),      # several stages, XCD-grouped tile order
])
def test_fp8_linear(M, K, N, act, bias):
    import torch
    from hstu_pointwise_attention_amd import ops
    rng = np.random.default_rng(M + 5 * K + N)
    x = round_to(rng.standard_normal((M, K)), "bf16")
    w = round_to(rng.standard_normal((K, N)) / np.sqrt(K), "bf16")
    b = (0.2 * rng.standard_normal(N)).astype(np.float32) if bias else None
    xq, xs = ops.fp8_quantize_rows(_dev(x, torch.bfloat16))
    wq, ws = ops.fp8_prepare_weight(_dev(w, torch.bfloat16))
    y = ops.fp8_linear(xq, xs, wq, ws, _dev(b, torch.float32) if bias else None, silu=act)
    y = P.host(y)
    oxq, oxs = F.quantize_rows(x)
    owq, ows = F.quantize_weight(w)
    assert np.array_equal(P.host(xq).astype(np.uint8), oxq) and np.array_equal(P.host(wq).astype(np.uint8), owq)
    want = F.fp8_linear(oxq, oxs, owq, ows, b, apply_silu=act)
    assert P.rel_l2(y, want) <= P.BF16_REL
    assert float(np.max(np.abs(y - want))) <= 2.0 ** -7 * max(float(np.max(np.abs(want))), 1e-30)


def test_fp8_linear_no_rows():
    import torch
    from hstu_pointwise_attention_amd import ops
    xq = torch.zeros((0, 64), dtype=torch.uint8, device="cuda")
    wq = torch.zeros((128, 64), dtype=torch.uint8, device="cuda")
    y = ops.fp8_linear(xq, torch.zeros(0, device="cuda"), wq, torch.ones(128, device="cuda"))
    torch.cuda.synchronize()
    assert y.shape == (0, 128)


@pytest.mark.parametrize("gated", [True, False])
@pytest.mark.parametrize("M,N", [(5, 64), (333, 512), (2048, 1024)])
def test_layernorm_gate_fp8(M, N, gated):
    import torch
    from hstu_pointwise_attention_amd import ops
    rng = np.random.default_rng(M + N + gated)
    a = (rng.standard_normal((M, N)) * 2 + 0.5).astype(np.float32)
    u = round_to(rng.standard_normal((M, N + 8)), "bf16")
    tu = _dev(u, torch.bfloat16)[:, :N] if gated else None
    q, s = ops.layernorm_gate_fp8(_dev(a, torch.float32), tu)
    q, s = P.host(q).astype(np.uint8), P.host(s).astype(np.float32)
    wq, ws = F.layernorm_gate_fp8(a, u[:, :N] if gated else np.ones((M, N)))
    assert np.allclose(s, ws, rtol=1e-5, atol=0)
    diff = q != wq
    assert diff.mean() <= 1e-3, diff.mean()
    # a differing code is the neighbouring one: same sign, magnitude one step away
    same_sign = (q[diff] & 0x80) == (wq[diff] & 0x80)
    step = np.abs((q[diff] & 0x7F).astype(int) - (wq[diff] & 0x7F).astype(int))
    assert np.all(same_sign & (step == 1)) or not diff.any()


def _layer_case(lengths, n_targets, d_model, heads, head_dim, seed):
    """FP8 layer forward on the GPU, checked step by step on its own
    intermediates (the UVQK GEMM on identical codes, LayerNorm-gate-to-FP8 on
    the GPU's own A and U, the output GEMM on the GPU's own codes), then end to
    end against oracle.fp8.layer_fwd_fp8 with one E4M3 rounding unit (2^-4) of
    rel-L2: the GPU keeps UVQK in bf16, so requantising LayerNorm(A) * U may move
    a code by one step where the fp64 oracle's z differs at bf16 precision."""
    import torch
    from hstu_pointwise_attention_amd import ops
    from hstu_pointwise_attention_amd.attention import hstu_layer_fwd_fp8, prepare_fp8_weights
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, np.int64)
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    nt = np.asarray(n_targets, np.int64)
    M, HD = int(offs[-1]), heads * head_dim
    x = round_to(rng.standard_normal((M, d_model)), "bf16")
    w1 = round_to(rng.standard_normal((d_model, 4 * HD)) / np.sqrt(d_model), "bf16")
    b1 = (0.1 * rng.standard_normal(4 * HD)).astype(np.float32)
    w2 = round_to(rng.standard_normal((HD, d_model)) / np.sqrt(HD), "bf16")
    b2 = (0.1 * rng.standard_normal(d_model)).astype(np.float32)
    fw = prepare_fp8_weights(_dev(w1, torch.bfloat16), _dev(w2, torch.bfloat16))
    y, a, uvqk = hstu_layer_fwd_fp8(_dev(x, torch.bfloat16), fw, _dev(b1, torch.float32),
                                    _dev(b2, torch.float32), _dev(offs, torch.int64),
                                    _dev(nt, torch.int64), heads, head_dim)
    zq, zs = ops.layernorm_gate_fp8(a, uvqk[:, :HD])
    torch.cuda.synchronize()
    tag = f"fp8 layer lengths {list(lengths)} d_model {d_model} H{heads} D{head_dim}"
    print(tag, flush=True)
    y, a, uvqk, zq, zs = (P.host(t) for t in (y, a, uvqk, zq, zs))
    xq, xs = F.quantize_rows(x)
    w1q, w1s = F.quantize_weight(w1)
    w2q, w2s = F.quantize_weight(w2)
    assert P.rel_l2(uvqk, F.fp8_linear(xq, xs, w1q, w1s, b1, apply_silu=True)) <= P.BF16_REL, tag
    oq, os_ = F.layernorm_gate_fp8(a, uvqk[:, :HD])
    assert np.allclose(zs, os_, rtol=1e-5, atol=0) and (zq.astype(np.uint8) != oq).mean() <= 1e-3, tag
    assert P.rel_l2(y, F.fp8_addmm(zq.astype(np.uint8), zs, w2q, w2s, b2)) <= P.BF16_REL, tag
    want = F.layer_fwd_fp8(x, w1, b1, w2, b2, offs, nt, heads, head_dim)
    assert P.rel_l2(y, want["y"]) <= 2.0 ** -4, (tag, P.rel_l2(y, want["y"]))


def test_layer_fwd_fp8_small():
    _layer_case([128 + 32, 80 + 10, 5], [32, 10, 2], d_model=128, heads=2, head_dim=64, seed=21)


def test_layer_fwd_fp8_medium():
    _layer_case([1200, 1200], [200, 200], d_model=256, heads=2, head_dim=128, seed=22)
