"""The C ABI library loads, exports what the header declares, and rejects bad
arguments before launching anything (so these tests need no GPU)."""
import ctypes
import os
import re

import pytest

from hstu_pointwise_attention_amd import _lib
from hstu_pointwise_attention_amd.flops import unmasked_pairs_host, attention_flops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hstu_attn.h")

if not os.path.exists(_lib.LIB_PATH):
    pytest.skip("libhstu_attn.so not built", allow_module_level=True)

FAKE = ctypes.c_void_p(4096)   # never dereferenced: every case fails validation first


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def header_symbols():
    text = open(HEADER).read()
    return set(re.findall(r"HSTU_API\s+[\w\s\*]+?\b(hstu_\w+)\s*\(", text))


def test_exports_every_declared_symbol(lib):
    declared = header_symbols()
    assert declared == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def good_desc(**kw):
    d = _lib.AttnDesc()
    d.batch, d.heads, d.d_qk, d.d_v, d.max_len = 2, 2, 64, 64, 100
    d.n_time_buckets, d.rab_heads, d.dtype, d.total_tokens = 16, 1, _lib.DTYPE_BF16, 50
    d.stride_q = d.stride_k = d.stride_v = d.stride_u = 128
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def fwd_call(lib, d, ws_bytes=1 << 30, rab_time=FAKE, timestamps=FAKE, ws=ctypes.c_void_p(1 << 20)):
    return lib.hstu_attn_fwd(ctypes.byref(d), FAKE, None, timestamps, None, rab_time, FAKE, FAKE,
                             FAKE, FAKE, FAKE, None, ws, ws_bytes, None)


@pytest.mark.parametrize("field,value,status", [
    ("batch", -1, _lib.HSTU_EINVAL),
    ("heads", 0, _lib.HSTU_EINVAL),
    ("d_qk", 48, _lib.HSTU_EUNSUPPORTED),
    ("d_v", 32, _lib.HSTU_EUNSUPPORTED),
    ("dtype", 7, _lib.HSTU_EINVAL),
    ("max_len", 0, _lib.HSTU_EINVAL),
    ("n_time_buckets", 2000, _lib.HSTU_EINVAL),
    ("rab_heads", 3, _lib.HSTU_EINVAL),
    ("total_tokens", -5, _lib.HSTU_EINVAL),
    ("total_tokens", 1 << 31, _lib.HSTU_EINVAL),
    ("stride_q", 64, _lib.HSTU_EINVAL),
    ("stride_k", 130, _lib.HSTU_EINVAL),
    ("stride_v", (1 << 22) + 8, _lib.HSTU_EUNSUPPORTED),   # beyond the 32-bit tile range
    ("deterministic", 2, _lib.HSTU_EINVAL),
])
def test_desc_validation(lib, field, value, status):
    d = good_desc(**{field: value})
    assert fwd_call(lib, d) == status
    assert lib.hstu_last_error().decode()


def test_missing_inputs(lib):
    d = good_desc()
    assert fwd_call(lib, d, timestamps=None) == _lib.HSTU_EINVAL          # time bias without ts
    d0 = good_desc(n_time_buckets=0)
    assert fwd_call(lib, d0) == _lib.HSTU_EINVAL                           # table without buckets
    assert lib.hstu_attn_fwd(ctypes.byref(d), None, None, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                             FAKE, FAKE, None, FAKE, 1 << 30, None) == _lib.HSTU_EINVAL
    assert lib.hstu_attn_fwd(ctypes.byref(d), FAKE, None, FAKE, None, FAKE, None, FAKE, FAKE,
                             FAKE, FAKE, None, FAKE, 1 << 30, None) == _lib.HSTU_EINVAL
    assert lib.hstu_attn_fwd(None, FAKE, None, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             None, FAKE, 1 << 30, None) == _lib.HSTU_EINVAL


def test_workspace_checks(lib):
    d = good_desc()
    need = ctypes.c_size_t()
    assert lib.hstu_attn_fwd_workspace_size(ctypes.byref(d), ctypes.byref(need)) == 0
    assert need.value > 0
    assert fwd_call(lib, d, ws_bytes=need.value - 1) == _lib.HSTU_EWORKSPACE
    assert fwd_call(lib, d, ws=None) == _lib.HSTU_EWORKSPACE
    assert fwd_call(lib, d, ws=ctypes.c_void_p((1 << 20) + 8)) == _lib.HSTU_EWORKSPACE  # misaligned
    bneed = ctypes.c_size_t()
    assert lib.hstu_attn_bwd_workspace_size(ctypes.byref(d), ctypes.byref(bneed)) == 0
    assert bneed.value >= need.value + 50 * 128 * 2        # holds dA' = dO*U/L (bf16 [T, H, D])
    assert lib.hstu_attn_fwd_workspace_size(ctypes.byref(d), None) == _lib.HSTU_EINVAL


def _bwd_sizes(lib, d):
    pref, least = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.hstu_attn_bwd_workspace_size(ctypes.byref(d), ctypes.byref(pref)) == 0
    assert lib.hstu_attn_bwd_workspace_size_min(ctypes.byref(d), ctypes.byref(least)) == 0
    return pref.value, least.value


def test_bwd_workspace_min_and_preferred(lib):
    # bf16: the preferred size adds the dS-tile room (at least one 16 KB tile)
    pref, least = _bwd_sizes(lib, good_desc())
    assert pref >= least + 16384
    # fp32 recomputes dS for dQ: both figures agree
    d32 = good_desc(dtype=_lib.DTYPE_FP32, stride_q=128, stride_k=128, stride_v=128, stride_u=128)
    pref32, least32 = _bwd_sizes(lib, d32)
    assert pref32 == least32
    # the deterministic mode adds its partials to both figures
    pref_d, least_d = _bwd_sizes(lib, good_desc(deterministic=1))
    # (the per-sequence tile numbering is carved once for both)
    assert least_d > least and 16384 <= pref_d - least_d <= pref - least
    # below the minimum: rejected before any launch
    st = lib.hstu_attn_bwd(ctypes.byref(good_desc()), FAKE, None, FAKE, None, FAKE, FAKE, FAKE,
                           FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                           ctypes.c_void_p(1 << 20), least - 1, None)
    assert st == _lib.HSTU_EWORKSPACE


def test_bwd_report_validation(lib):
    d = good_desc()
    pref, least = _bwd_sizes(lib, d)
    info = _lib.BwdInfo()
    assert lib.hstu_attn_bwd_report(ctypes.byref(d), ctypes.c_void_p(1 << 20), pref, None,
                                    None) == _lib.HSTU_EINVAL
    assert lib.hstu_attn_bwd_report(ctypes.byref(d), ctypes.c_void_p(1 << 20), least - 1,
                                    ctypes.byref(info), None) == _lib.HSTU_EWORKSPACE
    assert lib.hstu_attn_bwd_report(ctypes.byref(good_desc(heads=0)), ctypes.c_void_p(1 << 20),
                                    pref, ctypes.byref(info), None) == _lib.HSTU_EINVAL
    # an empty batch ran nothing: no device read, nothing summed
    d0 = good_desc(batch=0, total_tokens=0, deterministic=1)
    pref0, _ = _bwd_sizes(lib, d0)
    assert lib.hstu_attn_bwd_report(ctypes.byref(d0), ctypes.c_void_p(1 << 20), pref0,
                                    ctypes.byref(info), None) == 0
    assert info.dq_from_ds == 0 and info.rab_deterministic == 1


def test_bwd_requires_gradients(lib):
    d = good_desc()
    # rab_pos given without d_rab_pos
    st = lib.hstu_attn_bwd(ctypes.byref(d), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                           FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None)
    assert st == _lib.HSTU_EINVAL
    # gated without du
    st = lib.hstu_attn_bwd(ctypes.byref(d), FAKE, None, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                           FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 1 << 30, None)
    assert st == _lib.HSTU_EINVAL


def cached_call(lib, d, hist_tokens=20, ts_hist=FAKE, ts_cand=FAKE, rab_time=FAKE, k_hist=FAKE,
                stride_kh=128, hist_offsets=FAKE, ws_bytes=1 << 30, ws=ctypes.c_void_p(1 << 20)):
    return lib.hstu_attn_fwd_cached(ctypes.byref(d), FAKE, FAKE, FAKE, hist_offsets, hist_tokens,
                                    ts_hist, ts_cand, None, rab_time, FAKE, FAKE, FAKE, FAKE,
                                    k_hist, FAKE, stride_kh, 128, FAKE, None, ws, ws_bytes, None)


def test_cached_validation(lib):
    d = good_desc()
    need = ctypes.c_size_t()
    assert lib.hstu_attn_fwd_cached_workspace_size(ctypes.byref(d), 20, ctypes.byref(need)) == 0
    fneed = ctypes.c_size_t()
    assert lib.hstu_attn_fwd_workspace_size(ctypes.byref(d), ctypes.byref(fneed)) == 0
    assert need.value > fneed.value                       # joined rows + per-sequence records
    assert lib.hstu_attn_fwd_cached_workspace_size(ctypes.byref(d), -1, ctypes.byref(need)) \
        == _lib.HSTU_EINVAL
    assert lib.hstu_attn_fwd_cached_workspace_size(ctypes.byref(d), 1 << 31, ctypes.byref(need)) \
        == _lib.HSTU_EINVAL                               # joined rows beyond 2^31
    assert cached_call(lib, d, ts_hist=None) == _lib.HSTU_EINVAL        # time bias, no history ts
    assert cached_call(lib, d, ts_cand=None) == _lib.HSTU_EINVAL        # time bias, no candidate ts
    assert cached_call(lib, d, k_hist=None) == _lib.HSTU_EINVAL         # history rows, no keys
    assert cached_call(lib, d, stride_kh=64) == _lib.HSTU_EINVAL        # stride below heads*d
    assert cached_call(lib, d, stride_kh=130) == _lib.HSTU_EINVAL       # not 16-byte rows
    assert cached_call(lib, d, hist_offsets=None) == _lib.HSTU_EINVAL
    assert cached_call(lib, d, ws_bytes=16) == _lib.HSTU_EWORKSPACE
    assert cached_call(lib, good_desc(d_qk=48, d_v=48)) == _lib.HSTU_EUNSUPPORTED
    # no candidate rows: nothing to compute, no tensors needed
    assert cached_call(lib, good_desc(total_tokens=0), ts_hist=None, ts_cand=None,
                       k_hist=None) == _lib.HSTU_OK


def test_layer_validation(lib):
    assert lib.hstu_linear(10, 48, 128, FAKE, 48, FAKE, None, FAKE, 1, None) == _lib.HSTU_EUNSUPPORTED
    assert lib.hstu_linear(10, 64, 100, FAKE, 64, FAKE, None, FAKE, 1, None) == _lib.HSTU_EUNSUPPORTED
    assert lib.hstu_linear(10, 64, 128, FAKE, 32, FAKE, None, FAKE, 1, None) == _lib.HSTU_EINVAL
    assert lib.hstu_linear(-1, 64, 128, FAKE, 64, FAKE, None, FAKE, 1, None) == _lib.HSTU_EINVAL
    assert lib.hstu_layernorm_gate(4, 100, FAKE, FAKE, 100, 1e-5, FAKE, None) == _lib.HSTU_EINVAL
    assert lib.hstu_layernorm_gate(4, 512, FAKE, FAKE, 500, 1e-5, FAKE, None) == _lib.HSTU_EINVAL
    assert lib.hstu_layernorm_gate(4, 512, FAKE, FAKE, 512, -1.0, FAKE, None) == _lib.HSTU_EINVAL


def layer_bwd_call(lib, M=64, d_model=128, heads=2, head_dim=64, max_len=0, ws_bytes=1 << 30, **kw):
    a = dict(seq_offsets=FAKE, x=FAKE, w1=FAKE, b1=FAKE, w2=FAKE, uvqk=FAKE, a=FAKE, dy=FAKE,
             dx=FAKE, dw1=FAKE, db1=FAKE, dw2=FAKE, db2=FAKE, ws=ctypes.c_void_p(1 << 20),
             eps=1e-5)
    a.update(kw)
    return lib.hstu_layer_bwd(M, 1, d_model, heads, head_dim, max_len, a["seq_offsets"], None, a["x"],
                              a["w1"], a["b1"], a["w2"], a["uvqk"], a["a"], a["eps"], a["dy"],
                              a["dx"], a["dw1"], a["db1"], a["dw2"], a["db2"], a["ws"], ws_bytes,
                              None)


def test_layer_bwd_validation(lib):
    size = ctypes.c_size_t(0)
    assert lib.hstu_layer_bwd_workspace_size(64, 1, 128, 2, 64, 0, ctypes.byref(size)) == _lib.HSTU_OK
    assert size.value > 0
    assert lib.hstu_layer_bwd_workspace_size(64, 1, 128, 2, 48, 0, ctypes.byref(size)) \
        == _lib.HSTU_EUNSUPPORTED
    assert lib.hstu_layer_bwd_workspace_size(64, 1, 100, 2, 64, 0, ctypes.byref(size)) \
        == _lib.HSTU_EUNSUPPORTED
    assert lib.hstu_layer_bwd_workspace_size(-1, 1, 128, 2, 64, 0, ctypes.byref(size)) \
        == _lib.HSTU_EINVAL
    big = ctypes.c_size_t(0)
    assert lib.hstu_layer_bwd_workspace_size(64, 1, 128, 2, 64, 4096, ctypes.byref(big)) == _lib.HSTU_OK
    assert big.value > size.value                          # room for the exported dS tiles
    assert lib.hstu_layer_bwd_workspace_size(64, 1, 128, 2, 64, -1, ctypes.byref(big)) \
        == _lib.HSTU_EINVAL
    assert layer_bwd_call(lib, max_len=-5) == _lib.HSTU_EINVAL
    assert layer_bwd_call(lib, head_dim=48) == _lib.HSTU_EUNSUPPORTED
    assert layer_bwd_call(lib, heads=1, head_dim=64) == _lib.HSTU_EUNSUPPORTED  # H*D = 64
    assert layer_bwd_call(lib, eps=-1.0) == _lib.HSTU_EINVAL
    assert layer_bwd_call(lib, dw1=None) == _lib.HSTU_EINVAL
    assert layer_bwd_call(lib, dy=None) == _lib.HSTU_EINVAL
    assert layer_bwd_call(lib, seq_offsets=None) == _lib.HSTU_EINVAL
    assert layer_bwd_call(lib, x=ctypes.c_void_p(4098)) == _lib.HSTU_EINVAL   # misaligned
    assert layer_bwd_call(lib, ws_bytes=16) == _lib.HSTU_EWORKSPACE
    assert layer_bwd_call(lib, ws=None) == _lib.HSTU_EWORKSPACE


def test_fp8_validation(lib):
    S = FAKE
    assert lib.hstu_fp8_quantize_rows(10, 24, S, 24, S, S, None) == _lib.HSTU_EUNSUPPORTED
    assert lib.hstu_fp8_quantize_rows(10, 32, S, 16, S, S, None) == _lib.HSTU_EINVAL      # ldx < K
    assert lib.hstu_fp8_quantize_rows(-1, 32, S, 32, S, S, None) == _lib.HSTU_EINVAL
    assert lib.hstu_fp8_quantize_rows(10, 32, ctypes.c_void_p(4104), 32, S, S, None) == _lib.HSTU_EINVAL
    assert lib.hstu_fp8_quantize_rows(10, 32, S, 32, S, None, None) == _lib.HSTU_EINVAL
    assert lib.hstu_fp8_prepare_weight(0, 16, S, S, S, None) == _lib.HSTU_EINVAL
    assert lib.hstu_fp8_prepare_weight(40, 16, S, S, S, None) == _lib.HSTU_EUNSUPPORTED
    assert lib.hstu_fp8_linear(10, 24, 16, S, S, S, S, None, S, 0, None) == _lib.HSTU_EUNSUPPORTED
    assert lib.hstu_fp8_linear(10, 32, 16, S, None, S, S, None, S, 0, None) == _lib.HSTU_EINVAL
    assert lib.hstu_fp8_linear(10, 32, 16, ctypes.c_void_p(4100), S, S, S, None, S, 0, None) \
        == _lib.HSTU_EINVAL
    assert lib.hstu_layernorm_gate_fp8(4, 100, S, None, 0, 1e-5, S, S, None) == _lib.HSTU_EINVAL
    assert lib.hstu_layernorm_gate_fp8(4, 128, S, S, 64, 1e-5, S, S, None) == _lib.HSTU_EINVAL
    assert lib.hstu_layernorm_gate_fp8(4, 128, S, None, 0, -1.0, S, S, None) == _lib.HSTU_EINVAL
    # nothing to do: no rows
    assert lib.hstu_fp8_linear(0, 32, 16, None, None, None, None, None, None, 0, None) == _lib.HSTU_OK


def test_bucketize_validation(lib):
    d = good_desc(max_len=40000)
    assert lib.hstu_rab_bucketize(ctypes.byref(d), FAKE, None, FAKE, FAKE, FAKE, FAKE, None) \
        == _lib.HSTU_EINVAL
    d = good_desc(n_time_buckets=300)
    assert lib.hstu_rab_bucketize(ctypes.byref(d), FAKE, None, FAKE, FAKE, None, FAKE, None) \
        == _lib.HSTU_EINVAL


def test_pair_offsets_validation(lib):
    d = good_desc(batch=-1)
    assert lib.hstu_rab_pair_offsets(ctypes.byref(d), FAKE, None, FAKE, None) == _lib.HSTU_EINVAL
    d = good_desc()
    assert lib.hstu_rab_pair_offsets(ctypes.byref(d), None, None, FAKE, None) == _lib.HSTU_EINVAL
    assert lib.hstu_rab_pair_offsets(ctypes.byref(d), FAKE, None, None, None) == _lib.HSTU_EINVAL
    assert lib.hstu_rab_pair_offsets(None, FAKE, None, FAKE, None) == _lib.HSTU_EINVAL


def test_host_pair_accounting_matches_oracle():
    import numpy as np
    from oracle.attention import unmasked_pairs
    rng = np.random.default_rng(0)
    for _ in range(20):
        L = rng.integers(0, 50, size=6)
        nt = np.minimum(rng.integers(0, 10, size=6), L)
        offs = np.concatenate([[0], np.cumsum(L)])
        assert unmasked_pairs_host(L, nt) == unmasked_pairs(offs, nt)
    f = attention_flops([3, 4], heads=2, d_qk=32, d_v=32)
    assert f["pair_heads"] == 2 * (6 + 10) and f["total"] == f["pair_heads"] * 14 * 32
