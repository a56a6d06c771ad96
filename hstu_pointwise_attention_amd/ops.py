"""Torch-facing wrappers of the C ABI: argument marshalling only.

Tensors supply device memory, torch's current stream supplies the HIP stream;
every step of the computation runs in the HIP library.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.DTYPE_BF16, torch.float32: _lib.DTYPE_FP32}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _token_stride(t: torch.Tensor, name: str, H: int, D: int) -> int:
    if t.dim() != 3 or t.shape[1] != H or t.shape[2] != D:
        raise ValueError(f"{name} must be [T, {H}, {D}], got {tuple(t.shape)}")
    if t.numel() == 0:
        return H * D                                  # no rows: any valid stride
    if t.stride(2) != 1 or t.stride(1) != D:
        raise ValueError(f"{name} must have contiguous heads and head dim (strides {t.stride()})")
    return t.stride(0)


def make_desc(q, k, v, u, seq_offsets, max_len, n_time_buckets=0, rab_heads=1) -> _lib.AttnDesc:
    T, H, D = q.shape
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in (("k", k), ("v", v), ("u", u)):
        if t is not None and t.dtype != q.dtype:
            raise TypeError(f"{name} dtype {t.dtype} != q dtype {q.dtype}")
    d = _lib.AttnDesc()
    d.batch = seq_offsets.numel() - 1
    d.heads = H
    d.d_qk = D
    d.d_v = v.shape[2]
    d.max_len = int(max_len)
    d.n_time_buckets = int(n_time_buckets)
    d.rab_heads = int(rab_heads)
    d.dtype = _DTYPES[q.dtype]
    d.total_tokens = T
    d.stride_q = _token_stride(q, "q", H, D)
    d.stride_k = _token_stride(k, "k", H, D)
    d.stride_v = _token_stride(v, "v", H, v.shape[2])
    d.stride_u = _token_stride(u, "u", H, v.shape[2]) if u is not None else 0
    return d


def _rab_meta(rab_pos, rab_time):
    nt = rab_time.shape[1] if rab_time is not None else 0
    tab = rab_pos if rab_pos is not None else rab_time
    hr = tab.shape[0] if tab is not None else 1
    return nt, hr


def _i64(t):
    return None if t is None else t.to(torch.int64).contiguous()


def _f32c(t):
    return None if t is None else t.to(torch.float32).contiguous()


def attn_fwd(q, k, v, u, seq_offsets, max_len, *, num_targets=None, timestamps=None,
             rab_pos=None, rab_time=None, save_a: bool = True):
    """Returns (O [T,H,Dv] in q's dtype, A [T,H,Dv] fp32 or None)."""
    lib = _lib.load()
    seq_offsets, num_targets, timestamps = _i64(seq_offsets), _i64(num_targets), _i64(timestamps)
    rab_pos, rab_time = _f32c(rab_pos), _f32c(rab_time)
    nt, hr = _rab_meta(rab_pos, rab_time)
    desc = make_desc(q, k, v, u, seq_offsets, max_len, nt, hr)
    T, H, _ = q.shape
    Dv = v.shape[2]
    o = torch.empty((T, H, Dv), dtype=q.dtype, device=q.device)
    a = torch.empty((T, H, Dv), dtype=torch.float32, device=q.device) if save_a else None
    nbytes = ctypes.c_size_t()
    _lib.check(lib.hstu_attn_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(nbytes)))
    ws = torch.empty(max(nbytes.value, 1), dtype=torch.uint8, device=q.device)
    _lib.check(lib.hstu_attn_fwd(ctypes.byref(desc), _ptr(seq_offsets), _ptr(num_targets),
                                 _ptr(timestamps), _ptr(rab_pos), _ptr(rab_time), _ptr(q), _ptr(k),
                                 _ptr(v), _ptr(u), _ptr(o), _ptr(a), _ptr(ws), nbytes.value,
                                 _stream()))
    return o, a


def attn_fwd_cached(q, k, v, u, cand_offsets, cand_first, n_cands, k_hist, v_hist,
                    hist_offsets, max_len, *, ts_hist=None, ts_cand=None, rab_pos=None,
                    rab_time=None, save_a: bool = True):
    """Candidate scoring against a cached history (hstu_attn_fwd_cached).

    q, k, v, u: this call's candidate rows [M, H, D] (cand_offsets [B+1]);
    k_hist, v_hist: the history rows [Th, H, D] (hist_offsets [B+1]);
    cand_first [B], n_cands [B]: position of the call's candidates among each
    sequence's candidates. Returns (O [M,H,Dv], A [M,H,Dv] fp32 or None).
    """
    lib = _lib.load()
    cand_offsets, cand_first, n_cands = _i64(cand_offsets), _i64(cand_first), _i64(n_cands)
    hist_offsets, ts_hist, ts_cand = _i64(hist_offsets), _i64(ts_hist), _i64(ts_cand)
    rab_pos, rab_time = _f32c(rab_pos), _f32c(rab_time)
    nt, hr = _rab_meta(rab_pos, rab_time)
    desc = make_desc(q, k, v, u, cand_offsets, max_len, nt, hr)
    M, H, D = q.shape
    Dv = v.shape[2]
    for name, t in (("k_hist", k_hist), ("v_hist", v_hist)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} dtype {t.dtype} != q dtype {q.dtype}")
    skh = _token_stride(k_hist, "k_hist", H, D)
    svh = _token_stride(v_hist, "v_hist", H, Dv)
    Th = k_hist.shape[0]
    if v_hist.shape[0] != Th:
        raise ValueError("k_hist and v_hist must have the same rows")
    o = torch.empty((M, H, Dv), dtype=q.dtype, device=q.device)
    a = torch.empty((M, H, Dv), dtype=torch.float32, device=q.device) if save_a else None
    nbytes = ctypes.c_size_t()
    _lib.check(lib.hstu_attn_fwd_cached_workspace_size(ctypes.byref(desc), Th, ctypes.byref(nbytes)))
    ws = torch.empty(max(nbytes.value, 1), dtype=torch.uint8, device=q.device)
    _lib.check(lib.hstu_attn_fwd_cached(ctypes.byref(desc), _ptr(cand_offsets), _ptr(cand_first),
                                        _ptr(n_cands), _ptr(hist_offsets), Th, _ptr(ts_hist),
                                        _ptr(ts_cand), _ptr(rab_pos), _ptr(rab_time), _ptr(q),
                                        _ptr(k), _ptr(v), _ptr(u), _ptr(k_hist), _ptr(v_hist),
                                        skh, svh, _ptr(o), _ptr(a), _ptr(ws), nbytes.value,
                                        _stream()))
    return o, a


def attn_bwd(q, k, v, u, seq_offsets, max_len, a_saved, d_o, *, num_targets=None,
             timestamps=None, rab_pos=None, rab_time=None, deterministic: bool = False,
             ds_room: bool = True, report: bool = False):
    """Returns dict dq, dk, dv, du (None without gate), d_rab_pos, d_rab_time.

    deterministic: sum the rab gradients in a fixed order (desc.deterministic).
    ds_room: give the workspace the dS-export room (the preferred size) or
    only the minimum (dQ then recomputes dS). report: also return, under
    "info", what hstu_attn_bwd_report says the call did (waits for the stream).
    """
    lib = _lib.load()
    seq_offsets, num_targets, timestamps = _i64(seq_offsets), _i64(num_targets), _i64(timestamps)
    rab_pos, rab_time = _f32c(rab_pos), _f32c(rab_time)
    nt, hr = _rab_meta(rab_pos, rab_time)
    desc = make_desc(q, k, v, u, seq_offsets, max_len, nt, hr)
    desc.deterministic = 1 if deterministic else 0
    d_o = d_o.contiguous()
    T, H, D = q.shape
    Dv = v.shape[2]
    dq = torch.empty((T, H, D), dtype=q.dtype, device=q.device)
    dk = torch.empty((T, H, D), dtype=q.dtype, device=q.device)
    dv = torch.empty((T, H, Dv), dtype=q.dtype, device=q.device)
    du = torch.empty((T, H, Dv), dtype=q.dtype, device=q.device) if u is not None else None
    drp = torch.empty_like(rab_pos) if rab_pos is not None else None
    drt = torch.empty_like(rab_time) if rab_time is not None else None
    nbytes = ctypes.c_size_t()
    size_fn = lib.hstu_attn_bwd_workspace_size if ds_room else lib.hstu_attn_bwd_workspace_size_min
    _lib.check(size_fn(ctypes.byref(desc), ctypes.byref(nbytes)))
    ws = torch.empty(max(nbytes.value, 1), dtype=torch.uint8, device=q.device)
    _lib.check(lib.hstu_attn_bwd(ctypes.byref(desc), _ptr(seq_offsets), _ptr(num_targets),
                                 _ptr(timestamps), _ptr(rab_pos), _ptr(rab_time), _ptr(q), _ptr(k),
                                 _ptr(v), _ptr(u), _ptr(a_saved), _ptr(d_o), _ptr(dq), _ptr(dk),
                                 _ptr(dv), _ptr(du), _ptr(drp), _ptr(drt), _ptr(ws), nbytes.value,
                                 _stream()))
    out = dict(dq=dq, dk=dk, dv=dv, du=du, d_rab_pos=drp, d_rab_time=drt)
    if report:
        info = _lib.BwdInfo()
        _lib.check(lib.hstu_attn_bwd_report(ctypes.byref(desc), _ptr(ws), nbytes.value,
                                            ctypes.byref(info), _stream()))
        out["info"] = {"dq_from_ds": bool(info.dq_from_ds),
                       "rab_deterministic": bool(info.rab_deterministic),
                       "ds_sequences": int(info.ds_sequences)}
    return out


def rab_bucketize(seq_offsets, max_len, *, num_targets=None, timestamps=None,
                  n_time_buckets=0, want_pos=True):
    """Bucket export over the unmasked pairs: (bp uint16 or None, bt uint8 or None)."""
    lib = _lib.load()
    dev = seq_offsets.device
    seq_offsets, num_targets, timestamps = _i64(seq_offsets), _i64(num_targets), _i64(timestamps)
    d = _lib.AttnDesc()
    d.batch = seq_offsets.numel() - 1
    d.heads = 1
    d.max_len = int(max_len)
    d.n_time_buckets = int(n_time_buckets)
    po = torch.empty(d.batch + 1, dtype=torch.int64, device=dev)
    _lib.check(lib.hstu_rab_pair_offsets(ctypes.byref(d), _ptr(seq_offsets), _ptr(num_targets),
                                         _ptr(po), _stream()))
    n = int(po[-1])                       # the output size (waits for the stream)
    bp = torch.empty(max(n, 1), dtype=torch.int16, device=dev) if want_pos else None
    bt = torch.empty(max(n, 1), dtype=torch.uint8, device=dev) if timestamps is not None else None
    _lib.check(lib.hstu_rab_bucketize(ctypes.byref(d), _ptr(seq_offsets), _ptr(num_targets),
                                      _ptr(timestamps), _ptr(po), _ptr(bp), _ptr(bt), _stream()))
    bp = bp[:n].view(torch.uint16) if bp is not None else None   # a view: no conversion kernel
    bt = bt[:n] if bt is not None else None
    return bp, bt


def linear(x, w, bias=None, silu: bool = False):
    """y = act(x @ w + bias) in bf16 with fp32 accumulation."""
    lib = _lib.load()
    M, K = x.shape
    N = w.shape[1]
    if x.stride(1) != 1:
        raise ValueError("x must have a contiguous last dim")
    w = w.contiguous()
    bias = _f32c(bias)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _lib.check(lib.hstu_linear(M, K, N, _ptr(x), x.stride(0), _ptr(w), _ptr(bias), _ptr(y),
                               1 if silu else 0, _stream()))
    return y


def layernorm_gate(a, u, eps: float = 1e-5):
    """LayerNorm(a) * u over the last dim; a fp32 [M, N], u bf16 [M, N] (row-strided)."""
    lib = _lib.load()
    M, N = a.shape
    a = a.contiguous()
    if u.stride(1) != 1:
        raise ValueError("u must have a contiguous last dim")
    out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _lib.check(lib.hstu_layernorm_gate(M, N, _ptr(a), _ptr(u), u.stride(0), float(eps), _ptr(out),
                                       _stream()))
    return out


def fp8_quantize_rows(x):
    """Row-wise E4M3 codes (uint8 [M, K]) and scales (fp32 [M]) of bf16 x [M, K]."""
    lib = _lib.load()
    M, K = x.shape
    if x.stride(1) != 1:
        raise ValueError("x must have a contiguous last dim")
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _lib.check(lib.hstu_fp8_quantize_rows(M, K, _ptr(x), x.stride(0), _ptr(q), _ptr(scale), _stream()))
    return q, scale


def fp8_prepare_weight(w):
    """Codes [N, K] and per-output-feature scales [N] of a bf16 weight w [K, N]."""
    lib = _lib.load()
    K, N = w.shape
    w = w.contiguous()
    q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    scale = torch.empty((N,), dtype=torch.float32, device=w.device)
    _lib.check(lib.hstu_fp8_prepare_weight(K, N, _ptr(w), _ptr(q), _ptr(scale), _stream()))
    return q, scale


def fp8_linear(xq, x_scale, wq, w_scale, bias=None, silu: bool = False):
    """y = act(x_scale w_scale (xq wq^T) + bias), bf16 [M, N]; xq [M, K], wq [N, K] E4M3 codes."""
    lib = _lib.load()
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("wq must be [N, K]")
    xq, wq = xq.contiguous(), wq.contiguous()
    x_scale, w_scale, bias = _f32c(x_scale), _f32c(w_scale), _f32c(bias)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _lib.check(lib.hstu_fp8_linear(M, K, N, _ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale),
                                   _ptr(bias), _ptr(y), 1 if silu else 0, _stream()))
    return y


def layernorm_gate_fp8(a, u=None, eps: float = 1e-5):
    """Row-wise E4M3 codes and scales of LayerNorm(a) * u (u None: no gate); a fp32 [M, N]."""
    lib = _lib.load()
    M, N = a.shape
    a = a.contiguous()
    if u is not None and u.stride(1) != 1:
        raise ValueError("u must have a contiguous last dim")
    q = torch.empty((M, N), dtype=torch.uint8, device=a.device)
    scale = torch.empty((M,), dtype=torch.float32, device=a.device)
    _lib.check(lib.hstu_layernorm_gate_fp8(M, N, _ptr(a), _ptr(u), u.stride(0) if u is not None else 0,
                                           float(eps), _ptr(q), _ptr(scale), _stream()))
    return q, scale


def layer_bwd(x, w1, b1, w2, seq_offsets, num_targets, heads: int, head_dim: int, uvqk, a, dy,
              eps: float = 1e-5, max_len: int = 0):
    """Gradients of one HSTU layer (hstu_layer_bwd): dict dx (bf16), dw1, db1, dw2, db2 (fp32).

    x [M, d_model], w1 [d_model, 4*H*D], b1 [4*H*D], w2 [H*D, d_model] as in the
    forward; uvqk [M, 4*H*D] and a [M, H*D] the forward's outputs; dy [M, d_model];
    max_len a bound on the sequence lengths (0: none), which sizes the attention
    backward's dS export.
    """
    lib = _lib.load()
    M, dm = x.shape
    W = w1.shape[1]
    x, w1, w2, uvqk, dy = (t.contiguous() for t in (x, w1, w2, uvqk, dy))
    a = a.contiguous()
    b1 = _f32c(b1)
    seq_offsets, num_targets = _i64(seq_offsets), _i64(num_targets)
    dev = x.device
    dx = torch.empty((M, dm), dtype=torch.bfloat16, device=dev)
    dw1 = torch.empty((dm, W), dtype=torch.float32, device=dev)
    db1 = torch.empty((W,), dtype=torch.float32, device=dev)
    dw2 = torch.empty((w2.shape[0], dm), dtype=torch.float32, device=dev)
    db2 = torch.empty((dm,), dtype=torch.float32, device=dev)
    B = seq_offsets.numel() - 1
    nbytes = ctypes.c_size_t()
    _lib.check(lib.hstu_layer_bwd_workspace_size(M, B, dm, heads, head_dim, int(max_len),
                                                 ctypes.byref(nbytes)))
    ws = torch.empty(max(nbytes.value, 1), dtype=torch.uint8, device=dev)
    _lib.check(lib.hstu_layer_bwd(M, B, dm, heads, head_dim, int(max_len), _ptr(seq_offsets),
                                  _ptr(num_targets),
                                  _ptr(x), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(uvqk), _ptr(a),
                                  float(eps), _ptr(dy), _ptr(dx), _ptr(dw1), _ptr(db1), _ptr(dw2),
                                  _ptr(db2), _ptr(ws), nbytes.value, _stream()))
    return dict(dx=dx, dw1=dw1, db1=db1, dw2=dw2, db2=db2)
