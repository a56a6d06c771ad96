"""ctypes loader for ``libhstu_attn.so`` (the C ABI in ``include/hstu_attn.h``).

The library is loaded after torch so that it binds to the HIP runtime torch
already loaded (both use the soname ``libamdhip64.so.7``). There is no other
implementation behind these names: if the library is missing, loading fails.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhstu_attn.so")

HSTU_OK = 0
HSTU_EINVAL = -1
HSTU_EUNSUPPORTED = -2
HSTU_EWORKSPACE = -3
HSTU_EHIP = -4
DTYPE_BF16 = 0
DTYPE_FP32 = 1

STATUS_NAMES = {0: "HSTU_OK", -1: "HSTU_EINVAL", -2: "HSTU_EUNSUPPORTED",
                -3: "HSTU_EWORKSPACE", -4: "HSTU_EHIP"}

# Every symbol the header declares.
EXPORTS = ("hstu_attn_fwd_workspace_size", "hstu_attn_bwd_workspace_size",
           "hstu_attn_bwd_workspace_size_min", "hstu_attn_bwd_report", "hstu_attn_fwd",
           "hstu_attn_fwd_noalloc",
           "hstu_attn_fwd_cached_workspace_size", "hstu_attn_fwd_cached",
           "hstu_attn_bwd", "hstu_rab_pair_offsets", "hstu_rab_bucketize", "hstu_linear", "hstu_layernorm_gate",
           "hstu_layer_bwd_workspace_size", "hstu_layer_bwd",
           "hstu_fp8_quantize_rows", "hstu_fp8_prepare_weight", "hstu_fp8_linear",
           "hstu_layernorm_gate_fp8",
           "hstu_profile_begin", "hstu_profile_end", "hstu_kernel_name", "hstu_kernel_count",
           "hstu_last_error")


class HstuError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("d_qk", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("max_len", ctypes.c_int32),
        ("n_time_buckets", ctypes.c_int32),
        ("rab_heads", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("stride_q", ctypes.c_int64),
        ("stride_k", ctypes.c_int64),
        ("stride_v", ctypes.c_int64),
        ("stride_u", ctypes.c_int64),
        ("deterministic", ctypes.c_int32),
    ]


class BwdInfo(ctypes.Structure):
    _fields_ = [("dq_from_ds", ctypes.c_int32), ("rab_deterministic", ctypes.c_int32),
                ("ds_sequences", ctypes.c_int32)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIGS = {
    "hstu_attn_fwd_workspace_size": [ctypes.POINTER(AttnDesc), ctypes.POINTER(ctypes.c_size_t)],
    "hstu_attn_bwd_workspace_size": [ctypes.POINTER(AttnDesc), ctypes.POINTER(ctypes.c_size_t)],
    "hstu_attn_bwd_workspace_size_min": [ctypes.POINTER(AttnDesc), ctypes.POINTER(ctypes.c_size_t)],
    "hstu_attn_bwd_report": [ctypes.POINTER(AttnDesc), _P, ctypes.c_size_t, ctypes.POINTER(BwdInfo), _P],
    "hstu_attn_fwd": [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                      ctypes.c_size_t, _P],
    "hstu_attn_fwd_noalloc": [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "hstu_attn_fwd_cached_workspace_size": [ctypes.POINTER(AttnDesc), _I64,
                                            ctypes.POINTER(ctypes.c_size_t)],
    "hstu_attn_fwd_cached": [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _I64, _P, _P, _P, _P,
                             _P, _P, _P, _P, _P, _P, _I64, _I64, _P, _P, _P, ctypes.c_size_t, _P],
    "hstu_attn_bwd": [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                      _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "hstu_rab_bucketize": [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P, _P],
    "hstu_rab_pair_offsets": [ctypes.POINTER(AttnDesc), _P, _P, _P, _P],
    "hstu_linear": [_I64, _I64, _I64, _P, _I64, _P, _P, _P, ctypes.c_int32, _P],
    "hstu_layernorm_gate": [_I64, _I64, _P, _P, _I64, ctypes.c_float, _P, _P],
    "hstu_layer_bwd_workspace_size": [_I64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)],
    "hstu_layer_bwd": [_I64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                       ctypes.c_int32, _P, _P,
                       _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _P, _P, _P, _P,
                       ctypes.c_size_t, _P],
    "hstu_fp8_quantize_rows": [_I64, _I64, _P, _I64, _P, _P, _P],
    "hstu_fp8_prepare_weight": [_I64, _I64, _P, _P, _P, _P],
    "hstu_fp8_linear": [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P],
    "hstu_layernorm_gate_fp8": [_I64, _I64, _P, _P, _I64, ctypes.c_float, _P, _P, _P],
    "hstu_profile_begin": [],
    "hstu_profile_end": [ctypes.c_int32, _P, _P],
    "hstu_kernel_count": [],
}

_lib = None


def load(path: str = LIB_PATH):
    """Load (once) and return the library with typed entry points."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m hstu_pointwise_attention_amd.build`")
    import torch  # noqa: F401  (binds the library to torch's HIP runtime)
    lib = ctypes.CDLL(path)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.hstu_last_error.argtypes = []
    lib.hstu_last_error.restype = ctypes.c_char_p
    lib.hstu_kernel_name.argtypes = [ctypes.c_int32]
    lib.hstu_kernel_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != HSTU_OK:
        msg = _lib.hstu_last_error().decode() if _lib is not None else ""
        raise HstuError(status, msg)


class KernelTimer:
    """Per-kernel HIP-event timing of the library's launches (see hstu_profile_*)."""

    def __enter__(self):
        self.lib = load()
        check(self.lib.hstu_profile_begin())
        return self

    def __exit__(self, *exc):
        n = self.lib.hstu_kernel_count()
        ms = (ctypes.c_double * n)()
        cnt = (ctypes.c_int32 * n)()
        check(self.lib.hstu_profile_end(n, ms, cnt))
        self.results = {self.lib.hstu_kernel_name(i).decode(): (ms[i], cnt[i])
                        for i in range(n) if cnt[i] > 0}
        return False

    def avg_ms(self, name: str) -> float:
        total, count = self.results.get(name, (0.0, 0))
        return total / count if count else float("nan")
