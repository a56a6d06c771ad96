"""hstu_attn_fwd_noalloc: the forward with its workspace inside the library.

Two calls in a row through the C ABI, the second on a smaller batch, each
compared with hstu_attn_fwd on the same inputs (same kernels, so bit for bit)
and with the oracle at the bf16 / fp32 bars. The size check runs on the host
before any launch, so it needs no GPU.
"""
import ctypes

import numpy as np
import pytest

import workloads as W
from tests import parity as P


def _desc(inp, dev):
    from hstu_pointwise_attention_amd import ops
    nt = inp["rab_time"].shape[1] if inp["rab_time"] is not None else 0
    hr = (inp["rab_pos"] if inp["rab_pos"] is not None else inp["rab_time"]).shape[0]
    return ops.make_desc(dev["q"], dev["k"], dev["v"], dev["u"], dev["seq_offsets"], inp["max_len"],
                         nt, hr)


def _noalloc(inp, dev):
    import torch
    from hstu_pointwise_attention_amd import _lib, ops
    lib = _lib.load()
    d = _desc(inp, dev)
    T, H, _ = dev["q"].shape
    Dv = dev["v"].shape[2]
    o = torch.full((T, H, Dv), float("nan"), dtype=dev["q"].dtype, device="cuda")
    a = torch.full((T, H, Dv), float("nan"), dtype=torch.float32, device="cuda")
    _lib.check(lib.hstu_attn_fwd_noalloc(ctypes.byref(d), ops._ptr(dev["seq_offsets"]),
                                         ops._ptr(dev["num_targets"]), ops._ptr(dev["timestamps"]),
                                         ops._ptr(dev["rab_pos"]), ops._ptr(dev["rab_time"]),
                                         ops._ptr(dev["q"]), ops._ptr(dev["k"]), ops._ptr(dev["v"]),
                                         ops._ptr(dev["u"]), ops._ptr(o), ops._ptr(a), ops._stream()))
    return o, a


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_matches_fwd_two_calls(dtype):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = W.make_attention_inputs(W.LONG if dtype == "bf16" else
                                  W.AttnWorkload("na", 61, 6, 2, 64, 64, 300, 64, True, "fp32",
                                                 "fixed", (300, 0, 129, 64, 1, 200)))
    small = W.make_attention_inputs(W.TINY if dtype == "fp32" else
                                    W.AttnWorkload("na2", 62, 3, 2, 128, 128, 100, 32, True,
                                                   "bf16", "fixed", (65, 1, 100)))
    small["num_targets"] = np.array([3, 0, 1] if dtype == "bf16" else [0, 2, 0, 5], np.int64)
    assert int(small["seq_offsets"][-1]) < int(big["seq_offsets"][-1])
    for inp in (big, small):
        dev = P.to_dev(inp)
        o, a = _noalloc(inp, dev)
        want_o, want_a = P.gpu_fwd(inp, dev)
        torch.cuda.synchronize()
        assert torch.equal(o, want_o) and torch.equal(a, want_a)
        P.check_fwd(inp, P.host(o), P.host(a), *P.oracle_fwd(inp), tag=f"noalloc {dtype}")


def test_noalloc_rejects_oversized_shape():
    from hstu_pointwise_attention_amd import _lib
    if not __import__("os").path.exists(_lib.LIB_PATH):
        pytest.skip("library not built")
    lib = _lib.load()
    d = _lib.AttnDesc()
    d.batch, d.heads, d.d_qk, d.d_v, d.max_len, d.rab_heads, d.dtype = 1000, 1, 32, 32, 10, 1, 0
    d.total_tokens = (1 << 31) - 1                 # workspace far above 16 MiB
    d.stride_q = d.stride_k = d.stride_v = 32
    fake = ctypes.c_void_p(4096)                   # never dereferenced: rejected on the host
    st = lib.hstu_attn_fwd_noalloc(ctypes.byref(d), fake, None, None, None, None, fake, fake,
                                   fake, None, fake, None, None)
    assert st == _lib.HSTU_EWORKSPACE
    assert "16777216" in lib.hstu_last_error().decode()
