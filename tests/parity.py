"""Shared helpers of the GPU parity tests: device transfer, oracle calls, checks."""
from __future__ import annotations

import numpy as np

import oracle

# Tolerances. bf16: output max-abs <= 2e-2 (the stated bar) and, tighter,
# output rel-L2 <= 1e-2 (at long lengths |O| is ~1e-2, where the max-abs bar
# alone says little); every gradient rel-L2 <= 1e-2. fp32: rel-L2 <= 1e-5.
BF16_O_MAXABS = 2e-2
BF16_REL = 1e-2
FP32_REL = 1e-5


def rel_l2(got, want) -> float:
    got = np.asarray(got, dtype=np.float64).ravel()
    want = np.asarray(want, dtype=np.float64).ravel()
    den = np.linalg.norm(want)
    num = np.linalg.norm(got - want)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def to_dev(inp: dict, device="cuda"):
    import torch
    dt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    out = {}
    for key in ("q", "k", "v", "u", "d_o"):
        x = inp.get(key)
        out[key] = None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=dt)
    for key in ("rab_pos", "rab_time"):
        x = inp.get(key)
        out[key] = None if x is None else torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
    for key in ("seq_offsets", "num_targets", "timestamps"):
        x = inp.get(key)
        out[key] = None if x is None else torch.from_numpy(np.asarray(x, dtype=np.int64)).to(device)
    return out


def host(t):
    return None if t is None else t.detach().float().cpu().numpy()


def oracle_fwd(inp):
    return oracle.attention_fwd(inp["q"], inp["k"], inp["v"], inp["u"], inp["seq_offsets"],
                                inp["max_len"], inp["num_targets"], inp["timestamps"],
                                inp["rab_pos"], inp["rab_time"])


def oracle_bwd(inp):
    return oracle.attention_bwd(inp["q"], inp["k"], inp["v"], inp["u"], inp["seq_offsets"],
                                inp["max_len"], inp["d_o"], inp["num_targets"], inp["timestamps"],
                                inp["rab_pos"], inp["rab_time"])


def gpu_fwd(inp, dev=None):
    from hstu_pointwise_attention_amd import ops
    dev = dev or to_dev(inp)
    return ops.attn_fwd(dev["q"], dev["k"], dev["v"], dev["u"], dev["seq_offsets"], inp["max_len"],
                        num_targets=dev["num_targets"], timestamps=dev["timestamps"],
                        rab_pos=dev["rab_pos"], rab_time=dev["rab_time"], save_a=True)


def gpu_bwd(inp, a, dev=None, **kw):
    """kw: deterministic, ds_room, report (ops.attn_bwd)."""
    from hstu_pointwise_attention_amd import ops
    dev = dev or to_dev(inp)
    return ops.attn_bwd(dev["q"], dev["k"], dev["v"], dev["u"], dev["seq_offsets"], inp["max_len"],
                        a if dev["u"] is not None else None, dev["d_o"],
                        num_targets=dev["num_targets"], timestamps=dev["timestamps"],
                        rab_pos=dev["rab_pos"], rab_time=dev["rab_time"], **kw)


def check_fwd(inp, O, A, want_O, want_A, tag=""):
    if inp["dtype"] == "fp32":
        assert rel_l2(O, want_O) <= FP32_REL, (tag, "O", rel_l2(O, want_O))
        assert rel_l2(A, want_A) <= FP32_REL, (tag, "A", rel_l2(A, want_A))
    else:
        err = float(np.max(np.abs(np.asarray(O, np.float64) - want_O))) if want_O.size else 0.0
        assert err <= BF16_O_MAXABS, (tag, "O max-abs", err)
        assert rel_l2(O, want_O) <= BF16_REL, (tag, "O rel", rel_l2(O, want_O))
        assert rel_l2(A, want_A) <= BF16_REL, (tag, "A rel", rel_l2(A, want_A))


def check_bwd(inp, got: dict, want: dict, tag=""):
    tol = FP32_REL if inp["dtype"] == "fp32" else BF16_REL
    for key in ("dq", "dk", "dv", "du", "d_rab_pos", "d_rab_time"):
        w = want.get(key)
        g = got.get(key)
        if w is None:
            assert g is None, (tag, key)
            continue
        e = rel_l2(host(g), w)
        assert e <= tol, (tag, key, e)
