"""Jagged HSTU pointwise attention for AMD MI355X (gfx950).

The computation lives in the HIP library ``libhstu_attn.so`` (C ABI:
``include/hstu_attn.h``); this package only marshals torch tensors into it.
Build the library with ``python -m hstu_pointwise_attention_amd.build``.
"""
from .attention import hstu_attention, hstu_layer_fwd
from .ops import attn_bwd, attn_fwd, layernorm_gate, linear, rab_bucketize
from .flops import attention_flops, unmasked_pairs_host

__all__ = ["hstu_attention", "hstu_layer_fwd", "attn_fwd", "attn_bwd", "rab_bucketize",
           "linear", "layernorm_gate", "attention_flops", "unmasked_pairs_host"]
