"""Seeded synthetic inputs for jagged HSTU attention.

This module only draws random inputs and lays them out. It holds none of the
attention arithmetic, so both the CPU oracle's tests and the GPU path's tests
can use it without sharing any of the method's code.

Workloads follow the shapes the pages benchmark: public sequential-recsys
batches (history lengths up to 200, the ``*-l200`` log folders of the
Generative Recommenders README, "Public Experiments"), long histories, and the
8192-length efficiency setting of the HSTU paper's Abstract ("Actions Speak
Louder than Words ...", which reports its speedup over FlashAttention2 at that
sequence length). No
public dataset is read: every tensor is drawn here from a seed.

Draw order for one workload (all draws in float64 from
``numpy.random.default_rng(seed)``):

1. sequence lengths;
2. timestamp gaps, per sequence in order (``L - 1`` gaps each);
3. Q, K, V, U, each ``[T, H, D]``, in that order;
4. rab_pos ``[Hr, 2*max_len-1]``, rab_time ``[Hr, n_time_buckets]``;
5. dO ``[T, H, Dv]``.

Each float tensor is rounded once to the workload's dtype: float32 values
for "fp32", and for "bf16" values rounded to bfloat16 (round to nearest
even, via float32), stored as float32 arrays whose values are exactly
representable in bfloat16. rab tables are float32 in every mode.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

T0_SECONDS = 1_700_000_000
GAP_MEAN_SECONDS = 3600.0


def round_to_bf16(x) -> np.ndarray:
    """Round to bfloat16 (nearest even) via float32; return float32 values."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32).reshape(f.shape)


def round_to(x, dtype: str) -> np.ndarray:
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16(x)
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    """One jagged attention workload (shape, distributions, seed)."""

    name: str
    seed: int
    batch: int
    heads: int
    d_qk: int
    d_v: int
    max_len: int
    n_time_buckets: int          # 0: no time bias
    use_pos_bias: bool
    dtype: str                   # "fp32" | "bf16"
    length_kind: str             # "fixed" | "uniform" | "powerlaw"
    length_args: tuple
    num_targets: int = 0         # candidates appended to every sequence
    rab_heads: int = 1           # 1: one table shared by all heads; else H
    input_std: float = 0.5
    rab_std: float = 0.02
    gated: bool = True
    backward: bool = True

    @property
    def n_pos_buckets(self) -> int:
        return 2 * self.max_len - 1 if self.use_pos_bias else 0


@dataclasses.dataclass(frozen=True)
class LayerWorkload:
    """Attention inside a full HSTU layer (forward only)."""

    name: str
    seed: int
    batch: int
    history: int
    candidates: int
    heads: int
    head_dim: int
    model_dim: int
    input_std: float = 1.0
    weight_std: float = 0.02
    dtype: str = "bf16"


# The five workloads. Sizes follow the pages' settings (see module docstring).
TINY = AttnWorkload("tiny_fp32", 1001, 4, 2, 32, 32, 50, 64, True, "fp32",
                    "fixed", (7, 13, 32, 50))
PUBLIC = AttnWorkload("public_l200_bf16", 1002, 128, 2, 32, 32, 200, 128, True,
                      "bf16", "uniform", (20, 200))
LONG = AttnWorkload("long_history_bf16", 1003, 32, 4, 64, 64, 1024, 128, True,
                    "bf16", "powerlaw", (64, 1024, 1.2))
EFFICIENCY = AttnWorkload("efficiency_8192_bf16", 1004, 8, 4, 128, 128, 8192, 128,
                          True, "bf16", "uniform", (4096, 8192))
MFALCON_LAYER = LayerWorkload("mfalcon_layer_bf16", 1005, 4, 8192, 1024, 4, 128, 512)

ATTN_WORKLOADS = (TINY, PUBLIC, LONG, EFFICIENCY)


def draw_lengths(rng: np.random.Generator, kind: str, args: tuple, batch: int) -> np.ndarray:
    if kind == "fixed":
        assert len(args) == batch
        return np.asarray(args, dtype=np.int64)
    if kind == "uniform":
        lo, hi = args  # integers, both ends included
        return rng.integers(lo, hi + 1, size=batch, dtype=np.int64)
    if kind == "powerlaw":
        # density proportional to L^-alpha on [lo, hi]; inverse-CDF draw,
        # floored to an integer and clipped to the range.
        lo, hi, alpha = args
        e = 1.0 - alpha
        a, b = lo ** e, hi ** e
        u = rng.random(batch)
        x = (a + u * (b - a)) ** (1.0 / e)
        return np.clip(np.floor(x), lo, hi).astype(np.int64)
    raise ValueError(kind)


def draw_timestamps(rng: np.random.Generator, lengths: np.ndarray) -> np.ndarray:
    """int64 seconds: t0, then t0 + floor(cumulative Exp(3600 s) gaps)."""
    out = []
    for L in lengths.tolist():
        if L == 0:
            continue
        gaps = rng.exponential(GAP_MEAN_SECONDS, size=L - 1)
        cum = np.concatenate([[0.0], np.cumsum(gaps)])
        out.append(T0_SECONDS + np.floor(cum).astype(np.int64))
    if not out:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(out).astype(np.int64)


def offsets_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


def make_attention_inputs(w: AttnWorkload, seed: Optional[int] = None,
                          lengths: Optional[np.ndarray] = None) -> dict:
    """Draw one batch for an attention workload.

    ``lengths`` overrides the drawn lengths (the draw still happens, so the
    rest of the stream is unchanged only when it is not given).
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    drawn = draw_lengths(rng, w.length_kind, w.length_args, w.batch)
    lengths = drawn if lengths is None else np.asarray(lengths, dtype=np.int64)
    B = len(lengths)
    offsets = offsets_from_lengths(lengths)
    T = int(offsets[-1])
    ts = draw_timestamps(rng, lengths) if w.n_time_buckets > 0 else None
    H, Dq, Dv = w.heads, w.d_qk, w.d_v
    s = w.input_std
    q = round_to(s * rng.standard_normal((T, H, Dq)), w.dtype)
    k = round_to(s * rng.standard_normal((T, H, Dq)), w.dtype)
    v = round_to(s * rng.standard_normal((T, H, Dv)), w.dtype)
    u = round_to(s * rng.standard_normal((T, H, Dv)), w.dtype) if w.gated else None
    Hr = w.rab_heads
    rab_pos = (w.rab_std * rng.standard_normal((Hr, w.n_pos_buckets))).astype(np.float32) \
        if w.use_pos_bias else None
    rab_time = (w.rab_std * rng.standard_normal((Hr, w.n_time_buckets))).astype(np.float32) \
        if w.n_time_buckets > 0 else None
    d_o = round_to(rng.standard_normal((T, H, Dv)), w.dtype) if w.backward else None
    nt = np.full(B, w.num_targets, dtype=np.int64) if w.num_targets else None
    if nt is not None:
        nt = np.minimum(nt, lengths)
    return dict(q=q, k=k, v=v, u=u, seq_offsets=offsets, num_targets=nt,
                timestamps=ts, rab_pos=rab_pos, rab_time=rab_time, d_o=d_o,
                max_len=w.max_len, n_time_buckets=w.n_time_buckets,
                lengths=lengths, dtype=w.dtype)


def make_layer_inputs(w: LayerWorkload, seed: Optional[int] = None) -> dict:
    """Inputs of one HSTU layer forward: X, W1, b1, W2, b2 and the jagged batch."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    L = w.history + w.candidates
    lengths = np.full(w.batch, L, dtype=np.int64)
    offsets = offsets_from_lengths(lengths)
    T = int(offsets[-1])
    d = w.model_dim
    x = round_to(w.input_std * rng.standard_normal((T, d)), w.dtype)
    w1 = round_to(w.weight_std * rng.standard_normal((d, 4 * w.heads * w.head_dim)), w.dtype)
    w2 = round_to(w.weight_std * rng.standard_normal((w.heads * w.head_dim, d)), w.dtype)
    b1 = np.zeros(4 * w.heads * w.head_dim, dtype=np.float32)
    b2 = np.zeros(d, dtype=np.float32)
    nt = np.full(w.batch, w.candidates, dtype=np.int64)
    return dict(x=x, w1=w1, b1=b1, w2=w2, b2=b2, seq_offsets=offsets,
                num_targets=nt, lengths=lengths, heads=w.heads,
                head_dim=w.head_dim, dtype=w.dtype)


def random_small_workload(rng: np.random.Generator, *, max_len: int = 64,
                          dtype: str = "fp32") -> AttnWorkload:
    """A small random shape for sweeps over tile edges."""
    H = int(rng.choice([1, 2, 4]))
    D = int(rng.choice([32, 64, 128]))
    B = int(rng.integers(1, 6))
    return AttnWorkload(f"sweep_{H}_{D}_{B}", int(rng.integers(1 << 30)), B, H, D, D,
                        max_len, int(rng.choice([0, 16, 64])), bool(rng.integers(2)),
                        dtype, "uniform", (0, max_len))
