"""Parity of the HIP path (through the C ABI) with the CPU oracle. Needs a gfx950 GPU."""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hstu_pointwise_attention_amd import _lib
    _lib.load()


def _bucket_oracle(inp, nb):
    """Oracle buckets over the unmasked pairs in export order."""
    offs = inp["seq_offsets"]
    nt = inp["num_targets"]
    bps, bts = [], []
    for b in range(len(offs) - 1):
        s, e = int(offs[b]), int(offs[b + 1])
        L = e - s
        if L == 0:
            continue
        hist = L - (0 if nt is None else int(nt[b]))
        rows = np.arange(L)
        bp = oracle.position_buckets(rows, np.arange(L), hist, inp["max_len"])
        bt = oracle.time_buckets(inp["timestamps"][s:e], inp["timestamps"][s:e], nb) \
            if inp["timestamps"] is not None else None
        for i in range(L):
            cols = np.arange(i + 1) if i < hist else np.concatenate([np.arange(hist), [i]])
            bps.append(bp[i, cols])
            if bt is not None:
                bts.append(bt[i, cols])
    bp = np.concatenate(bps) if bps else np.zeros(0, np.int64)
    bt = np.concatenate(bts) if bts else None
    return bp, bt


def _bucket_case(inp, nb):
    from hstu_pointwise_attention_amd import ops
    dev = P.to_dev(inp)
    bp, bt = ops.rab_bucketize(dev["seq_offsets"], inp["max_len"], num_targets=dev["num_targets"],
                               timestamps=dev["timestamps"], n_time_buckets=nb)
    want_bp, want_bt = _bucket_oracle(inp, nb)
    assert np.array_equal(bp.cpu().numpy().astype(np.int64), want_bp)
    if want_bt is not None:
        assert np.array_equal(bt.cpu().numpy().astype(np.int64), want_bt)


@pytest.mark.parametrize("w", [W.TINY, W.PUBLIC, W.LONG], ids=lambda w: w.name)
def test_bucketize_bit_exact(w):
    inp = W.make_attention_inputs(w)
    _bucket_case(inp, w.n_time_buckets)


def test_bucketize_edge_timestamps():
    rng = np.random.default_rng(7)
    lengths = np.array([5, 0, 9, 1, 12])
    offs = W.offsets_from_lengths(lengths)
    T = int(offs[-1])
    i64 = np.iinfo(np.int64)
    cases = [
        rng.integers(-10 ** 6, 10 ** 6, size=T),                      # unsorted, negative
        np.sort(rng.integers(0, 1 << 40, size=T)),                     # span wider than 2^31
        np.array([i64.min, i64.max] * (T // 2) + [0] * (T % 2)),       # extreme int64 values
        np.full(T, 12345),                                             # all ties
    ]
    for ts in cases:
        for nb in (1, 7, 64, 128):
            inp = dict(seq_offsets=offs, num_targets=np.array([1, 0, 3, 1, 12]),
                       timestamps=ts.astype(np.int64), max_len=6, dtype="fp32")
            _bucket_case(inp, nb)


def _run_parity(inp, backward=True, tag=""):
    O, A = P.gpu_fwd(inp)
    want_O, want_A = P.oracle_fwd(inp)
    P.check_fwd(inp, P.host(O), P.host(A), want_O, want_A, tag)
    if backward:
        got = P.gpu_bwd(inp, A)
        want = P.oracle_bwd(inp)
        P.check_bwd(inp, got, want, tag)


@pytest.mark.parametrize("w", [W.TINY, W.PUBLIC, W.LONG], ids=lambda w: w.name)
def test_workload_parity(w):
    _run_parity(W.make_attention_inputs(w), tag=w.name)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("seed", range(6))
def test_random_small_sweep(dtype, seed):
    """Random small shapes over tile edges: lengths 0..300, H, D, rab and targets varied."""
    rng = np.random.default_rng(1000 + seed)
    H = int(rng.choice([1, 2, 4]))
    D = int(rng.choice([32, 64] if dtype == "fp32" else [32, 64, 128]))
    B = int(rng.integers(1, 6))
    max_len = int(rng.choice([16, 64, 300]))
    nb = int(rng.choice([0, 16, 128]))
    lengths = rng.integers(0, 301, size=B)
    lengths[rng.integers(B)] = int(rng.choice([1, 64, 128, 129, 255, 300]))
    w = W.AttnWorkload("sweep", 0, B, H, D, D, max_len, nb, bool(rng.integers(2)) or nb == 0,
                       dtype, "fixed", tuple(int(x) for x in lengths),
                       rab_heads=int(rng.choice([1, H])), gated=bool(rng.integers(2)))
    inp = W.make_attention_inputs(w, seed=seed)
    if rng.integers(2):
        inp["num_targets"] = np.minimum(rng.integers(0, 40, size=B), lengths).astype(np.int64)
    _run_parity(inp, tag=f"{dtype} seed {seed} H{H} D{D} L{list(lengths)}")


def _timestamps(kind, offs, rng):
    """Per-sequence timestamps of one kind (int64 seconds)."""
    T = int(offs[-1])
    i64 = np.iinfo(np.int64)
    if kind == "unsorted":
        return rng.integers(-10 ** 6, 10 ** 6, size=T)
    if kind == "wide":                                   # spans wider than 2^31: 64-bit buckets
        return np.sort(rng.integers(0, 1 << 40, size=T))
    if kind == "extreme":
        return np.array(([i64.min, i64.max] * T)[:T], dtype=np.int64)
    if kind == "ties":
        return np.full(T, 1_700_000_000, dtype=np.int64)
    out = np.zeros(T, dtype=np.int64)
    for b in range(len(offs) - 1):
        s, e = int(offs[b]), int(offs[b + 1])
        seq = 1_700_000_000 + np.cumsum(rng.integers(0, 4000, size=e - s))
        if kind == "before_first" and e - s > 2:      # one value 2^30 + 5 s before the first
            seq[(e - s) // 2] = seq[0] - (1 << 30) - 5
        if kind == "mixed" and b % 2 == 1:             # every other sequence needs 64 bits
            seq = seq + np.arange(e - s, dtype=np.int64) * (1 << 28)
        out[s:e] = seq
    return out


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("kind", ["unsorted", "wide", "extreme", "ties", "before_first", "mixed"])
def test_timestamp_kinds(dtype, kind):
    """Timestamps off the sorted 32-bit fast paths, through forward and backward: unsorted and
    negative, spans past 2^31 (the 64-bit bucket kernels), extreme int64 values, all ties, a
    value more than 2^30 s before the first one, and a batch mixing both kernel kinds."""
    lengths = (5, 0, 70, 1, 130, 200)
    D = 64 if dtype == "fp32" else 128
    w = W.AttnWorkload("tskinds", 31, len(lengths), 2, D, D, 256, 128, True, dtype, "fixed",
                       lengths)
    inp = W.make_attention_inputs(w)
    inp["timestamps"] = _timestamps(kind, inp["seq_offsets"], np.random.default_rng(77)).astype(np.int64)
    _run_parity(inp, tag=f"{dtype} {kind}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_edge_lengths(dtype):
    """Empty sequences, L=1, exactly one tile, one past a tile, all-candidate sequences."""
    lengths = (0, 1, 128, 129, 0, 64, 65, 2)
    w = W.AttnWorkload("edges", 5, len(lengths), 2, 32, 32, 100, 32, True, dtype, "fixed", lengths)
    inp = W.make_attention_inputs(w)
    _run_parity(inp, tag="edges")
    inp["num_targets"] = np.array([0, 1, 5, 129, 0, 64, 3, 2], dtype=np.int64)
    _run_parity(inp, tag="edges+targets")


def test_empty_batch():
    from hstu_pointwise_attention_amd import ops
    import torch
    q = torch.zeros((0, 2, 32), dtype=torch.bfloat16, device="cuda")
    offs = torch.zeros(1, dtype=torch.int64, device="cuda")
    o, a = ops.attn_fwd(q, q, q, q, offs, 10)
    assert o.shape == (0, 2, 32)
    rp = torch.randn((1, 19), device="cuda")
    g = ops.attn_bwd(q, q, q, q, offs, 10, a, q, rab_pos=rp)
    assert float(g["d_rab_pos"].abs().sum()) == 0.0


def test_causality_nan_poison():
    """Future keys/queries set to NaN, future values perturbed: past rows bit-identical."""
    w = dataclasses.replace(W.TINY, dtype="bf16", length_args=(7, 13, 32, 50))
    inp = W.make_attention_inputs(w)
    O1, _ = P.gpu_fwd(inp)
    offs = inp["seq_offsets"]
    cut = {b: int(offs[b]) + L // 2 for b, L in enumerate(np.diff(offs))}
    p = {key: inp[key].copy() for key in ("q", "k", "v", "u")}
    for b in range(len(offs) - 1):
        e = int(offs[b + 1])
        p["k"][cut[b] + 1:e] = np.nan
        p["q"][cut[b] + 1:e] = np.nan
        p["v"][cut[b] + 1:e] = 3.0
    inp2 = dict(inp, **p)
    O2, _ = P.gpu_fwd(inp2)
    O1, O2 = P.host(O1), P.host(O2)
    for b in range(len(offs) - 1):
        s = int(offs[b])
        assert np.array_equal(O1[s:cut[b] + 1], O2[s:cut[b] + 1]), b


def test_batch_order_and_alone():
    inp = W.make_attention_inputs(W.PUBLIC)
    O, _ = P.gpu_fwd(inp)
    O = P.host(O)
    offs = inp["seq_offsets"]
    lens = np.diff(offs)
    perm = np.random.default_rng(3).permutation(len(lens))
    idx = np.concatenate([np.arange(offs[b], offs[b + 1]) for b in perm])
    inp2 = dict(inp)
    for key in ("q", "k", "v", "u", "timestamps"):
        inp2[key] = inp[key][idx]
    inp2["seq_offsets"] = W.offsets_from_lengths(lens[perm])
    O2, _ = P.gpu_fwd(inp2)
    assert np.array_equal(P.host(O2), O[idx])
    b = 17
    sl = slice(int(offs[b]), int(offs[b + 1]))
    inp3 = dict(inp)
    for key in ("q", "k", "v", "u", "timestamps"):
        inp3[key] = inp[key][sl]
    inp3["seq_offsets"] = np.array([0, lens[b]])
    O3, _ = P.gpu_fwd(inp3)
    assert np.array_equal(P.host(O3), O[sl])


def test_autograd_function_matches_ops():
    import torch
    from hstu_pointwise_attention_amd import hstu_attention
    inp = W.make_attention_inputs(W.TINY)
    dev = P.to_dev(inp)
    leaves = {k: dev[k].clone().requires_grad_(True) for k in ("q", "k", "v", "u", "rab_pos", "rab_time")}
    o = hstu_attention(leaves["q"], leaves["k"], leaves["v"], leaves["u"], dev["seq_offsets"],
                       inp["max_len"], timestamps=dev["timestamps"], rab_pos=leaves["rab_pos"],
                       rab_time=leaves["rab_time"])
    (o * dev["d_o"]).sum().backward()
    want = P.oracle_bwd(inp)
    for key, gk in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("u", "du"), ("rab_pos", "d_rab_pos"),
                    ("rab_time", "d_rab_time")):
        assert P.rel_l2(P.host(leaves[key].grad), want[gk]) <= P.FP32_REL, key


def test_bf16_dq_paths_agree():
    """The bf16 backward computes dQ from the key-block kernel's exported dS
    tiles when the batch's tiles fit the workspace sized from max_len, and by
    recomputing dS otherwise. Without a position bias max_len changes nothing
    else, so the same inputs run both ways: lengths 300, 200, 77 with H 2 hold
    2 * (9 + 6 + 2) = 34 tiles; max_len 512 sizes room for 2 * 5 * 7 = 70
    (export), max_len 64 for 2 * 2 * 7 = 28 (recompute). Both match the oracle
    and each other."""
    lengths = (300, 200, 77)
    w = W.AttnWorkload("dqpaths", 41, 3, 2, 64, 64, 512, 16, False, "bf16", "fixed", lengths)
    inp = W.make_attention_inputs(w)
    inp["num_targets"] = np.array([20, 0, 5], np.int64)
    want = P.oracle_bwd(inp)
    got = {}
    for max_len in (512, 64):
        run = dict(inp, max_len=max_len)
        _, A = P.gpu_fwd(run)
        got[max_len] = P.gpu_bwd(run, A)
        P.check_bwd(run, got[max_len], want, f"max_len {max_len}")
    assert P.rel_l2(P.host(got[512]["dq"]), P.host(got[64]["dq"])) <= P.BF16_REL
