"""Candidate scoring against a cached history (hstu_attn_fwd_cached), through
the C ABI (needs a gfx950 GPU).

The call's outputs are defined as the candidate rows of the single-shot
forward over [history, all candidates] with num_targets = number of
candidates, so the oracle is oracle.attention_fwd (or its sampled-row form)
on that whole sequence; each test splits every sequence's candidates into
micro-batches, runs one call per micro-batch against the same history keys
and values, and compares the concatenated candidate rows.
"""
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


def _splits(n, n_micro, rng):
    """Cut n candidates into n_micro consecutive pieces (some may be empty)."""
    cuts = np.sort(rng.integers(0, n + 1, size=n_micro - 1)) if n_micro > 1 else np.zeros(0, np.int64)
    return np.concatenate([[0], cuts, [n]]).astype(np.int64)


def _run_cached(inp, hist, n_cand, n_micro, rng, dtype_t):
    """One call per micro-batch; returns O, A of every candidate row, in sequence order."""
    import torch
    from hstu_pointwise_attention_amd import ops
    offs = inp["seq_offsets"]
    B = len(hist)
    H, D = inp["q"].shape[1], inp["q"].shape[2]
    hrows = np.concatenate([np.arange(offs[b], offs[b] + hist[b]) for b in range(B)]).astype(np.int64) \
        if B else np.zeros(0, np.int64)
    hist_offsets = np.concatenate([[0], np.cumsum(hist)]).astype(np.int64)
    dev = lambda x, dt=dtype_t: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt)
    k_hist = dev(inp["k"][hrows]).reshape(len(hrows), H, D)
    v_hist = dev(inp["v"][hrows]).reshape(len(hrows), H, D)
    ts = inp["timestamps"]
    ts_hist = dev(ts[hrows], torch.int64) if ts is not None else None
    rp = dev(inp["rab_pos"], torch.float32) if inp["rab_pos"] is not None else None
    rt = dev(inp["rab_time"], torch.float32) if inp["rab_time"] is not None else None
    cuts = [_splits(int(n_cand[b]), n_micro, rng) for b in range(B)]
    got_O = {b: [] for b in range(B)}
    got_A = {b: [] for b in range(B)}
    for mb in range(n_micro):
        rows, first, cnt = [], [], []
        for b in range(B):
            c0, c1 = int(cuts[b][mb]), int(cuts[b][mb + 1])
            s = int(offs[b]) + int(hist[b])
            rows.append(np.arange(s + c0, s + c1))
            first.append(c0)
            cnt.append(c1 - c0)
        rows = np.concatenate(rows).astype(np.int64)
        cand_offsets = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int64)
        u = dev(inp["u"][rows]) if inp["u"] is not None else None
        O, A = ops.attn_fwd_cached(dev(inp["q"][rows]), dev(inp["k"][rows]), dev(inp["v"][rows]), u,
                                   dev(cand_offsets, torch.int64), dev(np.array(first), torch.int64),
                                   dev(np.asarray(n_cand), torch.int64), k_hist, v_hist,
                                   dev(hist_offsets, torch.int64), inp["max_len"],
                                   ts_hist=ts_hist,
                                   ts_cand=dev(ts[rows], torch.int64) if ts is not None else None,
                                   rab_pos=rp, rab_time=rt)
        O, A = P.host(O), P.host(A)
        for b in range(B):
            got_O[b].append(O[cand_offsets[b]:cand_offsets[b + 1]])
            got_A[b].append(A[cand_offsets[b]:cand_offsets[b + 1]])
    O = np.concatenate([x for b in range(B) for x in got_O[b]]) if B else np.zeros((0, H, D))
    A = np.concatenate([x for b in range(B) for x in got_A[b]]) if B else np.zeros((0, H, D))
    return O, A


def _cand_rows(offs, hist, n_cand):
    return np.concatenate([np.arange(offs[b] + hist[b], offs[b] + hist[b] + n_cand[b])
                           for b in range(len(hist))]).astype(np.int64)


def _case(dtype, hist, n_cand, *, H, D, max_len, nb, pos, rab_heads, gated, n_micro, seed):
    import torch
    hist = np.asarray(hist, np.int64)
    n_cand = np.asarray(n_cand, np.int64)
    lengths = hist + n_cand
    w = W.AttnWorkload("cached", 0, len(lengths), H, D, D, max_len, nb, pos, dtype, "fixed",
                       tuple(int(x) for x in lengths), rab_heads=rab_heads, gated=gated,
                       backward=False)
    inp = W.make_attention_inputs(w, seed=seed)
    inp["num_targets"] = n_cand.copy()
    want_O, want_A = P.oracle_fwd(inp)
    rows = _cand_rows(inp["seq_offsets"], hist, n_cand)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    O, A = _run_cached(inp, hist, n_cand, n_micro, np.random.default_rng(seed + 77), dt)
    tag = f"{dtype} H{H} D{D} hist {list(hist)} cands {list(n_cand)} micro {n_micro}"
    print(tag, flush=True)
    P.check_fwd(inp, O, A, want_O[rows], want_A[rows], tag=tag)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("seed", range(5))
def test_cached_random(dtype, seed):
    """Random shapes: history 0..300 rows, 0..40 candidates, 1..4 micro-batches."""
    rng = np.random.default_rng(2000 + seed)
    B = int(rng.integers(1, 5))
    H = int(rng.choice([1, 2, 4]))
    D = int(rng.choice([32, 64, 128]))
    hist = rng.integers(0, 301, size=B)
    n_cand = rng.integers(0, 41, size=B)
    n_cand[rng.integers(B)] = int(rng.integers(1, 41))
    nb = int(rng.choice([0, 16, 128]))
    _case(dtype, hist, n_cand, H=H, D=D, max_len=400, nb=nb,
          pos=bool(rng.integers(2)) or nb == 0, rab_heads=int(rng.choice([1, H])),
          gated=bool(rng.integers(2)), n_micro=int(rng.integers(1, 5)), seed=seed)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_cached_edges(dtype):
    """No history, a single candidate, history ending on tile edges, empty micro-batches."""
    _case(dtype, [0, 1, 63, 64, 127, 128, 129], [3, 1, 5, 1, 64, 2, 130],
          H=2, D=32, max_len=300, nb=16, pos=True, rab_heads=1, gated=True, n_micro=3, seed=11)


def test_cached_split_history_fp32():
    """History long enough that each candidate block's history is split over
    several workgroups whose partial A are summed (fp32: exact to 1e-5)."""
    _case("fp32", [1200, 700, 1500], [40, 9, 70], H=2, D=64, max_len=1600, nb=128, pos=True,
          rab_heads=2, gated=True, n_micro=2, seed=16)


def test_cached_long_history_bf16():
    """Several history tiles and query blocks of candidates, head dim 128."""
    _case("bf16", [1500, 2100], [200, 70], H=2, D=128, max_len=2400, nb=128, pos=True,
          rab_heads=1, gated=True, n_micro=4, seed=12)


def test_cached_matches_single_shot_sizes():
    """The M-FALCON layer's attention shape on a sampled subset: 2 users with
    8192 history rows and 1024 candidates scored in micro-batches of 256,
    H 4, D 128, no bias (the layer's target-aware attention), bf16; sampled
    candidate rows against oracle.attention_fwd_rows."""
    import torch
    hist = np.array([8192, 8192], np.int64)
    n_cand = np.array([1024, 1024], np.int64)
    lengths = hist + n_cand
    w = W.AttnWorkload("cached_layer", 0, 2, 4, 128, 128, 9216, 0, False, "bf16", "fixed",
                       tuple(int(x) for x in lengths), gated=True, backward=False)
    inp = W.make_attention_inputs(w, seed=13)
    inp["num_targets"] = n_cand.copy()
    O, A = _run_cached(inp, hist, n_cand, 4, np.random.default_rng(90), torch.bfloat16)
    rows_all = _cand_rows(inp["seq_offsets"], hist, n_cand)
    pick = np.array([0, 1, 255, 256, 511, 1023, 1024, 1300, 2047], np.int64)
    wO, wA = oracle.attention_fwd_rows(inp["q"], inp["k"], inp["v"], inp["u"], inp["seq_offsets"],
                                       inp["max_len"], rows_all[pick], inp["num_targets"])
    err = float(np.max(np.abs(O[pick] - wO)))
    assert err <= P.BF16_O_MAXABS, ("O max-abs", err)
    assert P.rel_l2(O[pick], wO) <= P.BF16_REL
    assert P.rel_l2(A[pick], wA) <= P.BF16_REL


def test_cached_wide_timestamps():
    """Timestamp spans beyond 32 bits take the 64-bit instantiation."""
    rng = np.random.default_rng(14)
    hist = np.array([90, 40], np.int64)
    n_cand = np.array([12, 7], np.int64)
    lengths = hist + n_cand
    w = W.AttnWorkload("cached_wide", 0, 2, 2, 64, 64, 200, 128, True, "bf16", "fixed",
                       tuple(int(x) for x in lengths), gated=False, backward=False)
    inp = W.make_attention_inputs(w, seed=14)
    inp["num_targets"] = n_cand.copy()
    inp["timestamps"] = np.sort(rng.integers(0, 1 << 40, size=int(lengths.sum()))).astype(np.int64)
    import torch
    want_O, want_A = P.oracle_fwd(inp)
    rows = _cand_rows(inp["seq_offsets"], hist, n_cand)
    O, A = _run_cached(inp, hist, n_cand, 2, np.random.default_rng(15), torch.bfloat16)
    P.check_fwd(inp, O, A, want_O[rows], want_A[rows], tag="wide")
