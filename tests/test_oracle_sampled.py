"""Pins of the sampled-output oracle (oracle/sampled.py) against the scalar brute force (CPU)."""
import numpy as np
import pytest

import oracle
from oracle import sampled
from oracle.buckets import time_buckets
from tests import pins


def _scalar(c, d_o):
    return oracle.scalar_attention_bwd(c["q"], c["k"], c["v"], c["u"], c["seq_offsets"],
                                       c["max_len"], d_o, c["num_targets"], c["timestamps"],
                                       c["rab_pos"], c["rab_time"])


CASES = [
    dict(seed=31, targets=[1, 0, 0, 2]),
    dict(seed=32, targets=None, rab_heads=2),
    dict(seed=33, targets=[0, 3, 1, 1], gate=False),
    dict(seed=34, targets=None, pos=False),
]


@pytest.mark.parametrize("kw", CASES, ids=lambda k: f"seed{k['seed']}")
def test_rows_and_cols_match_scalar(kw):
    c, d_o = pins.tiny_case(**kw)
    want = _scalar(c, d_o)
    T = int(c["seq_offsets"][-1])
    toks = np.arange(T)
    args = (c["q"], c["k"], c["v"], c["u"], c["seq_offsets"], c["max_len"], d_o)
    rest = dict(num_targets=c["num_targets"], timestamps=c["timestamps"], rab_pos=c["rab_pos"],
                rab_time=c["rab_time"])
    dq, du = sampled.attention_bwd_rows(*args, toks, **rest)
    dk, dv = sampled.attention_bwd_cols(*args, toks, **rest)
    assert pins.rel(dq, np.array(want["dq"])) < 1e-12
    assert pins.rel(dk, np.array(want["dk"])) < 1e-12
    assert pins.rel(dv, np.array(want["dv"])) < 1e-12
    if c["u"] is None:
        assert du is None
    else:
        assert pins.rel(du, np.array(want["du"])) < 1e-12


@pytest.mark.parametrize("rab_heads", [1, 2])
def test_diagonal_sums_are_position_gradient(rab_heads):
    # no candidates, every length <= max_len: diagonal delta <-> bucket delta + max_len - 1
    c, d_o = pins.tiny_case(35, lengths=(3, 6, 1, 5), max_len=6, rab_heads=rab_heads)
    want = np.array(_scalar(c, d_o)["d_rab_pos"])
    deltas = np.arange(0, -6, -1)
    got = sampled.diagonal_ds_sums(c["q"], c["k"], c["v"], c["u"], c["seq_offsets"], c["max_len"],
                                   d_o, deltas, c["timestamps"], c["rab_pos"], c["rab_time"])
    idx = deltas + c["max_len"] - 1
    if rab_heads == 1:
        assert got.shape == (6,)
        assert pins.rel(got, want[0, idx]) < 1e-12
    else:
        assert got.shape == (2, 6)
        assert pins.rel(got, want[:, idx]) < 1e-12
    # entries of positive offsets are never read by causal pairs
    assert np.all(want[:, c["max_len"]:] == 0)


def test_time_bucket_pairs_match_grid():
    rng = np.random.default_rng(36)
    a = rng.integers(-2**62, 2**62, size=200)
    b = rng.integers(-2**62, 2**62, size=200)
    a[:4] = [np.iinfo(np.int64).max, np.iinfo(np.int64).min, 0, 5]
    b[:4] = [np.iinfo(np.int64).min, np.iinfo(np.int64).max, 0, 5]
    for nb in (64, 128):
        grid = time_buckets(a, b, nb)
        assert np.array_equal(sampled._time_bucket_pairs(a, b, nb), np.diag(grid))


def test_locate():
    offs = np.array([0, 3, 3, 10])
    assert sampled.locate(offs, 0) == (0, 0)
    assert sampled.locate(offs, 2) == (0, 2)
    assert sampled.locate(offs, 3) == (2, 0)      # empty sequence 1 is skipped
    assert sampled.locate(offs, 9) == (2, 6)


RAB_CASES = [
    dict(seed=41, targets=[1, 0, 0, 2]),
    dict(seed=42, targets=None, rab_heads=2),
    dict(seed=43, targets=[0, 3, 1, 1], gate=False),
    dict(seed=44, targets=None, pos=False),
]


@pytest.mark.parametrize("kw", RAB_CASES, ids=lambda k: f"seed{k['seed']}")
@pytest.mark.parametrize("workers", [1, 2])
def test_rab_gradients_match_scalar(kw, workers):
    c, d_o = pins.tiny_case(**kw)
    want = _scalar(c, d_o)
    gp, gt = sampled.rab_gradients(c["q"], c["k"], c["v"], c["u"], c["seq_offsets"], c["max_len"],
                                   d_o, c["num_targets"], c["timestamps"], c["rab_pos"],
                                   c["rab_time"], workers=workers, rows_per=3)
    for got, key in ((gp, "d_rab_pos"), (gt, "d_rab_time")):
        w = want[key]
        if w is None:
            assert got is None
        else:
            assert pins.rel(got, np.array(w)) < 1e-12, key
