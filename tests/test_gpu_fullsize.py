"""Full-size parity of the HIP path (needs a gfx950 GPU).

The efficiency workload (8 sequences, lengths U[4096, 8192], 4 heads, head
dim 128, bf16, both rab tables) runs through the C ABI exactly as the
benchmark times it; the oracle then evaluates sampled outputs one by one
(oracle/sampled.py): rows of O, A, dQ and dU, key rows of dK and dV,
d_rab_pos entries as diagonal sums of dS, and both rab-table gradients whole
(every entry, from dS over all 478 M unmasked pair-heads, spread over the
host's cores), in the default and in the deterministic mode. The bucket
export is compared bit for bit on rows at tile edges of every sequence,
with all their keys. The M-FALCON layer workload (4 users x (8192 + 1024
candidates), d_model 512) is checked on sampled rows of UVQK, A and Y, and
its backward on sampled rows of dX (with db2 whole).
"""
import os

import numpy as np
import pytest

import oracle
import workloads as W
from oracle import sampled
from oracle.layer import layer_fwd_rows
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hstu_pointwise_attention_amd import _lib
    _lib.load()


def _sample_rows(offs, rng, per_seq=6):
    """Per sequence: first and last rows, rows at 64/128 tile edges, random rows."""
    rows = []
    for b in range(len(offs) - 1):
        s, e = int(offs[b]), int(offs[b + 1])
        L = e - s
        picks = {0, L - 1, min(63, L - 1), min(64, L - 1), min(127, L - 1), min(128, L - 1)}
        picks |= set(int(x) for x in rng.integers(0, L, size=per_seq))
        rows += [s + i for i in sorted(picks)]
    return np.array(rows, dtype=np.int64)


@pytest.fixture(scope="module")
def eff_inputs():
    inp = W.make_attention_inputs(W.EFFICIENCY)
    return inp, P.to_dev(inp)


@pytest.fixture(scope="module")
def efficiency(eff_inputs):
    import torch
    inp, dev = eff_inputs
    O, A = P.gpu_fwd(inp, dev)
    g = P.gpu_bwd(inp, A, dev)
    torch.cuda.synchronize()
    got = {"O": P.host(O), "A": P.host(A)}
    got.update({k: P.host(v) for k, v in g.items()})
    print(f"efficiency workload: T={int(inp['seq_offsets'][-1])}", flush=True)
    return inp, got


@pytest.fixture(scope="module")
def eff_rab_oracle(eff_inputs):
    """Both rab-table gradients of the efficiency workload, every entry (float64)."""
    inp, _ = eff_inputs
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    print(f"oracle rab gradients on {workers} processes", flush=True)
    return sampled.rab_gradients(inp["q"], inp["k"], inp["v"], inp["u"], inp["seq_offsets"],
                                 inp["max_len"], inp["d_o"], inp["num_targets"], inp["timestamps"],
                                 inp["rab_pos"], inp["rab_time"], workers=workers)


def test_efficiency_forward_rows(efficiency):
    inp, got = efficiency
    rows = _sample_rows(inp["seq_offsets"], np.random.default_rng(7))
    wO, wA = oracle.attention_fwd_rows(inp["q"], inp["k"], inp["v"], inp["u"], inp["seq_offsets"],
                                       inp["max_len"], rows, inp["num_targets"], inp["timestamps"],
                                       inp["rab_pos"], inp["rab_time"])
    err = float(np.max(np.abs(got["O"][rows] - wO)))
    assert err <= P.BF16_O_MAXABS, ("O max-abs", err)
    assert P.rel_l2(got["O"][rows], wO) <= P.BF16_REL
    assert P.rel_l2(got["A"][rows], wA) <= P.BF16_REL


def test_efficiency_backward_rows_and_keys(efficiency):
    inp, got = efficiency
    rng = np.random.default_rng(8)
    args = (inp["q"], inp["k"], inp["v"], inp["u"], inp["seq_offsets"], inp["max_len"], inp["d_o"])
    rest = dict(num_targets=inp["num_targets"], timestamps=inp["timestamps"],
                rab_pos=inp["rab_pos"], rab_time=inp["rab_time"])
    rows = _sample_rows(inp["seq_offsets"], rng, per_seq=4)
    dq, du = sampled.attention_bwd_rows(*args, rows, **rest)
    assert P.rel_l2(got["dq"][rows], dq) <= P.BF16_REL, P.rel_l2(got["dq"][rows], dq)
    assert P.rel_l2(got["du"][rows], du) <= P.BF16_REL, P.rel_l2(got["du"][rows], du)
    keys = _sample_rows(inp["seq_offsets"], rng, per_seq=4)
    dk, dv = sampled.attention_bwd_cols(*args, keys, **rest)
    assert P.rel_l2(got["dk"][keys], dk) <= P.BF16_REL, P.rel_l2(got["dk"][keys], dk)
    assert P.rel_l2(got["dv"][keys], dv) <= P.BF16_REL, P.rel_l2(got["dv"][keys], dv)


def test_efficiency_rab_gradients(efficiency):
    inp, got = efficiency
    lengths = np.diff(inp["seq_offsets"])
    assert inp["num_targets"] is None and int(lengths.max()) <= inp["max_len"]
    # diagonals near the main one (the largest entries), tile edges, and far ones
    deltas = np.array([0, -1, -2, -3, -31, -32, -63, -64, -65, -127, -128, -129, -500,
                       -2047, -4095, -4096, -6000, -8000])
    want = sampled.diagonal_ds_sums(inp["q"], inp["k"], inp["v"], inp["u"], inp["seq_offsets"],
                                    inp["max_len"], inp["d_o"], deltas, inp["timestamps"],
                                    inp["rab_pos"], inp["rab_time"])
    g = got["d_rab_pos"][0, deltas + inp["max_len"] - 1]
    assert P.rel_l2(g, want) <= P.BF16_REL, (P.rel_l2(g, want), g, want)
    # positive offsets are never read by causal pairs
    assert np.all(got["d_rab_pos"][0, inp["max_len"]:] == 0)
    # both tables hold the same total of dS
    tp, tt = float(np.sum(got["d_rab_pos"])), float(np.sum(got["d_rab_time"]))
    scale = float(np.sum(np.abs(got["d_rab_pos"])))
    assert abs(tp - tt) <= 1e-3 * scale, (tp, tt, scale)


def test_efficiency_rab_gradients_whole(efficiency, eff_rab_oracle):
    """Every entry of d_rab_pos (16383) and d_rab_time (128), element by element."""
    inp, got = efficiency
    wp, wt = eff_rab_oracle
    for key, want in (("d_rab_pos", wp), ("d_rab_time", wt)):
        e = P.rel_l2(got[key], want)
        assert e <= P.BF16_REL, (key, e)
    # entries no pair reads stay exactly zero (positive offsets: no candidates)
    assert np.all(got["d_rab_pos"][0, inp["max_len"]:] == 0)
    assert np.all(wp[0, inp["max_len"]:] == 0)


def test_efficiency_deterministic(eff_inputs, eff_rab_oracle):
    """The deterministic mode at full size: two runs bit for bit equal, the
    same parity, and the report says the fixed-order sums and the dS export ran."""
    import torch
    from hstu_pointwise_attention_amd import ops
    inp, dev = eff_inputs
    _, A = P.gpu_fwd(inp, dev)
    runs = []
    for _ in range(2):
        g = ops.attn_bwd(dev["q"], dev["k"], dev["v"], dev["u"], dev["seq_offsets"], inp["max_len"],
                         A, dev["d_o"], timestamps=dev["timestamps"], rab_pos=dev["rab_pos"],
                         rab_time=dev["rab_time"], deterministic=True, report=True)
        torch.cuda.synchronize()
        assert g["info"] == {"dq_from_ds": True, "rab_deterministic": True,
                             "ds_sequences": len(inp["lengths"])}, g["info"]
        runs.append({k: v.clone() for k, v in g.items() if k != "info"})
    for key in runs[0]:
        assert torch.equal(runs[0][key], runs[1][key]), key
    wp, wt = eff_rab_oracle
    assert P.rel_l2(P.host(runs[0]["d_rab_pos"]), wp) <= P.BF16_REL
    assert P.rel_l2(P.host(runs[0]["d_rab_time"]), wt) <= P.BF16_REL


def _edge_rows(L, rng):
    picks = {0, 1, 63, 64, 65, 127, 128, 129, 255, 256, 4095, 4096, L - 129, L - 128, L - 65,
             L - 64, L - 2, L - 1}
    picks |= set(int(x) for x in rng.integers(0, L, size=4))
    return sorted(i for i in picks if 0 <= i < L)


def test_efficiency_bucket_export_rows(eff_inputs):
    """hstu_rab_bucketize at full size, bit for bit, on rows at tile edges of
    every sequence (and random rows), each with all of its keys."""
    from hstu_pointwise_attention_amd import ops
    inp, dev = eff_inputs
    bp, bt = ops.rab_bucketize(dev["seq_offsets"], inp["max_len"], timestamps=dev["timestamps"],
                               n_time_buckets=inp["rab_time"].shape[1])
    offs = inp["seq_offsets"]
    ts = inp["timestamps"]
    rng = np.random.default_rng(12)
    base = 0
    n_rows = 0
    for b in range(len(offs) - 1):
        s, e = int(offs[b]), int(offs[b + 1])
        L = e - s
        for i in _edge_rows(L, rng):
            o = base + i * (i + 1) // 2
            cols = np.arange(i + 1)
            want_bp = oracle.position_buckets(np.array([i]), cols, L, inp["max_len"])[0]
            want_bt = oracle.time_buckets(ts[s + i:s + i + 1], ts[s:s + i + 1], inp["rab_time"].shape[1])[0]
            assert np.array_equal(bp[o:o + i + 1].cpu().numpy().astype(np.int64), want_bp), (b, i)
            assert np.array_equal(bt[o:o + i + 1].cpu().numpy().astype(np.int64), want_bt), (b, i)
            n_rows += 1
        base += L * (L + 1) // 2
    assert base == bp.numel() and n_rows > 8 * 16


@pytest.fixture(scope="module")
def layer():
    import torch
    from hstu_pointwise_attention_amd.attention import hstu_layer_fwd
    li = W.make_layer_inputs(W.MFALCON_LAYER)
    dev = "cuda"
    t = {k: torch.from_numpy(li[k]).to(dev, torch.bfloat16) for k in ("x", "w1", "w2")}
    t.update({k: torch.from_numpy(li[k]).to(dev) for k in ("b1", "b2", "seq_offsets", "num_targets")})
    y, a, uvqk = hstu_layer_fwd(t["x"], t["w1"], t["b1"], t["w2"], t["b2"], t["seq_offsets"],
                                t["num_targets"], li["heads"], li["head_dim"])
    torch.cuda.synchronize()
    print(f"layer workload: T={li['x'].shape[0]}", flush=True)
    return li, {"y": P.host(y), "a": P.host(a), "uvqk": P.host(uvqk)}


def test_layer_rows(layer):
    li, got = layer
    offs = li["seq_offsets"]
    rng = np.random.default_rng(9)
    # two users: history rows, the last history row, candidates
    rows = []
    for b in (0, 3):
        s = int(offs[b])
        hist = int(offs[b + 1] - offs[b]) - int(li["num_targets"][b])
        rows += [s, s + 1, s + 4095, s + hist - 1, s + hist, s + hist + 511,
                 int(offs[b + 1]) - 1] + [s + int(x) for x in rng.integers(0, hist, size=3)]
    rows = np.array(sorted(set(rows)), dtype=np.int64)
    want = layer_fwd_rows(li["x"], li["w1"], li["b1"], li["w2"], li["b2"], offs,
                          li["num_targets"], li["heads"], li["head_dim"], rows)
    for key in ("uvqk", "a", "y"):
        e = P.rel_l2(got[key][rows], want[key])
        assert e <= P.BF16_REL, (key, e)
    # the layer's output Y also under the bf16 output bar
    err = float(np.max(np.abs(got["y"][rows] - want["y"])))
    assert err <= P.BF16_O_MAXABS, ("Y max-abs", err)


@pytest.fixture(scope="module")
def layer_bwd():
    """The M-FALCON layer forward and backward through the C ABI, as bench.py
    times them, with a seeded dY (N(0, 1), bf16)."""
    import torch
    from hstu_pointwise_attention_amd.attention import hstu_layer_bwd, hstu_layer_fwd
    li = W.make_layer_inputs(W.MFALCON_LAYER)
    dy = W.round_to(np.random.default_rng(1009).standard_normal((li["x"].shape[0], li["w2"].shape[1])),
                    "bf16")
    dev = "cuda"
    t = {k: torch.from_numpy(li[k]).to(dev, torch.bfloat16) for k in ("x", "w1", "w2")}
    t.update({k: torch.from_numpy(li[k]).to(dev) for k in ("b1", "b2", "seq_offsets", "num_targets")})
    y, a, uvqk = hstu_layer_fwd(t["x"], t["w1"], t["b1"], t["w2"], t["b2"], t["seq_offsets"],
                                t["num_targets"], li["heads"], li["head_dim"])
    g = hstu_layer_bwd(t["x"], t["w1"], t["b1"], t["w2"], t["seq_offsets"], t["num_targets"],
                       li["heads"], li["head_dim"], uvqk, a,
                       torch.from_numpy(dy).to(dev, torch.bfloat16),
                       max_len=int(li["lengths"].max()))
    torch.cuda.synchronize()
    print(f"layer backward workload: T={li['x'].shape[0]}", flush=True)
    return li, dy, {k: P.host(v) for k, v in g.items()}


def test_layer_bwd_rows(layer_bwd):
    """Sampled rows of dX for user 1: the last history rows and candidates. For
    those keys, dK and dV involve only queries from 40 rows before the end of
    the history onwards, so the oracle needs A (and dA) for just those rows:
    oracle.attention_fwd_rows, the LayerNorm and gate backward, and the
    sampled attention gradients, chained as oracle.layer.layer_bwd does.
    db2 (a column sum of dY) is checked whole."""
    from oracle.layer import layernorm, layernorm_bwd, split_uvqk
    li, dy, got = layer_bwd
    H, D = li["heads"], li["head_dim"]
    HD = H * D
    offs, nt = li["seq_offsets"], li["num_targets"]
    b = 1
    s, e = int(offs[b]), int(offs[b + 1])
    L = e - s
    hist = L - int(nt[b])
    w1 = li["w1"].astype(np.float64)
    w2 = li["w2"].astype(np.float64)
    pre = li["x"][s:e].astype(np.float64) @ w1 + li["b1"].astype(np.float64)
    u, v, q, k = split_uvqk(oracle.silu(pre), H, D)
    one = np.array([0, L], np.int64)
    ntb = np.array([int(nt[b])], np.int64)
    rows = np.arange(hist - 40, L)
    _, A = oracle.attention_fwd_rows(q, k, v, None, one, L, rows, ntb)
    A2 = A.reshape(len(rows), HD)
    dz = dy[s:e][rows].astype(np.float64) @ w2.T
    du_rows = dz * layernorm(A2)
    dA = np.zeros((L, H, D))
    dA[rows] = layernorm_bwd(A2, dz * u.reshape(L, HD)[rows]).reshape(len(rows), H, D)
    pick = np.array([hist - 40, hist - 1, hist, hist + 511, L - 1], np.int64)
    dq, _ = sampled.attention_bwd_rows(q, k, v, None, one, L, dA, pick, ntb)
    dk, dv = sampled.attention_bwd_cols(q, k, v, None, one, L, dA, pick, ntb)
    n = len(pick)
    d_uvqk = np.concatenate([du_rows[pick - rows[0]], dv.reshape(n, HD), dq.reshape(n, HD),
                             dk.reshape(n, HD)], axis=1)
    z = pre[pick]
    sig = 1.0 / (1.0 + np.exp(-z))
    dx_want = (d_uvqk * sig * (1.0 + z * (1.0 - sig))) @ w1.T
    e_dx = P.rel_l2(got["dx"][s + pick], dx_want)
    assert e_dx <= P.BF16_REL, e_dx
    db2 = dy.astype(np.float64).sum(axis=0)
    assert P.rel_l2(got["db2"], db2) <= 1e-5


def test_layer_fp8_rows():
    """The FP8 layer forward at the M-FALCON shape on sampled rows of Y:
    quantisation is row-wise, so a row's UVQK, A and output codes follow from
    its own row and its sequence's keys and values (oracle.fp8 steps chained
    as oracle.fp8.layer_fwd_fp8 does); bar: one E4M3 rounding unit (2^-4) of
    rel-L2, as the small FP8 layer tests derive it."""
    import torch
    from oracle import fp8 as F8
    from oracle.layer import split_uvqk
    from hstu_pointwise_attention_amd.attention import hstu_layer_fwd_fp8, prepare_fp8_weights
    li = W.make_layer_inputs(W.MFALCON_LAYER)
    dev = "cuda"
    t = {k: torch.from_numpy(li[k]).to(dev, torch.bfloat16) for k in ("x", "w1", "w2")}
    t.update({k: torch.from_numpy(li[k]).to(dev) for k in ("b1", "b2", "seq_offsets", "num_targets")})
    fw = prepare_fp8_weights(t["w1"], t["w2"])
    y, _, _ = hstu_layer_fwd_fp8(t["x"], fw, t["b1"], t["b2"], t["seq_offsets"], t["num_targets"],
                                 li["heads"], li["head_dim"])
    torch.cuda.synchronize()
    y = P.host(y)
    H, D = li["heads"], li["head_dim"]
    offs, nt = li["seq_offsets"], li["num_targets"]
    b = 2
    s, e = int(offs[b]), int(offs[b + 1])
    L = e - s
    hist = L - int(nt[b])
    w1q, w1s = F8.quantize_weight(li["w1"])
    w2q, w2s = F8.quantize_weight(li["w2"])
    xq, xs = F8.quantize_rows(li["x"][s:e])
    uvqk = F8.fp8_linear(xq, xs, w1q, w1s, li["b1"], apply_silu=True)
    u, v, q, k = split_uvqk(uvqk, H, D)
    pick = np.array([0, 1, 4095, hist - 1, hist, hist + 700, L - 1], np.int64)
    _, A = oracle.attention_fwd_rows(q, k, v, None, np.array([0, L]), L, pick,
                                     np.array([int(nt[b])]))
    zq, zs = F8.layernorm_gate_fp8(A.reshape(len(pick), H * D), u.reshape(L, H * D)[pick])
    want = F8.fp8_addmm(zq, zs, w2q, w2s, li["b2"])
    e_y = P.rel_l2(y[s + pick], want)
    assert e_y <= 2.0 ** -4, e_y
