"""Parity of the HIP path (through the C ABI) with the CPU oracle. Needs a gfx950 GPU."""
import ctypes
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


def test_bucketize_long_rows_mixed():
    """Rows longer than a wave's 64 slots and shorter ones in one batch:
    position buckets clamped (max_len well below the lengths), unsorted
    timestamps, a sequence whose span needs 64-bit arithmetic in the middle
    of long rows, candidates, and empty sequences."""
    rng = np.random.default_rng(11)
    lengths = np.array([300, 0, 517, 64, 1, 260])
    offs = W.offsets_from_lengths(lengths)
    T = int(offs[-1])
    ts = rng.integers(-10 ** 8, 10 ** 8, size=T).astype(np.int64)      # unsorted, spans < 2^31
    s3 = int(offs[2])
    ts[s3 + 200:s3 + 240] += np.int64(3) << 33                          # |dt| > 2^31 for some pairs
    ts[int(offs[5]) + 17] = np.iinfo(np.int64).min                      # extreme value in a long row
    for max_len, nt in ((50, [5, 0, 40, 0, 1, 100]), (1024, [0, 0, 0, 64, 0, 0])):
        inp = dict(seq_offsets=offs, num_targets=np.array(nt), timestamps=ts, max_len=max_len,
                   dtype="fp32")
        for nb in (9, 128):
            _bucket_case(inp, nb)


def test_bucketize_differences_at_2_pow_31():
    """Key-timestamp differences of exactly +-(2^31 - 1), +-2^31 and
    +-(2^31 + 1) inside rows long enough for whole 512-slot steps of one row,
    where the export first computes buckets from 32-bit differences (buckets
    30, 31 and 31 before the clamp at 64 buckets)."""
    L = 1500
    offs = W.offsets_from_lengths(np.array([L, L]))
    base = np.int64(1) << 40
    ts = np.full(2 * L, base, dtype=np.int64)
    rng = np.random.default_rng(13)
    for s in (0, L):
        for d in (2 ** 31 - 1, 2 ** 31, 2 ** 31 + 1):
            for sign in (1, -1):
                idx = s + rng.integers(0, L, size=40)
                ts[idx] = base + sign * d
    inp = dict(seq_offsets=offs, num_targets=np.array([0, 100]), timestamps=ts, max_len=2048, dtype="fp32")
    _bucket_case(inp, 64)


def test_bucketize_many_sequences():
    """More sequences than the kernel stages in LDS (its search then reads
    pair_offsets from memory)."""
    rng = np.random.default_rng(12)
    lengths = rng.integers(0, 40, size=2600)
    offs = W.offsets_from_lengths(lengths)
    T = int(offs[-1])
    inp = dict(seq_offsets=offs, num_targets=np.minimum(rng.integers(0, 5, size=lengths.size), lengths),
               timestamps=np.cumsum(rng.integers(0, 5000, size=T)).astype(np.int64), max_len=40,
               dtype="fp32")
    _bucket_case(inp, 16)


def test_bucketize_unaligned_outputs():
    """Outputs that start off a 16-byte boundary give the same buckets,
    written only inside their ranges."""
    import torch
    from hstu_pointwise_attention_amd import _lib, ops
    inp = W.make_attention_inputs(W.LONG)
    dev = P.to_dev(inp)
    nb = W.LONG.n_time_buckets
    bp_ref, bt_ref = ops.rab_bucketize(dev["seq_offsets"], inp["max_len"], num_targets=dev["num_targets"],
                                       timestamps=dev["timestamps"], n_time_buckets=nb)
    n = bp_ref.numel()

    def vp(t, byte_shift=0):
        return ctypes.c_void_p(None if t is None else t.data_ptr() + byte_shift)

    lib = _lib.load()
    d = _lib.AttnDesc()
    d.batch = inp["seq_offsets"].size - 1
    d.heads = 1
    d.max_len = int(inp["max_len"])
    d.n_time_buckets = nb
    po = torch.empty(d.batch + 1, dtype=torch.int64, device="cuda")
    _lib.check(lib.hstu_rab_pair_offsets(ctypes.byref(d), vp(dev["seq_offsets"]), vp(dev["num_targets"]),
                                         vp(po), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
    for shift in (1, 3):
        bp = torch.full((n + 8,), 0x5A5A, dtype=torch.int16, device="cuda")
        bt = torch.full((n + 8,), 0xA5, dtype=torch.uint8, device="cuda")
        _lib.check(lib.hstu_rab_bucketize(ctypes.byref(d), vp(dev["seq_offsets"]), vp(dev["num_targets"]),
                                          vp(dev["timestamps"]), vp(po), vp(bp, 2 * shift), vp(bt, shift),
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
        torch.cuda.synchronize()
        assert torch.equal(bp[shift:shift + n].view(torch.uint16), bp_ref)
        assert torch.equal(bt[shift:shift + n], bt_ref)
        assert bool((bp[:shift] == 0x5A5A).all()) and bool((bp[shift + n:] == 0x5A5A).all())
        assert bool((bt[:shift] == 0xA5).all()) and bool((bt[shift + n:] == 0xA5).all())


def test_pair_offsets_match_oracle():
    """hstu_rab_pair_offsets: exclusive sums of each sequence's unmasked pairs
    (counted on the oracle's mask), with empty sequences, candidates, and more
    sequences than one workgroup's chunk."""
    import torch
    from hstu_pointwise_attention_amd import _lib, ops
    from oracle.attention import _mask
    rng = np.random.default_rng(21)
    for B in (0, 1, 7, 1500):
        L = rng.integers(0, 60, size=B)
        nt = np.minimum(rng.integers(0, 12, size=B), L)
        offs = np.concatenate([[0], np.cumsum(L)]).astype(np.int64)
        d = _lib.AttnDesc()
        d.batch = B
        po = torch.empty(B + 1, dtype=torch.int64, device="cuda")
        for targets in (None, nt):
            t = None if targets is None else torch.from_numpy(targets.astype(np.int64)).cuda()
            _lib.check(_lib.load().hstu_rab_pair_offsets(
                ctypes.byref(d), ops._ptr(torch.from_numpy(offs).cuda()), ops._ptr(t), ops._ptr(po),
                ops._stream()))
            got = po.cpu().numpy()
            counts = [int(_mask(np.arange(L[b]), int(L[b]), int(L[b] - (0 if targets is None else targets[b]))).sum())
                      for b in range(B)]
            want = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
            assert np.array_equal(got, want), (B, targets is None)


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


@pytest.mark.parametrize("pos,time", [(True, True), (False, False)])
def test_fp32_head_dim_128(pos, time):
    """fp32 at head dim 128 (one wave per SIMD in its tile kernels): several
    query and key blocks, a ragged last block, candidates, an empty and a
    one-row sequence, within the fp32 tolerance of the oracle."""
    lengths = (300, 0, 1, 129, 257)
    w = W.AttnWorkload("fp32d128", 61, len(lengths), 2, 128, 128, 320, 64 if time else 0, pos,
                       "fp32", "fixed", lengths)
    inp = W.make_attention_inputs(w)
    inp["num_targets"] = np.array([30, 0, 1, 0, 7], np.int64)
    _run_parity(inp, tag=f"fp32 D128 pos={pos} time={time}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("seed", range(6))
def test_random_small_sweep(dtype, seed):
    """Random small shapes over tile edges: lengths 0..300, H, D, rab and targets varied."""
    rng = np.random.default_rng(1000 + seed)
    H = int(rng.choice([1, 2, 4]))
    D = int(rng.choice([32, 64, 128]))
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
    D = 128
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
    tiles for the leading sequences whose tiles fit the room the workspace
    holds, and by recomputing dS for the others. Without a position bias
    max_len changes nothing else, so the same inputs run three ways: lengths
    300, 200, 77 with H 2 hold 2 * 9 + 2 * 6 + 2 * 2 = 34 tiles; max_len 512
    sizes room for 2 * 5 * 7 = 70 (every sequence exports), max_len 64 for
    2 * 2 * 7 = 28 (the first sequence's 18 tiles fit, the second's would end
    at 30: one sequence exports, two recompute), and the minimum workspace
    has no room (all recompute). The report names the split each time; all
    match the oracle and each other."""
    lengths = (300, 200, 77)
    w = W.AttnWorkload("dqpaths", 41, 3, 2, 64, 64, 512, 16, False, "bf16", "fixed", lengths)
    inp = W.make_attention_inputs(w)
    inp["num_targets"] = np.array([20, 0, 5], np.int64)
    want = P.oracle_bwd(inp)
    got = {}
    for name, max_len, room, n_ds in (("export", 512, True, 3), ("partial fit", 64, True, 1),
                                      ("min workspace", 512, False, 0)):
        run = dict(inp, max_len=max_len)
        _, A = P.gpu_fwd(run)
        got[name] = P.gpu_bwd(run, A, ds_room=room, report=True)
        info = got[name]["info"]
        assert info["ds_sequences"] == n_ds and info["dq_from_ds"] is (n_ds == 3), (name, info)
        P.check_bwd(run, got[name], want, name)
    for name in ("partial fit", "min workspace"):
        assert P.rel_l2(P.host(got["export"]["dq"]), P.host(got[name]["dq"])) <= P.BF16_REL


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_many_short_sequences(dtype):
    """6000 sequences of 0 to 9 rows (empty ones included) with candidates and
    both bias tables: the schedule's arrays (B + 1 + 4 (T / 128 + 2) ints)
    no longer fit its LDS and go through the workspace scratch, and the first
    launch of each call holds 6000 prep workgroups beside the schedule (and,
    in the backward, the dA' / dU pass)."""
    rng = np.random.default_rng(81)
    lengths = tuple(int(x) for x in rng.integers(0, 10, size=6000))
    w = W.AttnWorkload("many", 82, len(lengths), 2, 32, 32, 16, 16, True, dtype, "fixed", lengths)
    inp = W.make_attention_inputs(w)
    inp["num_targets"] = np.minimum(rng.integers(0, 3, size=len(lengths)), np.array(lengths)).astype(np.int64)
    _run_parity(inp, tag=f"many short {dtype}")


def test_bf16_partial_export_multiblock():
    """Sequences far longer than max_len (positions clamp) overflow the dS
    room sized from max_len after the first ones: the leading sequences take
    dQ from their exported tiles and the rest recompute it, over many key
    and query blocks, with both bias tables and candidate rows; the report
    counts the split and every gradient matches the oracle."""
    lengths = (1500, 1100, 1800, 900, 1300, 1700)
    w = W.AttnWorkload("partial", 71, len(lengths), 2, 64, 64, 512, 128, True, "bf16", "fixed", lengths)
    inp = W.make_attention_inputs(w)
    inp["num_targets"] = np.array([0, 40, 0, 0, 100, 0], np.int64)
    _, A = P.gpu_fwd(inp)
    got = P.gpu_bwd(inp, A, report=True)
    n_ds = got["info"]["ds_sequences"]
    assert 0 < n_ds < len(lengths) and not got["info"]["dq_from_ds"], got["info"]
    P.check_bwd(inp, got, P.oracle_bwd(inp), f"partial export ({n_ds} of {len(lengths)} sequences)")


@pytest.mark.parametrize("D", [32, 64, 128])
def test_bf16_ds_export_head_dims(D):
    """The dQ pass over exported dS tiles at every bf16 head dim: several key
    blocks per sequence (513 rows: five), candidate rows in every key-block
    position (a block of history keys, one straddling the history's end, and
    blocks of candidates only), and a length of one tile plus one row."""
    lengths = (513, 0, 1, 129, 300, 64)
    w = W.AttnWorkload("dsdims", 61, len(lengths), 2, D, D, 600, 128, True, "bf16", "fixed", lengths)
    inp = W.make_attention_inputs(w)
    inp["num_targets"] = np.array([100, 0, 1, 5, 200, 64], np.int64)
    O, A = P.gpu_fwd(inp)
    want_O, want_A = P.oracle_fwd(inp)
    P.check_fwd(inp, P.host(O), P.host(A), want_O, want_A, f"D{D}")
    got = P.gpu_bwd(inp, A, report=True)
    assert got["info"]["dq_from_ds"] is True, got["info"]
    P.check_bwd(inp, got, P.oracle_bwd(inp), f"D{D}")


def _det_case(name):
    if name == "tiny_fp32":
        return W.make_attention_inputs(W.TINY)
    if name in ("public", "long"):
        return W.make_attention_inputs(W.PUBLIC if name == "public" else W.LONG)
    # candidates with both tables (the position window path), 64-bit timestamps
    # in every other sequence, per-head tables, fp32 and bf16
    dtype = "fp32" if name.endswith("fp32") else "bf16"
    D = 128
    lengths = (130, 0, 70, 200, 1, 65)
    w = W.AttnWorkload("det", 51, len(lengths), 2, D, D, 160, 64, True, dtype, "fixed", lengths,
                       rab_heads=2)
    inp = W.make_attention_inputs(w)
    inp["num_targets"] = np.array([40, 0, 3, 70, 1, 0], np.int64)
    inp["timestamps"] = _timestamps("mixed", inp["seq_offsets"], np.random.default_rng(5)).astype(np.int64)
    return inp


@pytest.mark.parametrize("name", ["tiny_fp32", "public", "long", "cand_fp32", "cand_bf16"])
def test_deterministic_rab_repeatable(name):
    """desc.deterministic: the rab gradients (and every other output) repeat bit
    for bit over three runs, match the oracle, and the report says so."""
    import torch
    inp = _det_case(name)
    dev = P.to_dev(inp)
    _, A = P.gpu_fwd(inp, dev)
    runs = []
    for _ in range(3):
        g = P.gpu_bwd(inp, A, dev, deterministic=True, report=True)
        torch.cuda.synchronize()
        assert g["info"]["rab_deterministic"], g["info"]
        # the preferred workspace holds the dS room in this mode too (bf16)
        assert g["info"]["dq_from_ds"] == (inp["dtype"] == "bf16"), g["info"]
        runs.append(g)
    for key in ("dq", "dk", "dv", "du", "d_rab_pos", "d_rab_time"):
        if runs[0][key] is None:
            continue
        for r in runs[1:]:
            assert torch.equal(runs[0][key], r[key]), (name, key)
    P.check_bwd(inp, runs[0], P.oracle_bwd(inp), name)
