"""Checks that pin the oracle to facts other than itself.

Each ``pin_*`` takes an oracle-like namespace (``attention_fwd``,
``attention_bwd``, bucket functions) and raises AssertionError when the
implementation disagrees with a closed form, an invariant, a brute-force
evaluation, finite differences or autograd. ``tests/test_oracle_attention.py``
runs them on the oracle; ``tests/test_oracle_mutants.py`` plants plausible
mistakes in copies of the oracle's source and shows each one is caught.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from workloads import offsets_from_lengths

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers
def tiny_case(seed, lengths=(3, 5, 1, 6), H=2, D=3, Dv=None, max_len=4, nt_buckets=5,
              targets=None, rab_heads=1, gate=True, pos=True, std=0.7, rab_std=0.3):
    """Small float64 inputs with visible bias (rab std 0.3) for pins."""
    rng = np.random.default_rng(seed)
    Dv = D if Dv is None else Dv
    lengths = np.asarray(lengths, dtype=np.int64)
    offs = offsets_from_lengths(lengths)
    T = int(offs[-1])
    ts = np.sort(rng.integers(0, 40, size=T)).astype(np.int64)
    c = dict(
        q=std * rng.standard_normal((T, H, D)),
        k=std * rng.standard_normal((T, H, D)),
        v=std * rng.standard_normal((T, H, Dv)),
        u=std * rng.standard_normal((T, H, Dv)) if gate else None,
        seq_offsets=offs,
        max_len=max_len,
        num_targets=None if targets is None else np.asarray(targets, dtype=np.int64),
        timestamps=ts if nt_buckets else None,
        rab_pos=rab_std * rng.standard_normal((rab_heads, 2 * max_len - 1)) if pos else None,
        rab_time=rab_std * rng.standard_normal((rab_heads, nt_buckets)) if nt_buckets else None,
    )
    d_o = rng.standard_normal((T, H, Dv))
    return c, d_o


def fwd(o, c, **over):
    args = dict(c)
    args.update(over)
    return o.attention_fwd(args["q"], args["k"], args["v"], args["u"], args["seq_offsets"],
                           args["max_len"], args["num_targets"], args["timestamps"],
                           args["rab_pos"], args["rab_time"])


def bwd(o, c, d_o, **over):
    args = dict(c)
    args.update(over)
    return o.attention_bwd(args["q"], args["k"], args["v"], args["u"], args["seq_offsets"],
                           args["max_len"], d_o, args["num_targets"], args["timestamps"],
                           args["rab_pos"], args["rab_time"])


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(np.linalg.norm(b.ravel()), 1e-300)
    return np.linalg.norm((a - b).ravel()) / den


def _silu(x):
    return x / (1.0 + math.exp(-x))


# ----------------------------------------------------------------- bucket pins
def pin_time_bucket_values(o):
    cases = [(0, 0), (1, 1), (2, 1), (3, 2), (4, 2), (6, 2), (7, 3), (8, 3)]
    for k in range(2, 40):
        cases.append(((1 << k) - 1, k))
        cases.append(((1 << k) - 2, k - 1))
    for dt, want in cases:
        got = int(o.time_buckets(np.array([dt]), np.array([0]), 64)[0, 0])
        assert got == want, (dt, got, want)
        got = int(o.time_buckets(np.array([0]), np.array([dt]), 64)[0, 0])
        assert got == want, ("sign", dt, got, want)
    got = o.time_buckets(np.array([0]), np.array([10 ** 15]), 16)[0, 0]
    assert got == 15
    i64 = np.iinfo(np.int64)
    got = o.time_buckets(np.array([i64.max]), np.array([i64.min]), 128)[0, 0]
    assert got == 64, got  # |dt| + 1 = 2^64


def pin_time_bucket_bruteforce(o, seed=0):
    rng = np.random.default_rng(seed)
    for scale in (10, 1 << 20, 1 << 40, 1 << 62):
        a = rng.integers(-scale, scale, size=40, dtype=np.int64)
        b = rng.integers(-scale, scale, size=30, dtype=np.int64)
        for nb in (1, 7, 64, 128):
            got = o.time_buckets(a, b, nb)
            for r in range(len(a)):
                for c in range(len(b)):
                    want = min((abs(int(a[r]) - int(b[c])) + 1).bit_length() - 1, nb - 1)
                    assert got[r, c] == want


def pin_position_bucket_values(o):
    m = 50
    bp = o.position_buckets(np.arange(60), np.arange(60), hist=60, max_len=m)
    for i in range(60):
        assert bp[i, i] == m - 1
    assert bp[m - 1, 0] == 0
    assert bp[59, 0] == 0            # clamped below
    assert bp[0, 59] == 2 * m - 2    # clamped above
    assert bp[10, 3] == m - 1 - 7
    assert bp[3, 10] == m - 1 + 7
    # candidates (rows >= hist) all sit at position hist
    bp = o.position_buckets(np.array([5, 6, 7]), np.arange(8), hist=5, max_len=m)
    assert (bp[0] == bp[1]).all() and (bp[1] == bp[2]).all()
    assert bp[2, 4] == m - 2 and bp[2, 7] == m + 1


# ----------------------------------------------------------------- forward pins
def pin_scalar_bruteforce_fwd(o, scalar_fwd, seed=1):
    for kw in (dict(), dict(targets=[1, 2, 0, 3]), dict(rab_heads=2), dict(gate=False),
               dict(pos=False), dict(nt_buckets=0), dict(lengths=(0, 4, 0), D=2, Dv=3)):
        c, _ = tiny_case(seed, **kw)
        O, A = fwd(o, c)
        So, Sa = scalar_fwd(c["q"], c["k"], c["v"], c["u"], c["seq_offsets"], c["max_len"],
                            c["num_targets"], c["timestamps"], c["rab_pos"], c["rab_time"])
        assert rel(O, np.array(So).reshape(O.shape)) < 1e-12, kw
        assert rel(A, np.array(Sa).reshape(A.shape)) < 1e-12, kw


def pin_zero_query(o):
    c, _ = tiny_case(2, pos=False, nt_buckets=0)
    c["q"] = np.zeros_like(c["q"])
    O, A = fwd(o, c)
    assert np.all(O == 0.0) and np.all(A == 0.0)


def pin_zero_key_prefix_sum(o):
    """K = 0 and rab_pos = const: A_i = SiLU(c)/L * (prefix sum of V)_i."""
    cval = 0.37
    for targets in (None, [0, 2, 1, 3]):
        c, _ = tiny_case(3, nt_buckets=0, targets=targets)
        c["k"] = np.zeros_like(c["k"])
        c["rab_pos"] = np.full_like(c["rab_pos"], cval)
        _, A = fwd(o, c)
        offs = c["seq_offsets"]
        for b in range(len(offs) - 1):
            s, e = int(offs[b]), int(offs[b + 1])
            L = e - s
            if L == 0:
                continue
            hist = L - (0 if targets is None else targets[b])
            vb = c["v"][s:e]
            cs = np.cumsum(vb, axis=0)
            want = np.empty_like(vb)
            for i in range(L):
                if i < hist:
                    want[i] = cs[i]
                else:
                    want[i] = (cs[hist - 1] if hist > 0 else 0.0) + vb[i]
            want *= _silu(cval) / L
            assert rel(A[s:e], want) < 1e-13, (b, targets)


def pin_single_token(o):
    c, _ = tiny_case(4, lengths=(1,), H=1, D=4, max_len=6, nt_buckets=3)
    O, _ = fwd(o, c)
    s = float(c["q"][0, 0] @ c["k"][0, 0]) + c["rab_pos"][0, 5] + c["rab_time"][0, 0]
    want = _silu(s) * c["v"][0, 0] * c["u"][0, 0]
    assert rel(O[0, 0], want) < 1e-14


def pin_append_rescales(o):
    """Appending a token scales earlier rows of A by L/(L+1) (pins N = L)."""
    c, _ = tiny_case(5, lengths=(6,), max_len=8)
    c7, _ = tiny_case(5, lengths=(7,), max_len=8)
    for key in ("q", "k", "v", "u"):
        c7[key][:6] = c[key]
    c7["timestamps"][:6] = c["timestamps"]
    c7["timestamps"][6] = c["timestamps"][5] + 3
    c7["rab_pos"], c7["rab_time"] = c["rab_pos"], c["rab_time"]
    _, A6 = fwd(o, c)
    _, A7 = fwd(o, c7)
    assert rel(A7[:6], A6 * 6.0 / 7.0) < 1e-13


def pin_causality(o):
    c, _ = tiny_case(6, lengths=(9,), max_len=10)
    O, _ = fwd(o, c)
    for cut in (0, 3, 8):
        p = {key: c[key].copy() for key in ("q", "k", "v", "u")}
        p["k"][cut + 1:] = np.nan       # masked scores must be dropped by selection
        p["q"][cut + 1:] = 123.0
        p["v"][cut + 1:] = -7.0
        p["u"][cut + 1:] = 5.0
        O2, _ = fwd(o, c, **p)
        assert np.array_equal(O2[:cut + 1], O[:cut + 1]), cut
    # candidates do not see each other
    c, _ = tiny_case(7, lengths=(9,), max_len=10, targets=[4])
    O, _ = fwd(o, c)
    p = {key: c[key].copy() for key in ("k", "v")}
    p["k"][6] = 9.0
    p["v"][6] = 9.0
    O2, _ = fwd(o, c, **p)
    rows = [0, 1, 2, 3, 4, 5, 7, 8]
    assert np.array_equal(O2[rows], O[rows])
    assert not np.array_equal(O2[6], O[6])


def pin_batch_order(o):
    c, _ = tiny_case(8, lengths=(3, 5, 1, 6))
    O, _ = fwd(o, c)
    offs = c["seq_offsets"]
    perm = [2, 0, 3, 1]
    lens = np.diff(offs)
    idx = np.concatenate([np.arange(offs[b], offs[b + 1]) for b in perm])
    p = {key: (c[key][idx] if c[key] is not None else None)
         for key in ("q", "k", "v", "u", "timestamps")}
    p["seq_offsets"] = offsets_from_lengths(lens[perm])
    O2, _ = fwd(o, c, **p)
    assert np.array_equal(O2, O[idx])
    # one sequence alone
    b = 3
    sl = slice(int(offs[b]), int(offs[b + 1]))
    alone = {key: (c[key][sl] if c[key] is not None else None)
             for key in ("q", "k", "v", "u", "timestamps")}
    alone["seq_offsets"] = np.array([0, lens[b]])
    O3, _ = fwd(o, c, **alone)
    assert np.array_equal(O3, O[sl])


def pin_linearity(o):
    c, _ = tiny_case(9)
    rng = np.random.default_rng(99)
    v2 = rng.standard_normal(c["v"].shape)
    _, A1 = fwd(o, c)
    _, A2 = fwd(o, c, v=v2)
    _, A12 = fwd(o, c, v=c["v"] + 2.0 * v2)
    assert rel(A12, A1 + 2.0 * A2) < 1e-12
    O1, _ = fwd(o, c)
    O3, _ = fwd(o, c, u=3.0 * c["u"])
    assert rel(O3, 3.0 * O1) < 1e-14


def pin_worked_example(o):
    """Hand-derived example in ``tests/golden/worked_example.json``."""
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    env = {"ln3": math.log(3.0), "ln7": math.log(7.0)}

    def ev(x):
        if isinstance(x, list):
            return [ev(e) for e in x]
        return float(eval(x, {"__builtins__": {}}, env)) if isinstance(x, str) else float(x)

    inp = {k: (np.array(ev(v)) if v is not None else None) for k, v in g["inputs"].items()}
    c = dict(q=inp["q"], k=inp["k"], v=inp["v"], u=inp["u"],
             seq_offsets=np.array(g["inputs"]["seq_offsets"], dtype=np.int64),
             max_len=int(g["max_len"]), num_targets=None,
             timestamps=np.array(g["inputs"]["timestamps"], dtype=np.int64),
             rab_pos=inp["rab_pos"], rab_time=inp["rab_time"])
    O, A = fwd(o, c)
    exp = g["expected"]
    assert rel(A, np.array(ev(exp["a"])).reshape(A.shape)) < 1e-14
    assert rel(O, np.array(ev(exp["o"])).reshape(O.shape)) < 1e-14
    G = bwd(o, c, np.array(ev(g["inputs"]["d_o"])))
    for key in ("dq", "dk", "dv", "du", "d_rab_pos", "d_rab_time"):
        want = np.array(ev(exp[key])).reshape(G[key].shape)
        assert np.max(np.abs(G[key] - want)) < 1e-14, key


# ----------------------------------------------------------------- backward pins
def _loss(o, c, d_o):
    O, _ = fwd(o, c)
    return float(np.sum(O * d_o))


def pin_finite_differences(o, seed=10, n_probe=6, h=1e-6):
    for kw in (dict(), dict(targets=[1, 2, 0, 2]), dict(rab_heads=2, gate=False)):
        c, d_o = tiny_case(seed, **kw)
        G = bwd(o, c, d_o)
        rng = np.random.default_rng(seed + 1)
        names = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("u", "du"),
                 ("rab_pos", "d_rab_pos"), ("rab_time", "d_rab_time")]
        for key, gkey in names:
            if c[key] is None:
                continue
            flat = c[key].reshape(-1)
            gflat = G[gkey].reshape(-1)
            idx = rng.choice(flat.size, size=min(n_probe, flat.size), replace=False)
            if key in ("rab_pos", "rab_time"):
                idx = np.union1d(idx, np.nonzero(gflat)[0][:n_probe])
            for t in idx:
                x0 = flat[t]
                flat[t] = x0 + h
                lp = _loss(o, c, d_o)
                flat[t] = x0 - h
                lm = _loss(o, c, d_o)
                flat[t] = x0
                fd = (lp - lm) / (2 * h)
                assert abs(fd - gflat[t]) <= 1e-6 * max(1.0, abs(fd)), (kw, key, t, fd, gflat[t])


def _torch_dense_loss(torch, c, d_o, tensors):
    """Independent dense formulation: full LxL masks per sequence, autograd backward."""
    q, k, v, u, rp, rt = tensors
    offs = c["seq_offsets"]
    H = q.shape[1]
    m_len = c["max_len"]
    total = torch.zeros((), dtype=torch.float64)
    for b in range(len(offs) - 1):
        s, e = int(offs[b]), int(offs[b + 1])
        L = e - s
        if L == 0:
            continue
        hist = L - (0 if c["num_targets"] is None else int(c["num_targets"][b]))
        ii = torch.arange(L)[:, None]
        jj = torch.arange(L)[None, :]
        allowed = ((jj <= ii) & (jj < hist)) | (jj == ii)
        pos = torch.where(ii < hist, ii, torch.full_like(ii, hist))
        bp = torch.clamp(jj - pos, -(m_len - 1), m_len - 1) + (m_len - 1)
        if rt is not None:
            ts = [int(t) for t in c["timestamps"][s:e]]
            bt = torch.tensor([[min((abs(a - bb) + 1).bit_length() - 1, rt.shape[1] - 1)
                                for bb in ts] for a in ts])
        for h in range(H):
            hr = 0 if (rp if rp is not None else rt) is None or \
                (rp if rp is not None else rt).shape[0] == 1 else h
            S = q[s:e, h] @ k[s:e, h].T
            if rp is not None:
                S = S + rp[hr][bp]
            if rt is not None:
                S = S + rt[hr][bt]
            P = torch.where(allowed, torch.nn.functional.silu(S), torch.zeros_like(S)) / L
            A = P @ v[s:e, h]
            Ob = A * u[s:e, h] if u is not None else A
            total = total + (Ob * torch.from_numpy(d_o[s:e, h])).sum()
    return total


def pin_torch_autograd(o, seed=11):
    import torch
    for kw in (dict(), dict(targets=[2, 1, 0, 4], rab_heads=2)):
        c, d_o = tiny_case(seed, **kw)
        keys = ("q", "k", "v", "u", "rab_pos", "rab_time")
        ts = [torch.tensor(c[key], dtype=torch.float64, requires_grad=True)
              if c[key] is not None else None for key in keys]
        loss = _torch_dense_loss(torch, c, d_o, ts)
        loss.backward()
        G = bwd(o, c, d_o)
        for key, gkey, t in zip(keys, ("dq", "dk", "dv", "du", "d_rab_pos", "d_rab_time"), ts):
            if t is None:
                continue
            assert rel(G[gkey], t.grad.numpy()) < 1e-12, (kw, gkey)
        O, _ = fwd(o, c)
        lv = float(loss.detach())
        assert abs(float(np.sum(O * d_o)) - lv) <= 1e-12 * max(1.0, abs(lv))


def pin_zero_query_grads(o):
    """Q = 0, no bias: dV = 0 exactly and dQ_i = dA_i^T (sum_{j<=i} V_j K_j^T) / (2L)."""
    c, d_o = tiny_case(12, pos=False, nt_buckets=0)
    c["q"] = np.zeros_like(c["q"])
    G = bwd(o, c, d_o)
    assert np.all(G["dv"] == 0.0)
    offs = c["seq_offsets"]
    dA = d_o * c["u"]
    for b in range(len(offs) - 1):
        s, e = int(offs[b]), int(offs[b + 1])
        L = e - s
        if L == 0:
            continue
        for h in range(c["q"].shape[1]):
            outer = np.einsum("jv,jk->jvk", c["v"][s:e, h], c["k"][s:e, h])
            M = np.cumsum(outer, axis=0)                 # prefix sums of V_j K_j^T
            want = np.einsum("iv,ivk->ik", dA[s:e, h], M) / (2.0 * L)
            assert rel(G["dq"][s:e, h], want) < 1e-12


def pin_scalar_bruteforce_bwd(o, scalar_bwd, seed=13):
    for kw in (dict(), dict(targets=[1, 0, 0, 2], rab_heads=2), dict(gate=False, pos=False)):
        c, d_o = tiny_case(seed, **kw)
        G = bwd(o, c, d_o)
        S = scalar_bwd(c["q"], c["k"], c["v"], c["u"], c["seq_offsets"], c["max_len"], d_o,
                       c["num_targets"], c["timestamps"], c["rab_pos"], c["rab_time"])
        for key in G:
            if G[key] is None:
                assert S[key] is None
                continue
            assert rel(G[key], np.array(S[key]).reshape(G[key].shape)) < 1e-12, (kw, key)


FWD_PINS = [pin_zero_query, pin_zero_key_prefix_sum, pin_single_token, pin_append_rescales,
            pin_causality, pin_batch_order, pin_linearity, pin_worked_example]
BWD_PINS = [pin_finite_differences, pin_torch_autograd, pin_zero_query_grads]
BUCKET_PINS = [pin_time_bucket_values, pin_time_bucket_bruteforce, pin_position_bucket_values]
