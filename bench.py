"""Benchmark: jagged HSTU attention forward + backward on one MI355X.

One step = the whole hot path over one batch of the efficiency workload
(8 jagged sequences, lengths uniform in [4096, 8192], 4 heads, head dim 128,
position + time rab with 16383 + 128 buckets, bf16): per-sequence prep,
scheduling, fused forward, backward preprocessing, fused backward and dQ
conversion, all through the C ABI on torch's current stream, inputs already
in HBM. Throughput is algorithmic TFLOP/s over unmasked pairs only
(forward 2*Dqk + 2*Dv, backward 6*Dqk + 4*Dv per pair and head).

Prints one JSON line. Also measures one HSTU layer forward and backward at
the M-FALCON shape and candidate scoring against a cached history, and times
the CPU oracle on a bounded sample as a reported baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HSTU jagged attn fwd+bwd TFLOP/s @ max_len 8192; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA, published
# HBM traffic of the dominant kernel per launch, from two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE) scaled by the copy-kernel calibration; the
# summaries are under profiles/. None when not measured for the kernel as it
# stands.
TRAFFIC = {
    # key-block backward (hstu_bwd_k16_kernel, D=128, efficiency workload):
    # FETCH_SIZE 393752 KiB x 2.00 + WRITE_SIZE 1088013 KiB x 1.00
    "bwd": {"workload": "efficiency_8192_bf16", "bytes": 1920529818,
            "compulsory_bytes": 1233000000, "unit": "B"},
}
# The pages' only figure for this path, quoted as context (not a target, not
# comparable: another machine, and neither its hardware nor its workload
# details are stated).
PAGES_CLAIM = ("HSTU-based generative recommenders run 5.3x to 15.2x faster than "
               "FlashAttention2-based Transformers on 8192-length sequences (Abstract of "
               "'Actions Speak Louder than Words'; hardware not stated)")


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-layer", action="store_true")
    ap.add_argument("--workload", default="efficiency_8192_bf16")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--cached-only", action="store_true",
                    help="only time candidate scoring against a cached history")
    ap.add_argument("--fp8-only", action="store_true",
                    help="only time the FP8 projection GEMMs")
    ap.add_argument("--layer-only", action="store_true",
                    help="only time one HSTU layer forward and backward at the M-FALCON shape")
    return ap.parse_args()


def copy_calibration(steps: int) -> None:
    """A plain device-to-device copy of known size: FETCH_SIZE / WRITE_SIZE of
    this kernel against its 256 MiB read + 256 MiB write calibrate the
    counters used for the traffic figures."""
    import torch
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(max(steps, 1)):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": max(steps, 1)}), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by sequence, see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.cached_only:
        from hstu_pointwise_attention_amd import _lib as _l
        _l.load()
        print(json.dumps({"cached_scoring": bench_cached(torch)}), flush=True)
        return

    import workloads as W
    from hstu_pointwise_attention_amd import _lib, ops
    from hstu_pointwise_attention_amd.attention import hstu_layer_bwd, hstu_layer_fwd

    if args.fp8_only:
        _lib.load()
        print(json.dumps({"fp8_linear": bench_fp8(torch)}), flush=True)
        return

    if args.layer_only:
        _lib.load()
        print(json.dumps({"layer_mfalcon": bench_layer(torch, W, hstu_layer_fwd, hstu_layer_bwd)}),
              flush=True)
        return
    from hstu_pointwise_attention_amd.flops import attention_flops

    _lib.load()
    wl = {w.name: w for w in W.ATTN_WORKLOADS}[args.workload]
    inp = W.make_attention_inputs(wl)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dev = "cuda"
    T = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev, dt) for k in ("q", "k", "v", "u", "d_o")}
    offs = torch.from_numpy(inp["seq_offsets"]).to(dev)
    ts = torch.from_numpy(inp["timestamps"]).to(dev)
    rp = torch.from_numpy(inp["rab_pos"]).to(dev) if inp["rab_pos"] is not None else None
    rt = torch.from_numpy(inp["rab_time"]).to(dev) if inp["rab_time"] is not None else None
    fl = attention_flops(inp["lengths"], wl.heads, wl.d_qk, wl.d_v)

    def step(report=False):
        o, a = ops.attn_fwd(T["q"], T["k"], T["v"], T["u"], offs, wl.max_len, timestamps=ts,
                            rab_pos=rp, rab_time=rt, save_a=True)
        g = ops.attn_bwd(T["q"], T["k"], T["v"], T["u"], offs, wl.max_len, a, T["d_o"],
                         timestamps=ts, rab_pos=rp, rab_time=rt, report=report)
        return o, g

    for _ in range(args.warmup):
        step()
    # which dQ path the backward takes on this batch (waits for the stream; untimed)
    info = step(report=True)[1]["info"]
    torch.cuda.synchronize()

    # Timed region: K steps on torch's current stream, nothing else recorded in it.
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps
    tflops = fl["total"] / (ms_step * 1e-3) / 1e12

    # Per-kernel times in a separate pass: the library's HIP events around each
    # of its launches, on the stream the kernels run on.
    with _lib.KernelTimer() as kt:
        for _ in range(min(args.steps, 20)):
            step()
        torch.cuda.synchronize()

    kern = {name: round(kt.avg_ms(name), 5) for name in kt.results}

    def kms(k):
        # the dQ pass is two launches: dQ from the exported dS tiles ("dq_ds")
        # and by recomputing dS ("dq") for sequences whose tiles did not fit
        # (it exits at once when every sequence exported)
        if k == "dq" and "dq_ds" in kt.results:
            return kt.avg_ms("dq") + kt.avg_ms("dq_ds")
        return kt.avg_ms(k)

    fwd_ms = kms("fwd")
    # the backward: dA' / dU preprocessing (one launch with the backward's
    # sequence prep), key-block kernel, dQ kernel
    bwd_ms = sum(kms(k) for k in ("bwd_pre", "bwd", "dq"))
    bwd_tf = fl["bwd"] / (bwd_ms * 1e-3) / 1e12
    fwd_tf = fl["fwd"] / (fwd_ms * 1e-3) / 1e12
    per_kernel = {k: {"ms": round(kms(k), 5), "algorithmic_flops": f,
                      "tflops": round(f / (kms(k) * 1e-3) / 1e12, 2)}
                  for k, f in fl["kernels"].items()}
    # the dominant attention kernel by time
    dom = max(fl["kernels"], key=lambda k: kms(k))
    dom_ms, dom_flops = kms(dom), fl["kernels"][dom]
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": (TRAFFIC[dom]["bytes"] if dom in TRAFFIC and TRAFFIC[dom]["workload"] == wl.name
                            else None),
                "flops_per_launch": dom_flops, "avg_launch_ms": round(dom_ms, 5)}

    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": wl.name, "batch": wl.batch, "heads": wl.heads,
                   "head_dim": wl.d_qk, "max_len": wl.max_len,
                   "lengths": f"{wl.length_kind} {list(wl.length_args)}, seed {wl.seed}",
                   "tokens": int(inp["seq_offsets"][-1]), "pair_heads": fl["pair_heads"],
                   "flops_per_step": fl["total"],
                   "rab": f"position {2 * wl.max_len - 1 if wl.use_pos_bias else 0} + time "
                          f"{wl.n_time_buckets} buckets"},
        "dq_path": ("dS export" if info["dq_from_ds"] else
                    "recompute dS" if info["ds_sequences"] == 0 else
                    f"dS export for the first {info['ds_sequences']} sequences, recompute dS for the rest"),
        "context": {"pages_claim": PAGES_CLAIM},
        "fwd_tflops": round(fwd_tf, 2), "bwd_tflops": round(bwd_tf, 2),
        "attention_kernels": per_kernel,
        "kernels_avg_ms": kern,
        "roofline": roofline,
    }

    out["bucketize"] = bench_bucketize(torch, _lib, ops, inp, wl, offs, ts)

    if not args.no_layer:
        out["layer_mfalcon"] = bench_layer(torch, W, hstu_layer_fwd, hstu_layer_bwd)
        out["cached_scoring"] = bench_cached(torch)
        out["fp8_linear"] = bench_fp8(torch)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, wl)

    print(json.dumps(out), flush=True)


def bench_bucketize(torch, _lib, ops, inp, wl, offs, ts, iters=10):
    """The standalone rab bucketiser (hstu_rab_bucketize) on the efficiency
    workload: position (uint16) and time (uint8) buckets of every unmasked
    pair, timed by the library's HIP events around its kernel. Algorithmic
    bytes: 3 written per pair plus the 8-byte timestamps read once."""
    from hstu_pointwise_attention_amd.flops import unmasked_pairs_host
    pairs = unmasked_pairs_host(inp["lengths"], None)
    run = lambda: ops.rab_bucketize(offs, wl.max_len, timestamps=ts, n_time_buckets=wl.n_time_buckets)
    run()
    torch.cuda.synchronize()
    with _lib.KernelTimer() as kt:
        for _ in range(iters):
            run()
        torch.cuda.synchronize()
    ms = kt.avg_ms("bucketize")
    nbytes = 3 * pairs + 8 * int(inp["seq_offsets"][-1])
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "pairs": int(pairs), "bytes": int(nbytes), "gb_per_s": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


def bench_layer(torch, W, hstu_layer_fwd, hstu_layer_bwd, iters=10):
    """One HSTU layer at the M-FALCON-style shape, 4 users x (8192 history + 1024
    candidates): the forward, then the backward from a seeded dY (the forward's
    UVQK and A reused, the projection pre-activation recomputed inside), then
    the forward with both projections in FP8 (weights prepared once, outside
    the timed loop; activation quantisation inside it)."""
    from hstu_pointwise_attention_amd.flops import unmasked_pairs_host
    w = W.MFALCON_LAYER
    li = W.make_layer_inputs(w)
    dev = "cuda"
    x = torch.from_numpy(li["x"]).to(dev, torch.bfloat16)
    w1 = torch.from_numpy(li["w1"]).to(dev, torch.bfloat16)
    w2 = torch.from_numpy(li["w2"]).to(dev, torch.bfloat16)
    b1 = torch.from_numpy(li["b1"]).to(dev)
    b2 = torch.from_numpy(li["b2"]).to(dev)
    offs = torch.from_numpy(li["seq_offsets"]).to(dev)
    nt = torch.from_numpy(li["num_targets"]).to(dev)
    for _ in range(3):
        hstu_layer_fwd(x, w1, b1, w2, b2, offs, nt, w.heads, w.head_dim)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        hstu_layer_fwd(x, w1, b1, w2, b2, offs, nt, w.heads, w.head_dim)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    T = x.shape[0]
    pairs = unmasked_pairs_host(li["lengths"], li["num_targets"]) * w.heads
    attn = pairs * 4 * w.head_dim
    gemm = 2 * T * w.model_dim * (4 * w.heads * w.head_dim) + 2 * T * (w.heads * w.head_dim) * w.model_dim
    y, a, uvqk = hstu_layer_fwd(x, w1, b1, w2, b2, offs, nt, w.heads, w.head_dim)
    g = torch.Generator(device=dev).manual_seed(1007)
    dy = torch.randn(y.shape, generator=g, device=dev).to(torch.bfloat16)
    for _ in range(2):
        hstu_layer_bwd(x, w1, b1, w2, offs, nt, w.heads, w.head_dim, uvqk, a, dy,
                       max_len=w.history + w.candidates)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(iters):
        hstu_layer_bwd(x, w1, b1, w2, offs, nt, w.heads, w.head_dim, uvqk, a, dy,
                       max_len=w.history + w.candidates)
    e1.record()
    torch.cuda.synchronize()
    ms_b = e0.elapsed_time(e1) / iters
    # backward: attention 6*Dqk + 4*Dv per pair and head; each projection's
    # dX and dW cost twice its forward (the pre-activation recompute is not counted)
    attn_b = pairs * 10 * w.head_dim
    gemm_b = 2 * gemm
    from hstu_pointwise_attention_amd.attention import hstu_layer_fwd_fp8, prepare_fp8_weights
    fw = prepare_fp8_weights(w1, w2)
    for _ in range(3):
        hstu_layer_fwd_fp8(x, fw, b1, b2, offs, nt, w.heads, w.head_dim)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(iters):
        hstu_layer_fwd_fp8(x, fw, b1, b2, offs, nt, w.heads, w.head_dim)
    e1.record()
    torch.cuda.synchronize()
    ms_8 = e0.elapsed_time(e1) / iters
    return {"ms": round(ms, 4), "tflops": round((attn + gemm) / (ms * 1e-3) / 1e12, 2),
            "attn_flops": attn, "gemm_flops": gemm, "tokens": T,
            "fp8_ms": round(ms_8, 4), "fp8_tflops": round((attn + gemm) / (ms_8 * 1e-3) / 1e12, 2),
            "bwd_ms": round(ms_b, 4), "bwd_tflops": round((attn_b + gemm_b) / (ms_b * 1e-3) / 1e12, 2),
            "bwd_attn_flops": attn_b, "bwd_gemm_flops": gemm_b}


def bench_cached(torch, users=4, hist=8192, n_cand=1024, micro=128, heads=4, d=128, iters=5):
    """Candidate scoring against a cached history (hstu_attn_fwd_cached) at the
    M-FALCON layer's attention shape: 4 users x 8192 history rows, 1024
    candidates each, scored in micro-batches of 128 per user; H 4, D 128,
    bf16, no bias or gate (the layer's attention). Seeded synthetic inputs."""
    from hstu_pointwise_attention_amd import ops
    dev = "cuda"
    g = torch.Generator(device=dev).manual_seed(1006)
    rnd = lambda *shape: (0.5 * torch.randn(*shape, generator=g, device=dev)).to(torch.bfloat16)
    k_hist, v_hist = rnd(users * hist, heads, d), rnd(users * hist, heads, d)
    hist_offsets = torch.arange(users + 1, device=dev, dtype=torch.int64) * hist
    cand_offsets = torch.arange(users + 1, device=dev, dtype=torch.int64) * micro
    n_cands = torch.full((users,), n_cand, device=dev, dtype=torch.int64)
    n_micro = n_cand // micro
    batches = [(rnd(users * micro, heads, d), rnd(users * micro, heads, d), rnd(users * micro, heads, d),
                torch.full((users,), mb * micro, device=dev, dtype=torch.int64)) for mb in range(n_micro)]

    def score_all():
        for q, k, v, first in batches:
            ops.attn_fwd_cached(q, k, v, None, cand_offsets, first, n_cands, k_hist, v_hist,
                                hist_offsets, hist + n_cand, save_a=False)

    score_all()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        score_all()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters                 # all candidates of all users
    pairs = users * heads * n_cand * (hist + 1)
    flops = pairs * 4 * d
    return {"ms_all_candidates": round(ms, 4), "ms_per_micro_batch": round(ms / n_micro, 4),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "candidates_per_s": round(users * n_cand / (ms * 1e-3)),
            "shape": f"{users} users x {hist} history rows, {n_cand} candidates in micro-batches "
                     f"of {micro}, H {heads}, D {d}, bf16, no bias",
            "pair_heads": pairs, "flops": flops}


def bench_fp8(torch, iters=20):
    """FP8 (E4M3) projection GEMMs with prepared weights: the README's FP8 addmm
    benchmark shape (m 4096, k 512, n 512) and the M-FALCON layer's two
    projections (36864 tokens, 512 -> 2048 with SiLU, 512 -> 512), each
    beside the bf16 GEMM of the same shape; the activation quantisation
    (row-wise, from bf16) is timed on its own. Seeded synthetic inputs."""
    from hstu_pointwise_attention_amd import ops
    dev = "cuda"
    g = torch.Generator(device=dev).manual_seed(1008)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    out = {}
    for name, (M, K, N, act) in {"m4096_k512_n512": (4096, 512, 512, False),
                                 "layer_uvqk_36864_512_2048": (36864, 512, 2048, True),
                                 "layer_out_36864_512_512": (36864, 512, 512, False)}.items():
        x = torch.randn(M, K, generator=g, device=dev).to(torch.bfloat16)
        w = (torch.randn(K, N, generator=g, device=dev) / K ** 0.5).to(torch.bfloat16)
        b = torch.randn(N, generator=g, device=dev)
        wq, ws = ops.fp8_prepare_weight(w)
        xq, xs = ops.fp8_quantize_rows(x)
        ms8 = timed(lambda: ops.fp8_linear(xq, xs, wq, ws, b, silu=act))
        msq = timed(lambda: ops.fp8_quantize_rows(x))
        ms16 = timed(lambda: ops.linear(x, w, b, silu=act))
        fl = 2 * M * K * N
        out[name] = {"fp8_gemm_ms": round(ms8, 4), "fp8_tflops": round(fl / (ms8 * 1e-3) / 1e12, 2),
                     "pct_of_fp8_peak": round(100 * fl / (ms8 * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 2),
                     "quantize_ms": round(msq, 4), "bf16_gemm_ms": round(ms16, 4),
                     "bf16_tflops": round(fl / (ms16 * 1e-3) / 1e12, 2), "flops": fl}
    return out


def cpu_baseline(inp, wl):
    """The oracle (numpy fp64) on a bounded sample: the first sequence of the batch, heads 0 and 1
    (about 10 s on 16 host threads)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    from hstu_pointwise_attention_amd.flops import attention_flops
    s, e = int(inp["seq_offsets"][0]), int(inp["seq_offsets"][1])
    sl = slice(s, e)
    nh = 2 if wl.rab_heads == 1 else 1                                    # heads 0 and 1
    sub = {k: inp[k][sl, :nh] for k in ("q", "k", "v", "u", "d_o")}
    sub["timestamps"] = inp["timestamps"][sl]
    offs = np.array([0, e - s])
    t0 = time.perf_counter()
    oracle.attention_bwd(sub["q"], sub["k"], sub["v"], sub["u"], offs, wl.max_len, sub["d_o"],
                         None, sub["timestamps"], inp["rab_pos"], inp["rab_time"])
    sec = time.perf_counter() - t0
    # attention_bwd evaluates the forward once inside; count fwd + bwd work
    f = attention_flops([e - s], nh, wl.d_qk, wl.d_v)
    return {"value": round(f["total"] / sec / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(sec, 2),
            "sample": f"sequence 0 of the batch (L={e - s}), {nh} head(s), fwd+bwd, fp64 numpy"}


if __name__ == "__main__":
    main()
