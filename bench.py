"""Benchmark of the whitened truncated decomposition path on one MI355X.

One step = the whole path over one calibration batch of the attention-projection
workload: 65536 bf16 tokens x 4096 channels streamed into the activation covariance
(SYRK on MFMA), Cholesky, whitening, fp64 Gram + eigensolve, back-map to rank 1024,
per-component K-FAC scores (this workload has no gradients) and the global
sort-and-truncate at the budget of rank 1024.  Inputs are resident in HBM before the
timed region.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "calib tokens/s into cov (4096-d) + whitened-SVD layers/s at 4096×4096, r=1024"
HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3, "f64": 78.6}

# roofline class of each instrumented kernel: MFMA contractions against the dense peak of
# their input type, the fp64 Jacobi kernels against the fp64 peak (vector and matrix fp64
# peaks are equal on MI355X), streaming passes against HBM
ROOFLINE = {
    "syrk_bf16_kernel": {"bound": "mfma", "dtype": "bf16", "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s"},
    "syrk_f32_kernel": {"bound": "mfma", "dtype": "f32", "peak": PEAK_TFLOPS["f32"], "unit": "TFLOP/s"},
    "gemm_f32_kernel": {"bound": "mfma", "dtype": "f32", "peak": PEAK_TFLOPS["f32"], "unit": "TFLOP/s"},
    "gram_f64_kernel": {"bound": "alu", "dtype": "f64", "peak": PEAK_TFLOPS["f64"], "unit": "TFLOP/s"},
    "jacobi_pairs_v_kernel": {"bound": "alu", "dtype": "f64", "peak": PEAK_TFLOPS["f64"], "unit": "TFLOP/s"},
    "jacobi_apply_c_kernel": {"bound": "mfma", "dtype": "f64", "peak": PEAK_TFLOPS["f64"], "unit": "TFLOP/s"},
    "fisher_partial_kernel": {"bound": "alu", "dtype": "f32", "peak": PEAK_TFLOPS["f32"], "unit": "TFLOP/s"},
    "fisher_mfma_kernel": {"bound": "mfma", "dtype": "bf16", "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s"},
    "qaw_prepass_kernel": {"bound": "hbm", "dtype": "bf16", "peak": HBM_PEAK_GBS, "unit": "GB/s"},
    "tri_symv_kernel": {"bound": "hbm", "dtype": "f64", "peak": HBM_PEAK_GBS, "unit": "GB/s"},
    "tri_w_kernel": {"bound": "hbm", "dtype": "f64", "peak": HBM_PEAK_GBS, "unit": "GB/s"},
    "tri_fused_kernel": {"bound": "hbm", "dtype": "f64", "peak": HBM_PEAK_GBS, "unit": "GB/s"},
    "tri_syr2k_kernel": {"bound": "alu", "dtype": "f64", "peak": PEAK_TFLOPS["f64"], "unit": "TFLOP/s"},
    "bt_vtz_kernel": {"bound": "alu", "dtype": "f64", "peak": PEAK_TFLOPS["f64"], "unit": "TFLOP/s"},
    "bt_update_kernel": {"bound": "alu", "dtype": "f64", "peak": PEAK_TFLOPS["f64"], "unit": "TFLOP/s"},
}

# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE on this
# workload, scaled by the copy-kernel calibration (profiles/counters_tri_symv_attnproj_4096.md:
# fetch 24.43 MB + write 0.77 MB, the average over the 3968 launches of a 4096-wide
# tridiagonalisation); absent (None) for a kernel whose counters were not taken
TRAFFIC = {"tri_symv_kernel": 25.20e6}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--tokens", type=int, default=65536)
    p.add_argument("--d", type=int, default=4096)
    p.add_argument("--rank", type=int, default=1024)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true", help="skip the scoring / allocation measurements")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="before the steps, run a plain elementwise copy (neg) of this many MiB three times: "
                        "the known-size kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    return p.parse_args()


def cpu_baseline(d, n, rank):
    """The fp64 oracle on host cores, on a bounded sample of the same workload: the
    covariance of 16384 of the n tokens (scaled by n / 16384), then the full-size
    Cholesky, whitening, SVD, back-map, K-FAC scores and allocation of the layer."""
    import numpy as np
    import torch

    import oracle
    import synth

    try:
        from threadpoolctl import threadpool_info
        threads = max(int(i.get("num_threads", 1)) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:
        threads = len(os.sched_getaffinity(0))
    ns = min(16384, n)
    a = synth.activation_stream(ns, d, 1.0, 31, outlier_frac=0.01, dtype=torch.bfloat16).float().numpy()
    t0 = time.perf_counter()
    xs = oracle.covariance_sum(a)
    t_cov_meas = time.perf_counter() - t0
    del a
    w = synth.weight(d, d, 35).numpy()
    t0 = time.perf_counter()
    res = oracle.whiten_decompose(w, xs, ns, rank=rank)
    sc = oracle.kfac_scores(res["sigma"])
    oracle.allocate([sc.astype(np.float32)], [2 * d], rank * 2 * d)
    t_dec = time.perf_counter() - t0
    t_cov = t_cov_meas * (n / ns)
    return {"value": 1.0 / (t_cov + t_dec), "unit": "layers/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 covariance of {ns} of {n} tokens (time x{n / ns:g}) + full {d}x{d} "
                      f"Cholesky/whitening/SVD/back-map/K-FAC scores/allocation at rank {rank}",
            "cov_tokens_per_s": round(n / t_cov, 1), "seconds_measured": round(t_cov_meas + t_dec, 2)}


def _time(fn, torch, reps):
    """median wall time of fn() over reps runs, each bracketed by device synchronisation"""
    ts = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        ts.append(time.perf_counter() - t0)
    return sorted(ts)[len(ts) // 2]


def secondary(lrc, torch, dev):
    """Throughput of the scoring and allocation passes at the decoder-stack workload's
    shapes (synthetic inputs): empirical-Fisher scores of one 4096 x 4096 matrix over
    32768 tokens with all 4096 components, and the global sort-and-truncate over the
    stack's 917,504 components and over a scaled 64M-component pool."""
    import synth
    out = {}
    n, d, k = 32768, 4096, 4096
    a = synth.activation_stream(n, d, 1.0, 41, dtype=torch.bfloat16, device=dev)
    b = synth.activation_stream(n, d, 1.5, 42, dtype=torch.bfloat16, device=dev)
    g = torch.Generator(device="cuda")
    g.manual_seed(43)
    left = torch.randn(d, k, generator=g, device=dev) / d ** 0.5
    right = torch.randn(k, d, generator=g, device=dev) / d ** 0.5
    lrc.lrc_score_components(left=left, right=right, A=a, B=b, mode="fisher")   # warm-up
    t = _time(lambda: lrc.lrc_score_components(left=left, right=right, A=a, B=b, mode="fisher"), torch, 3)
    flops = 2.0 * n * k * (d + d) + 3.0 * n * k
    out["fisher_scores"] = {"workload": f"{n} bf16 tokens, {d}x{d} matrix, {k} components", "ms": round(t * 1e3, 3),
                            "TFLOP/s": round(flops / t / 1e12, 2),
                            "mfma_bf16_frac": round(flops / t / 1e12 / PEAK_TFLOPS["bf16"], 4)}
    del a, b, left, right
    # alternative scores from the singular values (224 matrices x 4096 components)
    n_mat, per = 224, 4096
    sig = torch.sort(torch.rand(n_mat, per, generator=g, device=dev), dim=1, descending=True)[0].reshape(-1)
    offs = torch.arange(0, n_mat * per + 1, per, dtype=torch.int64, device=dev)
    wgt = torch.rand(n_mat, generator=g, device=dev) + 0.5
    for mode in ("unirank", "swift"):
        lrc.lrc_rank_scores(sig, offs, wgt, mode=mode)
        t = _time(lambda: lrc.lrc_rank_scores(sig, offs, wgt, mode=mode), torch, 5)
        byt = 8.0 * n_mat * per   # sigma in, score out
        out[f"rank_scores_{mode}"] = {"workload": f"{n_mat * per} components ({n_mat} matrices)",
                                      "ms": round(t * 1e3, 3), "GB/s": round(byt / t / 1e9, 1)}
    del sig, offs, wgt
    # factor codec at the attention projection's rank-1024 factors
    left = torch.randn(d, 1024, generator=g, device=dev)
    right = torch.randn(1024, d, generator=g, device=dev)
    signs = torch.randint(0, 2, (1024,), generator=g, device=dev).float() * 2 - 1
    lrc.lrc_rotate_quantize(left, right, signs)
    t = _time(lambda: lrc.lrc_rotate_quantize(left, right, signs), torch, 5)
    byt = 5.0 * 2 * d * 1024   # fp32 factors in, int8 codes out
    out["rotate_quantize"] = {"workload": f"left {d}x1024, right 1024x{d} fp32 -> int8", "ms": round(t * 1e3, 3),
                              "GB/s": round(byt / t / 1e9, 1), "hbm_frac": round(byt / t / 1e9 / HBM_PEAK_GBS, 4)}
    del left, right, signs
    # decode-time low-rank FFN (hidden 4096, FFN 11008, every rank 2048, int8 factors)
    dff, rk = 11008, 2048

    def fac(rows, cols):
        return (torch.randint(-127, 128, (rows, cols), generator=g, device=dev, dtype=torch.int8),
                torch.rand(rows, generator=g, device=dev) * 0.004 + 0.001)

    gate = (*fac(rk, d), *fac(dff, rk))
    up = (*fac(rk, d), *fac(dff, rk))
    down = (*fac(dff, rk), *fac(d, rk))   # R_down stored transposed (d_ff x r)
    fbytes = 2.0 * rk * d + 2.0 * dff * rk + dff * rk + d * rk
    for nt in (1, 8):
        xin = torch.randn(nt, d, generator=g, device=dev)
        lrc.lrc_lowrank_ffn(xin, gate, up, down)
        t = _time(lambda: lrc.lrc_lowrank_ffn(xin, gate, up, down), torch, 10)
        out[f"lowrank_ffn_decode_{nt}tok"] = {"workload": f"{nt} tokens, 4096 -> 11008 -> 4096, ranks 2048, int8",
                                             "us": round(t * 1e6, 1), "tokens_per_s": round(nt / t, 1),
                                             "GB/s": round(fbytes / t / 1e9, 1),
                                             "hbm_frac": round(fbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
    del gate, up, down
    # hybrid decode: half the hidden channels low-rank (rank 2048), the other half dense int8
    nl = nd = dff // 2
    gate = (*fac(rk, d), *fac(nl, rk))
    up = (*fac(rk, d), *fac(nl, rk))
    down = (*fac(nl, rk), *fac(d, rk))
    dense = (*fac(nd, d), *fac(nd, d), *fac(d, nd))
    hbytes = 2.0 * rk * d + 2.0 * nl * rk + nl * rk + d * rk + 3.0 * nd * d
    for nt in (1, 8):
        xin = torch.randn(nt, d, generator=g, device=dev)
        lrc.lrc_hybrid_ffn(xin, gate, up, down, dense)
        t = _time(lambda: lrc.lrc_hybrid_ffn(xin, gate, up, down, dense), torch, 10)
        out[f"hybrid_ffn_decode_{nt}tok"] = {
            "workload": f"{nt} tokens, 4096 -> 11008 -> 4096, {nl} channels low-rank (ranks 2048), {nd} dense, int8",
            "us": round(t * 1e6, 1), "tokens_per_s": round(nt / t, 1), "GB/s": round(hbytes / t / 1e9, 1),
            "hbm_frac": round(hbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
    del gate, up, down, dense
    # FFN hybrid channel selection: gate and up 11008 x 4096 at rank 2048 (the factors'
    # values do not change the work), covariance of a 4096-wide stream
    wg = torch.randn(dff, d, generator=g, device=dev) / d ** 0.5
    wu = torch.randn(dff, d, generator=g, device=dev) / d ** 0.5
    fg = (torch.randn(dff, rk, generator=g, device=dev) / rk ** 0.5, torch.randn(rk, d, generator=g, device=dev))
    fu = (torch.randn(dff, rk, generator=g, device=dev) / rk ** 0.5, torch.randn(rk, d, generator=g, device=dev))
    xa = synth.activation_stream(8192, d, 1.0, 44, dtype=torch.bfloat16, device=dev)
    xsum = torch.zeros(d, d, device=dev)
    lrc.lrc_accumulate_cov(xa, xsum)
    del xa
    lrc.lrc_ffn_select_channels(wg, wu, fg, fu, xsum, 8192, dff // 2, 1e-3)
    t = _time(lambda: lrc.lrc_ffn_select_channels(wg, wu, fg, fu, xsum, 8192, dff // 2, 1e-3), torch, 3)
    # per projection: D = W - Left Right (2 d_ff r d) and E = D L_x (d_ff d (d + 1)), plus
    # the Cholesky of X (d^3 / 3)
    flops = 2 * (2.0 * dff * rk * d + dff * d * (d + 1.0)) + d ** 3 / 3.0
    out["ffn_channel_selection"] = {"workload": f"gate and up {dff}x{d}, rank {rk}, select {dff // 2} channels",
                                    "ms": round(t * 1e3, 3), "TFLOP/s": round(flops / t / 1e12, 2),
                                    "mfma_fp32_frac": round(flops / t / 1e12 / PEAK_TFLOPS["f32"], 4)}
    del wg, wu, fg, fu, xsum
    for m_items, label in ((917504, "decoder stack: 224 matrices"), (64 * 1024 * 1024, "scaled pool")):
        n_mat = 224 if m_items == 917504 else 16384
        per = m_items // n_mat
        offs = torch.arange(0, m_items + 1, per, dtype=torch.int64, device=dev)
        cost = torch.where(torch.arange(n_mat, device=dev) % 7 < 4, 8192, 15104).to(torch.int64)
        scores = torch.rand(m_items, generator=g, device=dev)
        budget = int(0.6 * float((cost * per).sum()))
        lrc.lrc_allocate_ranks(scores, offs, cost, budget)
        t = _time(lambda: lrc.lrc_allocate_ranks(scores, offs, cost, budget), torch, 5)
        # bytes a sort-and-truncate must move at least: scores in, order out, per item
        # cost gather/scan and mask (24 B), the 8 radix passes of 64-bit keys + 32-bit
        # ids read and written (8 x 2 x 12 B)
        byt = m_items * (24.0 + 8 * 2 * 12.0)
        out[f"allocation_{m_items}"] = {"workload": f"{m_items} components ({label})", "ms": round(t * 1e3, 3),
                                        "items_per_s": round(m_items / t, 1),
                                        "GB/s": round(byt / t / 1e9, 1),
                                        "hbm_frac": round(byt / t / 1e9 / HBM_PEAK_GBS, 4)}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode (covariance sums would be "
              "all-reduced and matrices dealt out to GPUs; that layer is not built).", file=sys.stderr)
        sys.exit(2)
    import torch

    import curvature_aware_rank_amd as lrc
    import synth

    dev = torch.device("cuda:0")
    d, n, r = args.d, args.tokens, args.rank
    a = synth.activation_stream(n, d, 1.0, 31, outlier_frac=0.01, dtype=torch.bfloat16, device=dev)
    w = synth.weight(d, d, 35, device=dev)
    cov = torch.empty(d, d, dtype=torch.float32, device=dev)
    offs = torch.tensor([0, d], dtype=torch.int64, device=dev)
    cost = torch.tensor([2 * d], dtype=torch.int64, device=dev)
    budget = r * 2 * d
    if args.copy_probe_mib:
        src = torch.ones(args.copy_probe_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        del src, dst
    torch.cuda.synchronize()

    def step():
        cov.zero_()
        lrc.lrc_accumulate_cov(a, cov)
        sig, left, right, info = lrc.lrc_whiten_decompose(w, r, cov, n)
        scores, _ = lrc.lrc_score_components(sigma=sig, mode="kfac")
        return lrc.lrc_allocate_ranks(scores, offs, cost, budget)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: K whole steps, nothing else on the stream
    t0 = time.perf_counter()
    for _ in range(args.steps):
        out = step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    n_kept = int(out[1][0])
    ms = 1e3 * elapsed / args.steps
    # the same K steps again with the library's measurement on: every instrumented launch
    # is bracketed by HIP events on the stream it is enqueued on, and the work each launch
    # performed is counted.  The events add host and GPU time per launch, so this pass is
    # kept apart from the timed one.
    lrc.lrc_profile_start()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof_ms = 1e3 * (time.perf_counter() - t1) / args.steps
    lrc.lrc_profile_stop()
    prof = lrc.lrc_profile_kernels()

    kernels = {}
    for name, k in prof.items():
        avg_ms = k["total_ms"] / max(k["launches"], 1)
        per_launch_flops = k["flops"] / max(k["launches"], 1)
        per_launch_bytes = k["bytes"] / max(k["launches"], 1)
        kernels[name] = {
            "launches_per_step": k["launches"] / args.steps,
            "ms_per_step": round(k["total_ms"] / args.steps, 3),
            "avg_launch_ms": round(avg_ms, 5),
            "TFLOP/s": round(per_launch_flops / (avg_ms * 1e-3) / 1e12, 3) if avg_ms > 0 else None,
            "GB/s": round(per_launch_bytes / (avg_ms * 1e-3) / 1e9, 1) if avg_ms > 0 else None,
        }
    dom = max(prof, key=lambda nm: prof[nm]["total_ms"])
    roof = ROOFLINE[dom]
    dk = prof[dom]
    avg_s = dk["total_ms"] / dk["launches"] * 1e-3
    work = (dk["flops"] if roof["unit"] == "TFLOP/s" else dk["bytes"]) / dk["launches"]
    achieved = work / avg_s / (1e12 if roof["unit"] == "TFLOP/s" else 1e9)

    syrk = prof["syrk_bf16_kernel"]
    syrk_s = syrk["total_ms"] * 1e-3 / args.steps        # one launch per step here
    res = {
        "metric": METRIC,
        "value": round(1e3 / ms, 4),
        "unit": "layers/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16/f32/f64",
        "data": "synthetic",
        "config": {"workload": f"attention projection W {d}x{d} fp32, {n} bf16 calibration tokens "
                               f"(power-law spectrum, 1% outlier channels x20), activation-only whitening, rank {r}",
                   "tokens_per_layer": n, "d": d, "rank": r},
        "cov_tokens_per_s": round(n / syrk_s, 1),
        "step_tokens_per_s": round(n * 1e3 / ms, 1),
        "n_kept": n_kept,
        "profiled_ms_per_step": round(prof_ms, 3),
        "roofline": {"bound": roof["bound"], "kernel": dom, "dtype": roof["dtype"],
                     "achieved": round(achieved, 3), "peak": roof["peak"], "unit": roof["unit"],
                     "frac": round(achieved / roof["peak"], 4), "traffic": TRAFFIC.get(dom),
                     "avg_launch_ms": round(dk["total_ms"] / dk["launches"], 5),
                     "launches_per_step": dk["launches"] / args.steps},
        "kernels": kernels,
    }
    if not args.no_secondary:
        res["secondary"] = secondary(lrc, torch, dev)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(d, n, r)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
