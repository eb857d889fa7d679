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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--tokens", type=int, default=65536)
    p.add_argument("--d", type=int, default=4096)
    p.add_argument("--rank", type=int, default=1024)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cov-reps", type=int, default=10, help="extra timed SYRK launches for its event timing")
    return p.parse_args()


def cpu_baseline(d, n, rank):
    """The fp64 oracle on host cores, on a bounded sample of the same workload:
    covariance of 8192 tokens (scaled by tokens) + the decomposition of a d/2 x d/2
    layer at rank/2 (scaled by the cube of the size)."""
    import numpy as np
    import torch

    import oracle
    import synth

    try:
        from threadpoolctl import threadpool_info
        threads = max(int(i.get("num_threads", 1)) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:
        threads = len(os.sched_getaffinity(0))
    ns = min(8192, n)
    a = synth.activation_stream(ns, d, 1.0, 31, outlier_frac=0.01, dtype=torch.bfloat16).float().numpy()
    t0 = time.perf_counter()
    oracle.covariance_sum(a)
    t_cov = (time.perf_counter() - t0) * (n / ns)
    ds, rs = d // 2, rank // 2
    a2 = synth.activation_stream(4 * ds, ds, 1.0, 32, outlier_frac=0.01, dtype=torch.bfloat16).float().numpy()
    xs = oracle.covariance_sum(a2)
    w = synth.weight(ds, ds, 33).numpy()
    t0 = time.perf_counter()
    res = oracle.whiten_decompose(w, xs, 4 * ds, rank=rs)
    sc = oracle.kfac_scores(res["sigma"])
    oracle.allocate([sc.astype(np.float32)], [2 * ds], rs * 2 * ds)
    t_dec = (time.perf_counter() - t0) * (d / ds) ** 3
    step = t_cov + t_dec
    return {"value": 1.0 / step, "unit": "layers/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 covariance of {ns} of {n} tokens (x{n / ns:g}) + Cholesky/whiten/SVD/back-map/"
                      f"scores/allocation at {ds}x{ds} r={rs} (x{(d / ds) ** 3:g} by d^3)",
            "cov_tokens_per_s": n / t_cov, "seconds_measured": round(t_cov * ns / n + t_dec / (d / ds) ** 3, 2)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode (see DESIGN.md for how it "
              "would shard).", file=sys.stderr)
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
    torch.cuda.synchronize()

    def step():
        cov.zero_()
        lrc.lrc_accumulate_cov(a, cov)
        sig, left, right, info = lrc.lrc_whiten_decompose(w, r, cov, n)
        scores = lrc.lrc_score_components(sigma=sig, mode="kfac")
        return lrc.lrc_allocate_ranks(scores, offs, cost, budget)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        out = step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    n_kept = int(out[1][0])
    ms = 1e3 * elapsed / args.steps

    # live event timing of the covariance SYRK launch on the stream it runs on
    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.cov_reps)]
    for e0, e1 in ev:
        cov.zero_()
        e0.record(st)
        lrc.lrc_accumulate_cov(a, cov)
        e1.record(st)
    torch.cuda.synchronize()
    cov_ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[len(ev) // 2]
    cov_flop = float(n) * d * (d + 1)          # lower triangle incl. diagonal, 2 flop per product
    cov_bytes = float(n) * d * 2               # each token row read once (bf16)
    t1 = time.perf_counter()
    for _ in range(args.steps):
        lrc.lrc_whiten_decompose(w, r, cov, n)
    torch.cuda.synchronize()
    dec_s = (time.perf_counter() - t1) / args.steps

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
        "cov_tokens_per_s": round(n / (cov_ms * 1e-3), 1),
        "step_tokens_per_s": round(n * 1e3 / ms, 1),
        "decomp_layers_per_s": round(1.0 / dec_s, 4),
        "n_kept": n_kept,
        "roofline": {"bound": "mfma", "kernel": "syrk_bf16_kernel", "achieved": round(cov_flop / (cov_ms * 1e-3) / 1e12, 2),
                     "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                     "frac": round(cov_flop / (cov_ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 4),
                     "traffic": None, "launch_ms": round(cov_ms, 4),
                     "hbm_GBps_min_bytes": round(cov_bytes / (cov_ms * 1e-3) / 1e9, 1)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(d, n, r)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
