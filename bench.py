"""Benchmark of the whitened truncated decomposition path on one MI355X.

One step = the whole path over one calibration batch of the attention-projection
workload: 65536 bf16 tokens x 4096 channels streamed into the activation covariance
(SYRK on MFMA), Cholesky, whitening, fp64 Gram + eigensolve, back-map to rank 1024,
per-component K-FAC scores (this workload has no gradients) and the global
sort-and-truncate at the budget of rank 1024.  Inputs are resident in HBM before the
timed region.  The K timed steps are independent layers spread over --streams HIP
streams (default 3 on the 8 hardware queues the bench asks HIP for; each stream has its
own covariance buffers and its own host thread that enqueues its steps); each stream
decomposes --layers-per-call of its layers per call (default 4, each layer with its own
covariance), so up to twelve layers are in flight at a time; `value` is K / the wall time of
the region.  The same K steps one after another on one stream, one layer per call, give
`value_one_stream` (one layer's latency).  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--streams S] [--layers-per-call L]
                    [--no-cpu-baseline] [--no-secondary]
    python bench.py --only syrk|tridiag|fisher|alloc|qaw|ffn-decode [--copy-probe-mib M]

The --only modes run one part of the path a few times (and, with --copy-probe-mib, a
plain device copy of known size first): they are the programs the rocprofv3 summaries
under profiles/ were taken from.  They never start the library's own event timing, so a
counter profiler sees ordinary kernel launches.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


METRIC = "calib tokens/s into cov (4096-d) + whitened-SVD layers/s at 4096×4096, r=1024"
HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3, "f64": 78.6}

# roofline class of each instrumented kernel: MFMA contractions against the dense peak of
# their input type, the fp64 kernels against the fp64 peak (vector and matrix fp64 peaks
# are equal on MI355X), streaming passes against HBM
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
    "tri_syr2k_kernel": {"bound": "alu", "dtype": "f64", "peak": PEAK_TFLOPS["f64"], "unit": "TFLOP/s"},
    "bt_vtz_kernel": {"bound": "alu", "dtype": "f64", "peak": PEAK_TFLOPS["f64"], "unit": "TFLOP/s"},
    "bt_update_kernel": {"bound": "alu", "dtype": "f64", "peak": PEAK_TFLOPS["f64"], "unit": "TFLOP/s"},
}

# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE on this
# workload, scaled by the copy-kernel calibration, with the commit of the kernel source the
# counters were taken on (profiles/counters_tri_symv_attnproj_4096.md: fetch 24.44 MB +
# write 0.77 MB, the average over the 3968 launches of a 4096-wide tridiagonalisation).
# A kernel without an entry reports traffic null.
TRAFFIC = {"tri_symv_kernel": {"bytes": 25.22e6, "kernel_source_commit": "8db424f"}}


def layer_flops(d, r):
    """Algorithmic flops of one decomposition of a d x d weight at rank r with G = I:
    Cholesky d^3/3, whitening d^3, Gram d^3, tridiagonalisation 4d^3/3, back-transformation
    and back-map 2 d^2 r each, triangular solve d^2 r."""
    return d ** 3 / 3 + d ** 3 + d ** 3 + 4 * d ** 3 / 3 + 4.0 * d * d * r + d * d * r


def layer_bytes(d):
    """Bytes the BLAS-2 half of a one-stage tridiagonalisation reads: the fp64 lower
    trailing matrix once per column, 8 B x d^3 / 6."""
    return 4.0 * d ** 3 / 3


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # enough steps to keep every stream busy (the timed region is under a second)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--tokens", type=int, default=65536)
    p.add_argument("--d", type=int, default=4096)
    p.add_argument("--rank", type=int, default=1024)
    p.add_argument("--streams", type=int, default=None,
                   help="HIP streams the timed steps run on, each fed by its own host thread (independent layers "
                        "in flight); default: one less than the hardware queues, at most 3")
    p.add_argument("--layers-per-call", type=int, default=4,
                   help="independent layers a stream decomposes per call (one covariance each)")
    p.add_argument("--hw-queues", type=int, default=8,
                   help="hardware queues HIP gives this process (GPU_MAX_HW_QUEUES, set before HIP starts)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true", help="skip the other workloads and passes")
    p.add_argument("--only", choices=["syrk", "tridiag", "fisher", "alloc", "qaw", "ffn-decode"], default=None,
                   help="run one part of the path (for rocprofv3) instead of the benchmark")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="first run a plain elementwise copy (neg) of this many MiB three times: the "
                        "known-size kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    return p.parse_args()


_T_START = time.perf_counter()


def progress(msg):
    """One line per finished part on stderr (the JSON result is the only stdout line)."""
    print(f"[bench {time.perf_counter() - _T_START:7.1f}s] {msg}", file=sys.stderr, flush=True)


def blas_info():
    """(vendor string, thread count) of the host BLAS numpy uses."""
    import numpy  # noqa: F401  (loads the BLAS)
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            i = infos[0]
            return f"{i.get('internal_api')} {i.get('version')} ({i.get('architecture')})", int(i["num_threads"])
    except Exception:
        pass
    return "unknown", len(os.sched_getaffinity(0))


def cpu_baseline(d, n, rank):
    """The fp64 oracle on host cores: config 1 whole (covariance over all n tokens, then
    Cholesky, whitening, SVD, back-map, K-FAC scores and allocation of the layer), plus
    bounded-sample estimates of the other workloads (each labelled with its sample)."""
    import numpy as np
    import torch

    import oracle
    import synth

    vendor, threads = blas_info()
    a = synth.activation_stream(n, d, 1.0, 31, outlier_frac=0.01, dtype=torch.bfloat16).float().numpy()
    t0 = time.perf_counter()
    xs = oracle.covariance_sum(a)
    t_cov = time.perf_counter() - t0
    del a
    w = synth.weight(d, d, 35).numpy()
    t0 = time.perf_counter()
    res = oracle.whiten_decompose(w, xs, n, rank=rank)
    sc = oracle.kfac_scores(res["sigma"])
    oracle.allocate([sc.astype(np.float32)], [2 * d], rank * 2 * d)
    t_dec = time.perf_counter() - t0
    cov_rate = n / t_cov                                  # tokens/s into a d-wide covariance
    per_cfg = {"attention_projection_4096": {"s": round(t_cov + t_dec, 2), "sample": "whole workload"}}
    spent = t_cov + t_dec
    progress(f"oracle: attention projection {t_cov + t_dec:.1f} s")

    # single linear layer 256 x 256, 4096 fp32 tokens, two-sided, rank 64: whole
    cs0 = synth.workload_spec("single_layer_256")
    a0 = synth.stream(cs0, "a").numpy()
    b0 = synth.stream(cs0, "b").numpy()
    w0 = synth.weight(256, 256, 3).numpy()
    t1 = time.perf_counter()
    oracle.whiten_decompose(w0, oracle.covariance_sum(a0), cs0.n_tokens, oracle.covariance_sum(b0), cs0.n_tokens,
                            rank=64)
    t0 = time.perf_counter() - t1
    per_cfg["single_layer_256"] = {"s": round(t0, 3), "sample": "whole workload"}
    spent += t0
    progress("oracle: single layer")

    # FFN pair: covariances per token measured on 2048 tokens of each stream of the up
    # projection (x 131072 / 2048, twice for the pair), the up projection's two-sided
    # decomposition at full size (the down projection's taken as equal)
    cs2 = synth.workload_spec("ffn_pair_11008x4096", n_tokens=2048)
    t_tok = 0.0
    covs = {}
    for key in ("a_up", "b_up"):
        s = synth.stream(cs2, key).float().numpy()
        if key.startswith("a"):
            s = oracle.qaw_fake_quant(s)[2]
        t1 = time.perf_counter()
        covs[key] = oracle.covariance_sum(s)
        t_tok += time.perf_counter() - t1
    t_cov2 = 2 * t_tok * (131072 / 2048)
    wu = synth.weight(11008, 4096, 45).numpy()
    t1 = time.perf_counter()
    oracle.whiten_decompose(wu, covs["a_up"], 2048, covs["b_up"], 2048, rank=2048)
    t_dec2 = time.perf_counter() - t1
    per_cfg["ffn_pair_11008x4096"] = {
        "s": round(t_cov2 + 2 * t_dec2, 1),
        "sample": "covariances of 2048 tokens per stream (x64, x2) + the up projection's decomposition (x2)"}
    spent += t_tok + t_dec2
    progress("oracle: FFN pair sample")

    # decoder stack: one 4096 x 4096 decomposition with every component and its Fisher
    # scores on 1024 tokens (x32 to the 32768 tokens), both x224; covariances at the
    # measured per-token rate (scaled by width squared); the 917,504-component allocation
    # whole
    cs3 = synth.workload_spec("decoder_stack_32_layers", n_tokens=1024)
    a3 = synth.stream(cs3, "attn_in").float().numpy()
    b3 = synth.stream(cs3, "g_q").float().numpy()
    w3 = synth.weight(4096, 4096, 1000).numpy()
    t1 = time.perf_counter()
    r3 = oracle.whiten_decompose(w3, xs, n, rank=4096)
    t_dec3 = time.perf_counter() - t1
    t1 = time.perf_counter()
    f3 = oracle.fisher_scores(a3, b3, r3["left"], r3["right"])
    t_fis = time.perf_counter() - t1
    pool = [f3.astype(np.float32)] * 224
    t1 = time.perf_counter()
    oracle.allocate(pool, [8192] * 224, 3885603225)
    t_alloc3 = time.perf_counter() - t1
    cov3 = 32 * 32768 / cov_rate * (3 + (11008 / 4096) ** 2)
    per_cfg["decoder_stack_32_layers"] = {
        "s": round(224 * (t_dec3 + 32 * t_fis) + cov3 + t_alloc3, 0),
        "sample": "one 4096x4096 decomposition (x224), its Fisher scores on 1024 tokens (x32, x224), covariances "
                  "at the measured per-token rate, the 917504-component allocation whole"}
    spent += t_dec3 + t_fis + t_alloc3
    progress("oracle: decoder stack sample")

    # per-head K/V: the shared covariance at the measured per-token rate, 64 head
    # decompositions whole
    lx, _ = oracle.cholesky_lower(xs / n)
    t1 = time.perf_counter()
    for h in range(64):
        wh = w[(h % 32) * 128:(h % 32 + 1) * 128]
        oracle.truncated_svd(oracle.whiten(wh, lx))
    t_heads = time.perf_counter() - t1
    per_cfg["kv_heads_64x128x4096"] = {"s": round(65536 / cov_rate + t_heads, 2),
                                       "sample": "covariance at the measured per-token rate, 64 head SVDs whole"}
    spent += t_heads

    return {"value": 1.0 / (t_cov + t_dec), "unit": "layers/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"the whole attention-projection layer: fp64 covariance of all {n} tokens + {d}x{d} "
                      f"Cholesky/whitening/SVD/back-map/K-FAC scores/allocation at rank {rank}",
            "blas": vendor, "blas_threads": threads, "cov_tokens_per_s": round(cov_rate, 1),
            "seconds_measured": round(spent, 1), "per_config_s": per_cfg}


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


def _time_queued(fn, torch, reps):
    """time per call of reps calls queued back to back on the stream (two events around
    them): the device's time per call whenever the host enqueues faster than the device
    runs, so the binding's per-call host work (output allocation, argument marshalling)
    is not counted as it is in _time's synchronised calls"""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / 1e3 / reps


def workloads(lrc, torch, dev, workers):
    """End-to-end GPU times of the other workloads (inputs resident, generation excluded).
    workers: the streams the decoder stack's matrices are spread over (the ones the timed
    steps ran on: the GPU has few hardware queues, and streams beyond them share one)."""
    import synth
    out = {}
    # single linear layer: 256 x 256, 4096 fp32 tokens, two-sided, rank 64
    cs = synth.workload_spec("single_layer_256")
    a = synth.stream(cs, "a", device=dev)
    b = synth.stream(cs, "b", device=dev)
    w = synth.weight(256, 256, 3, device=dev)
    xs = torch.empty(256, 256, device=dev)
    gs = torch.empty(256, 256, device=dev)

    def cfg0():
        xs.zero_()
        gs.zero_()
        lrc.lrc_accumulate_cov(a, xs)
        lrc.lrc_accumulate_cov(b, gs)
        return lrc.lrc_whiten_decompose(w, 64, xs, 4096, gs, 4096)

    cfg0()
    t = _time(cfg0, torch, 5)
    out["single_layer_256"] = {"workload": "256x256 fp32, 4096 fp32 tokens, two-sided, rank 64",
                               "ms": round(t * 1e3, 3)}
    progress("workload: single layer")
    del a, b, w, xs, gs

    # FFN pair: 131072 bf16 tokens per stream, QAW on the activations, two-sided, rank 2048
    cs = synth.workload_spec("ffn_pair_11008x4096")
    st = {k: synth.stream(cs, k, device=dev) for k in cs.streams}
    ws = [synth.weight(m.d_out, m.d_in, 45 + i, device=dev) for i, m in enumerate(cs.matrices)]
    covs = {k: torch.empty(v.shape[1], v.shape[1], device=dev) for k, v in st.items()}

    def cfg2():
        # the four covariances on the current stream, then the two decompositions on the
        # worker streams (independent matrices)
        for k, c in covs.items():
            c.zero_()
            lrc.lrc_accumulate_cov(st[k], c, quant=k.startswith("a"))
        main_st = torch.cuda.current_stream()
        for wst in workers:
            wst.wait_stream(main_st)

        def feed(mi):
            m, wm = cs.matrices[mi], ws[mi]
            torch.cuda.set_device(dev)
            with torch.cuda.stream(workers[mi % len(workers)]):
                lrc.lrc_whiten_decompose(wm, 2048, covs[m.a_stream], cs.n_tokens, covs[m.b_stream], cs.n_tokens)

        with ThreadPoolExecutor(max_workers=len(cs.matrices)) as ex:
            list(ex.map(feed, range(len(cs.matrices))))   # re-raises a failure of any thread
        for wst in workers:
            main_st.wait_stream(wst)

    cfg2()
    t = _time(cfg2, torch, 2)
    out["ffn_pair_11008x4096"] = {"workload": "up 11008x4096 + down 4096x11008, 131072 bf16 tokens per stream, "
                                              "int8 QAW, two-sided, rank 2048", "streams": len(workers),
                                  "ms": round(t * 1e3, 1)}
    progress("workload: FFN pair")
    # the QAW pre-pass alone, measured on the library's events (bf16 read, int8 codes and
    # the two bf16 terms written)
    lrc.lrc_profile_start()
    c = covs["a_down"]
    c.zero_()
    lrc.lrc_accumulate_cov(st["a_down"], c, quant=True)
    torch.cuda.synchronize()
    lrc.lrc_profile_stop()
    q = lrc.lrc_profile_kernels().get("qaw_prepass_kernel")
    if q and q["total_ms"] > 0:
        gbs = q["bytes"] / (q["total_ms"] * 1e-3) / 1e9
        out["qaw_prepass"] = {"workload": "131072 bf16 tokens x 11008", "ms": round(q["total_ms"], 3),
                              "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    del st, ws, covs, c

    # decoder stack: 32 layers x (4 covariances + 7 decompositions with every component +
    # 7 empirical-Fisher score passes) and one allocation over the 917,504 components; one
    # layer's streams and weights are generated once and reused by every layer (the work
    # does not depend on the values).  A layer's covariances are made on the main stream
    # (two sets, alternating by layer, so that the next layer's accumulate while this
    # layer's decompositions run); its seven matrices, in four groups by input covariance,
    # are decomposed and scored on the worker streams, round robin, each worker stream
    # enqueued by a host thread of its own; the allocation runs once all of them are done.
    cs = synth.workload_spec("decoder_stack_32_layers")
    n = cs.n_tokens
    st = {k: synth.stream(cs, k, device=dev) for k in cs.streams}
    ws = [synth.weight(m.d_out, m.d_in, 1000 + i, device=dev) for i, m in enumerate(cs.matrices)]
    cov_keys = ("attn_in", "o_in", "mlp_in", "down_in")
    cov_sets = [{k: torch.empty(st[k].shape[1], st[k].shape[1], device=dev) for k in cov_keys} for _ in range(2)]
    scores = torch.empty(224 * 4096, device=dev)
    offs = torch.arange(0, 224 * 4096 + 1, 4096, dtype=torch.int64, device=dev)
    cost = torch.tensor([m.d_out + m.d_in for m in cs.matrices] * 32, dtype=torch.int64, device=dev)
    budget = int(0.6 * 32 * sum(m.d_out * m.d_in for m in cs.matrices))
    # matrices that share an input covariance (q, k, v; gate, up) are decomposed in one
    # batched call: their Cholesky is formed once and their reductions share every launch
    groups = []
    for key in dict.fromkeys(m.a_stream for m in cs.matrices):
        members = [mi for mi, m in enumerate(cs.matrices) if m.a_stream == key]
        groups.append((members, torch.stack([ws[mi] for mi in members]) if len(members) > 1 else ws[members[0]]))
    ns = len(workers)
    main_st = torch.cuda.current_stream()
    done = [[torch.cuda.Event() for _ in range(ns)] for _ in range(2)]   # per covariance set
    pool = ThreadPoolExecutor(max_workers=ns)   # one host thread enqueues each worker stream
    torch.cuda.synchronize()
    progress("workload: decoder stack inputs ready")
    t0 = time.perf_counter()
    for layer in range(32):
        covs = cov_sets[layer % 2]
        if layer >= 2:   # this set's previous layer has been decomposed
            for e in done[layer % 2]:
                main_st.wait_event(e)
        for k, c in covs.items():
            c.zero_()
            lrc.lrc_accumulate_cov(st[k], c)
        ready = torch.cuda.Event()
        ready.record(main_st)
        for wst in workers:
            wst.wait_event(ready)
        def feed(i, layer=layer, covs=covs):
            torch.cuda.set_device(dev)
            with torch.cuda.stream(workers[i]):
                for gi in range(i, len(groups), ns):
                    members, wg = groups[gi]
                    m0 = cs.matrices[members[0]]
                    _, left, right, _ = lrc.lrc_whiten_decompose(wg, 4096, covs[m0.a_stream], n)
                    for bi, mi in enumerate(members):
                        m = cs.matrices[mi]
                        j = (layer * 7 + mi) * 4096
                        lf, rt = (left[bi], right[bi]) if wg.dim() == 3 else (left, right)
                        lrc.lrc_score_components(lf, rt, A=st[m.a_stream], B=st[m.b_stream], scores=scores[j:j + 4096])
                    del left, right
            done[layer % 2][i].record(workers[i])

        list(pool.map(feed, range(ns)))
    for wst in workers:
        main_st.wait_stream(wst)
    lrc.lrc_allocate_ranks(scores, offs, cost, budget)
    torch.cuda.synchronize()
    t = time.perf_counter() - t0
    out["decoder_stack_32_layers"] = {
        "workload": "32 layers x (q,k,v,o 4096x4096, gate/up 11008x4096, down 4096x11008), 32768 bf16 tokens per "
                    "stream, every component decomposed and Fisher-scored, allocation of 917504 components at 60%",
        "streams": ns, "calls_per_layer": len(groups), "s": round(t, 2), "matrices_per_s": round(224 / t, 2)}
    progress(f"workload: decoder stack {t:.1f} s on {ns} stream(s)")
    pool.shutdown()
    del st, ws, groups, cov_sets, scores

    # per-head K/V: 65536 bf16 tokens, 64 head slices of 128 x 4096, K-FAC scores, 40% budget
    cs = synth.workload_spec("kv_heads_64x128x4096")
    a = synth.stream(cs, "a", device=dev)
    w3 = torch.cat([synth.weight(4096, 4096, 137, device=dev), synth.weight(4096, 4096, 139, device=dev)]).view(
        64, 128, 4096)
    cov = torch.empty(4096, 4096, device=dev)
    offs = torch.arange(0, 64 * 128 + 1, 128, dtype=torch.int64, device=dev)
    cost = torch.full((64,), 128 + 4096, dtype=torch.int64, device=dev)

    def cfg4():
        cov.zero_()
        lrc.lrc_accumulate_cov(a, cov)
        sig, _, _, _ = lrc.lrc_whiten_decompose(w3, 128, cov, 65536)
        sc, _ = lrc.lrc_score_components(sigma=sig.reshape(-1), mode="kfac")
        return lrc.lrc_allocate_ranks(sc, offs, cost, int(0.4 * 2 * 4096 * 4096))

    cfg4()
    t = _time(cfg4, torch, 3)
    out["kv_heads_64x128x4096"] = {"workload": "64 heads of 128x4096 sharing one covariance of 65536 bf16 tokens, "
                                               "K-FAC scores, allocation at 40%", "ms": round(t * 1e3, 2)}
    progress("workload: K/V heads")
    return out


def _fac(torch, g, dev, rows, cols):
    return (torch.randint(-127, 128, (rows, cols), generator=g, device=dev, dtype=torch.int8),
            torch.rand(rows, generator=g, device=dev) * 0.004 + 0.001)


def _ffn_factors(torch, g, dev, d, d_ff, rk):
    """int8 factor sets of a low-rank SwiGLU FFN: gate and up (R rk x d, L d_ff x rk), down
    with R_down (rk x d_ff) stored transposed (d_ff x rk) beside its rk row scales."""
    gate = (*_fac(torch, g, dev, rk, d), *_fac(torch, g, dev, d_ff, rk))
    up = (*_fac(torch, g, dev, rk, d), *_fac(torch, g, dev, d_ff, rk))
    q_rd, s_rd = _fac(torch, g, dev, rk, d_ff)
    down = (q_rd.t().contiguous(), s_rd, *_fac(torch, g, dev, d, rk))
    return gate, up, down


def passes(lrc, torch, dev):
    """Throughput of the scoring and allocation passes at the decoder-stack workload's
    shapes (synthetic inputs), and of the follow-on kernels."""
    import synth
    out = {}
    # a long covariance stream: 1,048,576 bf16 tokens x 4096 in one call (16 copies of a
    # 65536-token block, 8 GiB resident), so that launches and the split reduction are
    # amortised over many tokens
    blk = synth.activation_stream(65536, 4096, 1.0, 40, outlier_frac=0.01, dtype=torch.bfloat16, device=dev)
    big = blk.repeat(16, 1)
    del blk
    cov = torch.zeros(4096, 4096, device=dev)
    lrc.lrc_accumulate_cov(big, cov)
    t = _time_queued(lambda: lrc.lrc_accumulate_cov(big, cov), torch, 3)
    nt = big.shape[0]
    out["cov_stream_1m"] = {"workload": f"{nt} bf16 tokens x 4096 in one call", "ms": round(t * 1e3, 3),
                            "tokens_per_s": round(nt / t, 1),
                            "mfma_bf16_frac": round(nt * 4096 * 4097.0 / t / 1e12 / PEAK_TFLOPS["bf16"], 4)}
    del big, cov
    progress("pass: long covariance stream")
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
    progress("pass: Fisher scores")
    del a, b, left, right
    # alternative scores from the singular values (224 matrices x 4096 components)
    n_mat, per = 224, 4096
    sig = torch.sort(torch.rand(n_mat, per, generator=g, device=dev), dim=1, descending=True)[0].reshape(-1)
    offs = torch.arange(0, n_mat * per + 1, per, dtype=torch.int64, device=dev)
    wgt = torch.rand(n_mat, generator=g, device=dev) + 0.5
    for mode in ("unirank", "swift"):
        lrc.lrc_rank_scores(sig, offs, wgt, mode=mode)
        t = _time(lambda: lrc.lrc_rank_scores(sig, offs, wgt, mode=mode), torch, 5)
        tq = _time_queued(lambda: lrc.lrc_rank_scores(sig, offs, wgt, mode=mode), torch, 50)
        byt = 8.0 * n_mat * per   # sigma in, score out
        out[f"rank_scores_{mode}"] = {"workload": f"{n_mat * per} components ({n_mat} matrices)",
                                      "ms": round(t * 1e3, 3), "ms_queued": round(tq * 1e3, 4),
                                      "GB/s": round(byt / tq / 1e9, 1)}
    del sig, offs, wgt
    # factor codec at the attention projection's rank-1024 factors
    left = torch.randn(d, 1024, generator=g, device=dev)
    right = torch.randn(1024, d, generator=g, device=dev)
    signs = torch.randint(0, 2, (1024,), generator=g, device=dev).float() * 2 - 1
    lrc.lrc_rotate_quantize(left, right, signs)
    t = _time(lambda: lrc.lrc_rotate_quantize(left, right, signs), torch, 5)
    tq = _time_queued(lambda: lrc.lrc_rotate_quantize(left, right, signs), torch, 50)
    byt = 5.0 * 2 * d * 1024   # fp32 factors in, int8 codes out
    out["rotate_quantize"] = {"workload": f"left {d}x1024, right 1024x{d} fp32 -> int8", "ms": round(t * 1e3, 3),
                              "ms_queued": round(tq * 1e3, 4), "GB/s": round(byt / tq / 1e9, 1),
                              "hbm_frac": round(byt / tq / 1e9 / HBM_PEAK_GBS, 4)}
    del left, right, signs
    # decode-time low-rank FFN (hidden 4096, FFN 11008, every rank 2048, int8 factors)
    dff, rk = 11008, 2048
    gate, up, down = _ffn_factors(torch, g, dev, d, dff, rk)
    fbytes = 2.0 * rk * d + 2.0 * dff * rk + dff * rk + d * rk
    for nt in (1, 8):
        xin = torch.randn(nt, d, generator=g, device=dev)
        lrc.lrc_lowrank_ffn(xin, gate, up, down)
        t = _time(lambda: lrc.lrc_lowrank_ffn(xin, gate, up, down), torch, 10)
        tq = _time_queued(lambda: lrc.lrc_lowrank_ffn(xin, gate, up, down), torch, 100)
        out[f"lowrank_ffn_decode_{nt}tok"] = {"workload": f"{nt} tokens, 4096 -> 11008 -> 4096, ranks 2048, int8",
                                             "us": round(t * 1e6, 1), "us_queued": round(tq * 1e6, 1),
                                             "tokens_per_s": round(nt / t, 1), "GB/s": round(fbytes / tq / 1e9, 1),
                                             "hbm_frac": round(fbytes / tq / 1e9 / HBM_PEAK_GBS, 4)}
    del gate, up, down
    # hybrid decode: half the hidden channels low-rank (rank 2048), the other half dense int8
    nl = nd = dff // 2
    gate, up, down = _ffn_factors(torch, g, dev, d, nl, rk)
    dense = (*_fac(torch, g, dev, nd, d), *_fac(torch, g, dev, nd, d), *_fac(torch, g, dev, d, nd))
    hbytes = 2.0 * rk * d + 2.0 * nl * rk + nl * rk + d * rk + 3.0 * nd * d
    for nt in (1, 8):
        xin = torch.randn(nt, d, generator=g, device=dev)
        lrc.lrc_hybrid_ffn(xin, gate, up, down, dense)
        t = _time(lambda: lrc.lrc_hybrid_ffn(xin, gate, up, down, dense), torch, 10)
        tq = _time_queued(lambda: lrc.lrc_hybrid_ffn(xin, gate, up, down, dense), torch, 100)
        out[f"hybrid_ffn_decode_{nt}tok"] = {
            "workload": f"{nt} tokens, 4096 -> 11008 -> 4096, {nl} channels low-rank (ranks 2048), {nd} dense, int8",
            "us": round(t * 1e6, 1), "us_queued": round(tq * 1e6, 1), "tokens_per_s": round(nt / t, 1),
            "GB/s": round(hbytes / tq / 1e9, 1), "hbm_frac": round(hbytes / tq / 1e9 / HBM_PEAK_GBS, 4)}
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
    progress("pass: codec, decode FFN, channel selection")
    for m_items, label in ((917504, "decoder stack: 224 matrices"), (64 * 1024 * 1024, "scaled pool")):
        n_mat = 224 if m_items == 917504 else 16384
        per = m_items // n_mat
        offs = torch.arange(0, m_items + 1, per, dtype=torch.int64, device=dev)
        cost = torch.where(torch.arange(n_mat, device=dev) % 7 < 4, 8192, 15104).to(torch.int64)
        scores = torch.rand(m_items, generator=g, device=dev)
        budget = int(0.6 * float((cost * per).sum()))
        lrc.lrc_allocate_ranks(scores, offs, cost, budget)
        t = _time(lambda: lrc.lrc_allocate_ranks(scores, offs, cost, budget), torch, 5)
        tq = _time_queued(lambda: lrc.lrc_allocate_ranks(scores, offs, cost, budget), torch, 20)
        # bytes a sort-and-truncate must move at least: scores in, order out, per item
        # cost gather/scan and mask (24 B), the 8 radix passes of 64-bit keys + 32-bit
        # ids read and written (8 x 2 x 12 B)
        byt = m_items * (24.0 + 8 * 2 * 12.0)
        out[f"allocation_{m_items}"] = {"workload": f"{m_items} components ({label})", "ms": round(t * 1e3, 3),
                                        "ms_queued": round(tq * 1e3, 4), "items_per_s": round(m_items / tq, 1),
                                        "GB/s": round(byt / tq / 1e9, 1),
                                        "hbm_frac": round(byt / tq / 1e9 / HBM_PEAK_GBS, 4)}
        # the same cut without the order (radix select weighted by cost): bytes per item are
        # the scores read by the three full select levels and the mask pass (4 x 4 B) and
        # the mask written (1 B; the mask pass also counts the ranks); the candidate list of
        # the later levels (a few percent of the items) is left out
        sel = lambda: lrc.lrc_allocate_ranks(scores, offs, cost, budget, want_order=False)
        sel()
        t = _time(sel, torch, 5)
        tq = _time_queued(sel, torch, 20)
        byt = m_items * (4 * 4.0 + 1.0)
        out[f"allocation_{m_items}_no_order"] = {
            "workload": f"{m_items} components ({label}), n_kept/ranks/mask only", "ms": round(t * 1e3, 3),
            "ms_queued": round(tq * 1e3, 4), "items_per_s": round(m_items / tq, 1), "GB/s": round(byt / tq / 1e9, 1),
            "hbm_frac": round(byt / tq / 1e9 / HBM_PEAK_GBS, 4)}
    return out


def copy_probe(torch, dev, mib):
    """A plain elementwise copy (torch.neg) of mib MiB, three times: a kernel of known
    size whose FETCH_SIZE / WRITE_SIZE readings calibrate the counters."""
    src = torch.ones(mib << 18, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


def only(args, lrc, torch, dev):
    """The --only modes (programs for rocprofv3; no library event timing)."""
    import synth
    if args.copy_probe_mib:
        copy_probe(torch, dev, args.copy_probe_mib)
    res = {"mode": args.only}
    if args.only == "syrk":
        # three accumulations of the attention projection's token block
        a = synth.activation_stream(args.tokens, args.d, 1.0, 31, outlier_frac=0.01, dtype=torch.bfloat16,
                                    device=dev)
        cov = torch.zeros(args.d, args.d, device=dev)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(3):
            cov.zero_()
            lrc.lrc_accumulate_cov(a, cov)
        e.record()
        torch.cuda.synchronize()
        res["ms_per_accumulation"] = round(s.elapsed_time(e) / 3, 4)
    elif args.only == "fisher":
        # empirical-Fisher scores at the decoder stack's attention shape: 32768 bf16 tokens,
        # a 4096 x 4096 matrix, all 4096 components; one untimed and five timed calls
        n, d, k = 32768, 4096, 4096
        a = synth.activation_stream(n, d, 1.0, 41, dtype=torch.bfloat16, device=dev)
        b = synth.activation_stream(n, d, 1.5, 42, dtype=torch.bfloat16, device=dev)
        g = torch.Generator(device=dev)
        g.manual_seed(43)
        left = torch.randn(d, k, generator=g, device=dev) / d ** 0.5
        right = torch.randn(k, d, generator=g, device=dev) / d ** 0.5
        lrc.lrc_score_components(left=left, right=right, A=a, B=b)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(5):
            lrc.lrc_score_components(left=left, right=right, A=a, B=b)
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / 5
        flops = 2.0 * n * k * (d + d) + 3.0 * n * k
        res["ms_per_call"] = round(ms, 4)
        res["TFLOP/s"] = round(flops / (ms * 1e-3) / 1e12, 1)
    elif args.only == "alloc":
        # global sort-and-truncate: the decoder stack's 917,504-component pool (224
        # matrices, costs 8192 / 15104) and a 64M-component pool; one untimed and five
        # timed calls each, queued back to back, with the order (sort) and without it
        # (select)
        g = torch.Generator(device=dev)
        g.manual_seed(45)
        for m_items, n_mat in ((917504, 224), (64 * 1024 * 1024, 16384)):
            per = m_items // n_mat
            offs = torch.arange(0, m_items + 1, per, dtype=torch.int64, device=dev)
            cost = torch.where(torch.arange(n_mat, device=dev) % 7 < 4, 8192, 15104).to(torch.int64)
            scores = torch.rand(m_items, generator=g, device=dev)
            budget = int(0.6 * float((cost * per).sum()))
            for want, tag in ((True, ""), (False, "_no_order")):   # sort, then the order-free select
                lrc.lrc_allocate_ranks(scores, offs, cost, budget, want_order=want)
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                s.record()
                for _ in range(5):
                    lrc.lrc_allocate_ranks(scores, offs, cost, budget, want_order=want)
                e.record()
                torch.cuda.synchronize()
                res[f"ms_per_call_{m_items}{tag}"] = round(s.elapsed_time(e) / 5, 4)
            del offs, cost, scores
    elif args.only == "qaw":
        # int8-QAW activation covariance of the FFN pair's down projection: 131072 bf16
        # tokens x 11008 (per-token fake quantisation pre-pass, then the two-term SYRK into
        # the 11008 x 11008 sum); one untimed and two timed calls.  The stream's rotation is
        # drawn on the host: the device QR of an 11008 x 11008 matrix has crashed inside
        # the vendor solver under rocprofv3's counter collection.
        cs = synth.workload_spec("ffn_pair_11008x4096")
        a = synth.stream(cs, "a_down", device=dev, rotation_device="cpu")
        cov = torch.zeros(a.shape[1], a.shape[1], device=dev)
        lrc.lrc_accumulate_cov(a, cov, quant=True)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(2):
            lrc.lrc_accumulate_cov(a, cov, quant=True)
        e.record()
        torch.cuda.synchronize()
        res["tokens"], res["d"] = int(a.shape[0]), int(a.shape[1])
        res["ms_per_accumulation"] = round(s.elapsed_time(e) / 2, 4)
    elif args.only == "tridiag":
        # one covariance and one whitened decomposition of the attention projection
        a = synth.activation_stream(args.tokens, args.d, 1.0, 31, outlier_frac=0.01, dtype=torch.bfloat16,
                                    device=dev)
        w = synth.weight(args.d, args.d, 35, device=dev)
        cov = torch.zeros(args.d, args.d, device=dev)
        lrc.lrc_accumulate_cov(a, cov)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        _, _, _, info = lrc.lrc_whiten_decompose(w, args.rank, cov, args.tokens)
        torch.cuda.synchronize()
        res["decomposition_ms"] = round((time.perf_counter() - t0) * 1e3, 2)
        res["info"] = int(info[0])
    else:
        # decode-time FFN: low-rank and hybrid forms at 1 and 8 tokens, 20 untimed + 50 timed calls
        g = torch.Generator(device=dev)
        g.manual_seed(1)
        d, dff, rk = 4096, 11008, 2048
        nl = nd = dff // 2
        dense = (*_fac(torch, g, dev, nd, d), *_fac(torch, g, dev, nd, d), *_fac(torch, g, dev, d, nd))
        cases = [("lowrank", _ffn_factors(torch, g, dev, d, dff, rk), None),
                 ("hybrid", _ffn_factors(torch, g, dev, d, nl, rk), dense)]
        for name, (gate, up, down), dn in cases:
            for nt in (1, 8):
                x = torch.randn(nt, d, generator=g, device=dev)
                if dn is None:
                    def fn():
                        lrc.lrc_lowrank_ffn(x, gate, up, down)
                else:
                    def fn():
                        lrc.lrc_hybrid_ffn(x, gate, up, down, dn)
                for _ in range(20):
                    fn()
                torch.cuda.synchronize()
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record()
                for _ in range(50):
                    fn()
                e.record()
                torch.cuda.synchronize()
                res[f"{name}_{nt}tok_us"] = round(s.elapsed_time(e) / 50 * 1e3, 1)
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode (covariance sums would be "
              "all-reduced and matrices dealt out to GPUs; that layer is not built).", file=sys.stderr)
        sys.exit(2)
    # HIP gives a process 4 hardware queues unless GPU_MAX_HW_QUEUES says otherwise (read
    # when HIP initialises, so before torch touches the GPU).  The default stream takes one,
    # and streams beyond the queues share one and serialise.  Measured with one host thread
    # per stream: 3 streams on 4 queues 29.8 layers/s; on 8 queues 4 streams 32.6, 5 or 6
    # streams 16-19 (more queues active than the command processor serves at once).
    os.environ["GPU_MAX_HW_QUEUES"] = str(max(1, min(args.hw_queues, 32)))
    import torch

    import curvature_aware_rank_amd as lrc
    import synth

    dev = torch.device("cuda:0")
    if args.only:
        only(args, lrc, torch, dev)
        return
    d, n, r = args.d, args.tokens, args.rank
    a = synth.activation_stream(n, d, 1.0, 31, outlier_frac=0.01, dtype=torch.bfloat16, device=dev)
    w = synth.weight(d, d, 35, device=dev)
    if args.streams is None:
        args.streams = min(3, max(1, int(os.environ["GPU_MAX_HW_QUEUES"]) - 1))
    ns = max(1, args.streams)
    lpc = max(1, args.layers_per_call)
    streams = [torch.cuda.Stream() for _ in range(ns)]
    # per stream: one covariance buffer per layer of a call
    covs = [torch.empty(lpc, d, d, dtype=torch.float32, device=dev) for _ in range(ns)]
    cov = covs[0][0]
    wb = w.unsqueeze(0).expand(lpc, d, d).contiguous()
    offs = torch.tensor([0, d], dtype=torch.int64, device=dev)
    cost = torch.tensor([2 * d], dtype=torch.int64, device=dev)
    budget = r * 2 * d
    if args.copy_probe_mib:
        copy_probe(torch, dev, args.copy_probe_mib)
    torch.cuda.synchronize()

    def step(c=cov):
        c.zero_()
        lrc.lrc_accumulate_cov(a, c)
        sig, left, right, info = lrc.lrc_whiten_decompose(w, r, c, n)
        scores, _ = lrc.lrc_score_components(sigma=sig, mode="kfac")
        return lrc.lrc_allocate_ranks(scores, offs, cost, budget), info

    def layers(cs, g):
        """g whole steps (independent layers) in one decomposition call: each layer's
        tokens into its own covariance, the g whitened decompositions together (the
        tridiagonal reductions share their launches), then each layer's scores and
        allocation."""
        if g == 1:
            return step(cs[0])
        cs[:g].zero_()
        for j in range(g):
            lrc.lrc_accumulate_cov(a, cs[j])
        sig, left, right, info = lrc.lrc_whiten_decompose(wb[:g], r, cs[:g], n)
        out = None
        for j in range(g):
            scores, _ = lrc.lrc_score_components(sigma=sig[j].contiguous(), mode="kfac")
            out = lrc.lrc_allocate_ranks(scores, offs, cost, budget)
        return out, info

    def run_steps(k_steps, n_streams, per_call=1):
        """k_steps whole steps: stream i (its own covariance buffers; the layers are
        independent) runs steps i, i + n_streams, ..., per_call of them per decomposition
        call, enqueued by a host thread of its own (an enqueue blocks while the stream's
        hardware queue is full, which would starve the other streams if one thread fed
        them all); returns the last outputs of each."""
        last = {}

        def feed(i):
            torch.cuda.set_device(dev)
            mine = len(range(i, k_steps, n_streams))
            with torch.cuda.stream(streams[i]):
                for j0 in range(0, mine, per_call):
                    last[i] = layers(covs[i], min(per_call, mine - j0))

        if n_streams == 1:
            feed(0)
            return last
        with ThreadPoolExecutor(max_workers=n_streams) as ex:
            list(ex.map(feed, range(n_streams)))   # re-raises a failure of any thread
        return last

    progress("inputs resident")
    run_steps(max(args.warmup, ns * lpc), ns, lpc)
    torch.cuda.synchronize()
    # timed region: K whole steps issued round robin on the streams, nothing else queued;
    # the clock stops when every stream has drained
    t0 = time.perf_counter()
    last = run_steps(args.steps, ns, lpc)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    for out, info in last.values():
        assert int(info.max()) == 0 and int(info.min()) == 0 and int(out[4][0]) == 0
    n_kept = int(last[0][0][1][0])
    ms = 1e3 * elapsed / args.steps
    progress(f"{args.steps} steps on {ns} stream(s), {lpc} per call: {ms:.2f} ms per step")
    # the same K steps one after another on one stream: the latency of one layer
    t0 = time.perf_counter()
    run_steps(args.steps, 1)
    torch.cuda.synchronize()
    ms_one = 1e3 * (time.perf_counter() - t0) / args.steps
    progress(f"{args.steps} steps on one stream: {ms_one:.2f} ms per step")
    # the covariance alone: K accumulations back to back, timed with events around the loop
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s_ev.record()
    for _ in range(args.steps):
        lrc.lrc_accumulate_cov(a, cov)
    e_ev.record()
    torch.cuda.synchronize()
    cov_ms = s_ev.elapsed_time(e_ev) / args.steps
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
    progress("instrumented steps")

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
    tr = TRAFFIC.get(dom)
    dec_ms = ms_one - cov_ms   # one layer's own decomposition time (no other layer in flight)
    res = {
        "metric": METRIC,
        "value": round(1e3 / ms, 4),
        "unit": "layers/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "steps_in_flight": ns * lpc,
        "ms_per_step_one_stream": round(ms_one, 3),
        "value_one_stream": round(1e3 / ms_one, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16/f32/f64",
        "data": "synthetic",
        "config": {"workload": f"attention projection W {d}x{d} fp32, {n} bf16 calibration tokens "
                               f"(power-law spectrum, 1% outlier channels x20), activation-only whitening, rank {r}",
                   "tokens_per_layer": n, "d": d, "rank": r, "streams": ns, "layers_per_call": lpc,
                   "hw_queues": int(os.environ["GPU_MAX_HW_QUEUES"])},
        "cov_tokens_per_s": round(n / (cov_ms * 1e-3), 1),
        "cov_ms": round(cov_ms, 4),
        "cov_mfma_bf16_frac": round(n * d * (d + 1.0) / (cov_ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 4),
        "step_tokens_per_s": round(n * 1e3 / ms, 1),
        "n_kept": n_kept,
        "layer": {"decomposition_ms": round(dec_ms, 3), "algorithmic_flops": layer_flops(d, r),
                  "mfma_f32_frac": round(layer_flops(d, r) / (dec_ms * 1e-3) / 1e12 / PEAK_TFLOPS["f32"], 4),
                  "one_stage_tridiag_bytes": layer_bytes(d),
                  "hbm_frac": round(layer_bytes(d) / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "profiled_ms_per_step": round(prof_ms, 3),
        "roofline": {"bound": roof["bound"], "kernel": dom, "dtype": roof["dtype"],
                     "achieved": round(achieved, 3), "peak": roof["peak"], "unit": roof["unit"],
                     "frac": round(achieved / roof["peak"], 4), "traffic": tr["bytes"] if tr else None,
                     "traffic_kernel_source_commit": tr["kernel_source_commit"] if tr else None,
                     "avg_launch_ms": round(dk["total_ms"] / dk["launches"], 5),
                     "launches_per_step": dk["launches"] / args.steps},
        "kernels": kernels,
    }
    if not args.no_secondary:
        res["secondary"] = passes(lrc, torch, dev)
        # the decoder stack issues four calls per layer: four worker streams (the timed
        # steps' streams plus new ones up to four)
        workers = streams + [torch.cuda.Stream() for _ in range(max(0, 4 - len(streams)))]
        res["workloads"] = workloads(lrc, torch, dev, workers)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(d, n, r)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
