"""Timing driver for the decode-time FFN kernels: the low-rank SwiGLU FFN with int8 factors
(hidden 4096, FFN 11008, ranks 2048) and the hybrid form (5504 channels low-rank at ranks
2048, 5504 dense int8), each at 1 and 8 tokens, 20 untimed then 50 timed calls.  Prints
the mean time per call (HIP events); run it under rocprofv3 --kernel-trace --stats for
the per-kernel split, from the repository root."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

import torch  # noqa: E402

import curvature_aware_rank_amd as lrc  # noqa: E402

dev = torch.device("cuda:0")
g = torch.Generator(device=dev)
g.manual_seed(1)
d, dff, rk = 4096, 11008, 2048


def fac(rows, cols):
    return (torch.randint(-127, 128, (rows, cols), generator=g, device=dev, dtype=torch.int8),
            torch.rand(rows, generator=g, device=dev) * 0.004 + 0.001)


def timed(label, fn, nbytes):
    for _ in range(20):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(50):
        fn()
    e.record()
    torch.cuda.synchronize()
    us = s.elapsed_time(e) / 50 * 1e3
    print(f"{label}: {us:.1f} us per call, {nbytes / us / 1e3:.0f} GB/s of int8 weights", flush=True)


gate, up, down = (*fac(rk, d), *fac(dff, rk)), (*fac(rk, d), *fac(dff, rk)), (*fac(dff, rk), *fac(d, rk))
lr_bytes = 2.0 * rk * d + 3.0 * dff * rk + d * rk
for nt in (1, 8):
    x = torch.randn(nt, d, generator=g, device=dev)
    timed(f"lowrank_ffn {nt} tok", lambda: lrc.lrc_lowrank_ffn(x, gate, up, down), lr_bytes)
del gate, up, down
nl = nd = dff // 2
gate, up, down = (*fac(rk, d), *fac(nl, rk)), (*fac(rk, d), *fac(nl, rk)), (*fac(nl, rk), *fac(d, rk))
dense = (*fac(nd, d), *fac(nd, d), *fac(d, nd))
hy_bytes = 2.0 * rk * d + 3.0 * nl * rk + d * rk + 3.0 * nd * d
for nt in (1, 8):
    x = torch.randn(nt, d, generator=g, device=dev)
    timed(f"hybrid_ffn {nt} tok", lambda: lrc.lrc_hybrid_ffn(x, gate, up, down, dense), hy_bytes)
