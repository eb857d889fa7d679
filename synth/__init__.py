"""Seeded synthetic inputs shared by the GPU path's tests, the oracle's tests and the benchmark.

This module holds random draws only, none of the decomposition's arithmetic.  The
shapes stand in for the LLaMA-class projections the pages evaluate on (hidden size
4096, FFN size 11008, 32 layers, 32 heads of 128) and for their calibration sets:

* a calibration stream is ``A = (Z * sqrt(lam)) @ Q^T`` with ``Z ~ N(0, 1)`` of shape
  tokens x d, ``lam_i = i^-p`` (a power-law covariance spectrum) and ``Q`` a Haar
  rotation (QR of a Gaussian matrix, column signs fixed by ``diag(R)``);
* optional outlier channels: ``round(frac * d)`` columns, picked by a seeded
  permutation, multiplied by ``outlier_scale`` after the rotation;
* optional per-layer scale ``c``: the stream is multiplied by ``sqrt(c)`` so that its
  covariance scales by ``c``;
* the stream is rounded to the requested dtype (bf16 with round-to-nearest-even);
* a weight is ``W ~ N(0, 1/d_in)`` in fp32, stored out x in (``y = W x``).

Every draw takes an explicit seed.  Generation runs on the device given (torch), so
the largest streams are drawn on the GPU; callers that feed the oracle copy the very
same bytes to the host.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

__all__ = [
    "haar_rotation", "activation_stream", "weight", "WORKLOADS", "LayerSpec",
    "workload_spec", "layer_scale",
]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=str(torch.device(device)))
    g.manual_seed(int(seed) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def haar_rotation(d: int, seed: int, device="cpu") -> torch.Tensor:
    """d x d orthogonal matrix, Haar-distributed (QR of a Gaussian, sign-fixed)."""
    z = torch.randn(d, d, generator=_gen(seed, device), device=device, dtype=torch.float32)
    q, r = torch.linalg.qr(z)
    sgn = torch.sign(torch.diagonal(r))
    sgn[sgn == 0] = 1
    return q * sgn.unsqueeze(0)


def activation_stream(n: int, d: int, exponent: float, seed: int, *, outlier_frac: float = 0.0,
                      outlier_scale: float = 20.0, scale: float = 1.0,
                      dtype=torch.bfloat16, device="cpu", block: int = 8192,
                      rotation_device=None) -> torch.Tensor:
    """Token-major calibration matrix (n x d) with a power-law covariance spectrum.
    ``rotation_device`` draws the rotation elsewhere (the host, say) and moves it to
    ``device``; the draw then differs from one made on ``device``."""
    q = haar_rotation(d, seed, rotation_device or device).to(device)
    lam_sqrt = torch.arange(1, d + 1, dtype=torch.float64).pow(-0.5 * exponent)
    lam_sqrt = lam_sqrt.to(device=device, dtype=torch.float32)
    g = _gen(seed + 1, device)
    n_out = int(round(outlier_frac * d))
    cols = None
    if n_out > 0:
        perm = torch.randperm(d, generator=_gen(seed + 2, "cpu"))
        cols = perm[:n_out].sort().values.to(device)
    out = torch.empty(n, d, dtype=dtype, device=device)
    qt = q.t().contiguous()
    amp = math.sqrt(scale)
    for t0 in range(0, n, block):
        tb = min(block, n - t0)
        z = torch.randn(tb, d, generator=g, device=device, dtype=torch.float32)
        a = (z * lam_sqrt) @ qt
        if cols is not None:
            a[:, cols] *= outlier_scale
        if amp != 1.0:
            a *= amp
        out[t0:t0 + tb] = a.to(dtype)
    return out


def weight(d_out: int, d_in: int, seed: int, device="cpu") -> torch.Tensor:
    """fp32 weight, out x in, entries N(0, 1/d_in)."""
    w = torch.randn(d_out, d_in, generator=_gen(seed, device), device=device, dtype=torch.float32)
    return w * (1.0 / math.sqrt(d_in))


def layer_scale(layer: int, seed: int) -> float:
    """Per-layer covariance scale c_l = 10^U(-1, 1) (a x0.1 .. x10 spread)."""
    g = _gen(seed * 1000 + layer, "cpu")
    u = torch.rand(1, generator=g, dtype=torch.float64).item()
    return 10.0 ** (2.0 * u - 1.0)


@dataclass
class LayerSpec:
    """One weight matrix of a workload: its shape and the streams that calibrate it."""
    name: str
    d_out: int
    d_in: int
    a_stream: str            # key of the activation stream (width d_in)
    b_stream: str | None     # key of the gradient stream (width d_out), None if none
    two_sided: bool          # whiten with G as well as X


@dataclass
class WorkloadSpec:
    name: str
    workload: str
    n_tokens: int
    rank: int | None               # fixed rank per matrix (None: allocation decides)
    rank_ratio: float | None
    budget_fraction: float | None  # global budget as a fraction of dense parameters
    dtype: torch.dtype
    qaw: bool
    streams: dict = field(default_factory=dict)   # key -> (width, exponent, outlier_frac, seed)
    matrices: list = field(default_factory=list)  # LayerSpec
    heads: int = 0
    head_dim: int = 0


WORKLOADS = {
    "single_layer_256": "single linear layer 256x256 fp32, two-sided K-FAC whitening, 4096 tokens, rank 64",
    "attention_projection_4096": "attention projection 4096x4096, 65536 bf16 tokens, activation-only whitening, rank 1024",
    "ffn_pair_11008x4096": "FFN pair up 11008x4096 / down 4096x11008, 131072 bf16 tokens, two-sided, int8 QAW, rank ratio 0.5",
    "decoder_stack_32_layers": "32-layer decoder stack (224 matrices), 32768 tokens per layer, Fisher scores, 60% budget",
    "kv_heads_64x128x4096": "K/V per-head 128x4096 slices (64 heads), 65536 bf16 tokens, 40% budget",
}


def workload_spec(name: str, n_tokens: int | None = None, seed: int = 1234) -> WorkloadSpec:
    """Shapes and stream recipes of the five workloads (n_tokens may be shrunk for tests)."""
    if name == "single_layer_256":
        n = n_tokens or 4096
        cs = WorkloadSpec("single_layer_256", WORKLOADS["single_layer_256"], n, 64, None, None, torch.float32, False)
        cs.streams = {"a": (256, 1.2, 0.0, seed + 11), "b": (256, 1.2, 0.0, seed + 23)}
        cs.matrices = [LayerSpec("w", 256, 256, "a", "b", True)]
    elif name == "attention_projection_4096":
        n = n_tokens or 65536
        cs = WorkloadSpec("attention_projection_4096", WORKLOADS["attention_projection_4096"], n, 1024, None, None, torch.bfloat16, False)
        cs.streams = {"a": (4096, 1.0, 0.01, seed + 31)}
        cs.matrices = [LayerSpec("w", 4096, 4096, "a", None, False)]
    elif name == "ffn_pair_11008x4096":
        n = n_tokens or 131072
        cs = WorkloadSpec("ffn_pair_11008x4096", WORKLOADS["ffn_pair_11008x4096"], n, None, 0.5, None, torch.bfloat16, True)
        cs.streams = {"a_up": (4096, 1.0, 0.01, seed + 41), "b_up": (11008, 1.5, 0.0, seed + 43),
                      "a_down": (11008, 1.0, 0.01, seed + 47), "b_down": (4096, 1.5, 0.0, seed + 53)}
        cs.matrices = [LayerSpec("up", 11008, 4096, "a_up", "b_up", True),
                       LayerSpec("down", 4096, 11008, "a_down", "b_down", True)]
    elif name == "decoder_stack_32_layers":
        n = n_tokens or 32768
        cs = WorkloadSpec("decoder_stack_32_layers", WORKLOADS["decoder_stack_32_layers"], n, None, None, 0.6, torch.bfloat16, False)
        # per layer; the layer index is folded into the seeds by the caller
        cs.streams = {"attn_in": (4096, 1.0, 0.0, seed + 61), "o_in": (4096, 1.0, 0.0, seed + 67),
                      "mlp_in": (4096, 1.0, 0.0, seed + 71), "down_in": (11008, 1.0, 0.0, seed + 73),
                      "g_q": (4096, 1.5, 0.0, seed + 79), "g_k": (4096, 1.5, 0.0, seed + 83),
                      "g_v": (4096, 1.5, 0.0, seed + 89), "g_o": (4096, 1.5, 0.0, seed + 97),
                      "g_gate": (11008, 1.5, 0.0, seed + 101), "g_up": (11008, 1.5, 0.0, seed + 103),
                      "g_down": (4096, 1.5, 0.0, seed + 107)}
        cs.matrices = [LayerSpec("q", 4096, 4096, "attn_in", "g_q", False),
                       LayerSpec("k", 4096, 4096, "attn_in", "g_k", False),
                       LayerSpec("v", 4096, 4096, "attn_in", "g_v", False),
                       LayerSpec("o", 4096, 4096, "o_in", "g_o", False),
                       LayerSpec("gate", 11008, 4096, "mlp_in", "g_gate", False),
                       LayerSpec("up", 11008, 4096, "mlp_in", "g_up", False),
                       LayerSpec("down", 4096, 11008, "down_in", "g_down", False)]
    elif name == "kv_heads_64x128x4096":
        n = n_tokens or 65536
        cs = WorkloadSpec("kv_heads_64x128x4096", WORKLOADS["kv_heads_64x128x4096"], n, None, None, 0.4, torch.bfloat16, False)
        cs.streams = {"a": (4096, 1.0, 0.01, seed + 131)}
        cs.matrices = [LayerSpec("k", 4096, 4096, "a", None, False),
                       LayerSpec("v", 4096, 4096, "a", None, False)]
        cs.heads, cs.head_dim = 32, 128
    else:
        raise ValueError(f"no workload {name!r}")
    return cs


def stream(cs: WorkloadSpec, key: str, *, layer: int = 0, device="cpu", n_tokens: int | None = None,
           width: int | None = None, rotation_device=None) -> torch.Tensor:
    """Draw one calibration stream of a workload (layer folds into the seed for the stack)."""
    d, p, frac, sd = cs.streams[key]
    d = width or d
    scale = layer_scale(layer, sd) if (cs.name == "decoder_stack_32_layers" and not key.startswith("g_")) else 1.0
    return activation_stream(n_tokens or cs.n_tokens, d, p, sd + 7919 * layer, outlier_frac=frac,
                             scale=scale, dtype=cs.dtype, device=device, rotation_device=rotation_device)
