"""Python binding of liblrc (argument marshalling only).

Every computation runs in the HIP kernels of liblrc.so; this module checks tensor
shapes, dtypes and devices, allocates device workspace with torch, passes raw device
pointers and torch's current HIP stream, and turns status codes into exceptions.  There
is no fallback: if liblrc.so is missing or no GPU is present the calls raise.

Like the library, the binding never waits for the GPU: failures the kernels find are
reported in the returned device `info` tensors, which the caller reads after its own
synchronisation.  Every tensor whose pointer is passed (contiguous copies included) is
held in a local variable until the C call has returned, so the caching allocator cannot
hand its memory to another tensor while the enqueued kernels may still read it.

Names match the C ABI in include/lrc.h.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LRC_OK", "LRC_EINVAL", "LRC_EDTYPE", "LRC_EWORKSPACE", "LRC_EHIP", "LRC_ENOTPD",
    "LRC_ENOCONV", "LRC_ENONFINITE", "LRC_F32", "LRC_BF16", "LRC_COV_QUANT_INT8_TOKEN",
    "LRC_SCORE_FISHER", "LRC_SCORE_KFAC", "LRC_RANKSCORE_UNIRANK", "LRC_RANKSCORE_SWIFT", "LrcError", "lib",
    "library_path", "lrc_accumulate_cov", "lrc_whiten_decompose", "lrc_score_components", "lrc_allocate_ranks",
    "lrc_rank_scores", "lrc_rotate_quantize", "lrc_quantize_rows", "lrc_lowrank_ffn", "lrc_ffn_select_channels",
    "lrc_hybrid_ffn",
    "lrc_status_string", "lrc_profile_start", "lrc_profile_stop", "lrc_profile_kernels",
]

LRC_OK, LRC_EINVAL, LRC_EDTYPE, LRC_EWORKSPACE, LRC_EHIP, LRC_ENOTPD, LRC_ENOCONV, LRC_ENONFINITE = range(8)
LRC_F32, LRC_BF16 = 0, 1
LRC_COV_QUANT_INT8_TOKEN = 0x1
LRC_SCORE_FISHER = 0x1
LRC_SCORE_KFAC = 0x2
LRC_RANKSCORE_UNIRANK = 0x1
LRC_RANKSCORE_SWIFT = 0x2

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "liblrc.so")

_i64, _u32, _sz, _vp, _i32 = ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int

_SIGS = {
    "lrc_accumulate_cov": (_i32, [_vp, _i32, _i64, _i64, _i64, _vp, _i64, _u32, _vp, _vp, _sz, _vp]),
    "lrc_accumulate_cov_workspace": (_sz, [_i32, _i64, _i64, _u32]),
    "lrc_whiten_decompose": (_i32, [_vp, _i64, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64,
                                    _i64, ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "lrc_whiten_decompose_workspace": (_sz, [_i64, _i64, _i64, _i64, _i32, _i32]),
    "lrc_whiten_decompose_strided": (_i32, [_vp, _i64, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _vp, _i64,
                                            _i64, _i64, _i64, ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "lrc_whiten_decompose_strided_workspace": (_sz, [_i64, _i64, _i64, _i64, _i64, _i64]),
    "lrc_score_components": (_i32, [_vp, _vp, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _u32, _i32, _i32,
                                    _i64, _vp, _vp, _vp, _sz, _vp]),
    "lrc_score_components_workspace": (_sz, [_i64, _i64, _i64, _i64, _u32]),
    "lrc_allocate_ranks": (_i32, [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "lrc_allocate_ranks_workspace": (_sz, [_i64, _i64]),
    "lrc_allocate_ranks_noalloc": (_i32, [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "lrc_allocate_ranks_noalloc_max_items": (_i64, []),
    "lrc_rank_scores": (_i32, [_vp, _vp, _i64, _i64, _vp, ctypes.c_float, _u32, _vp, _vp, _vp]),
    "lrc_rotate_quantize": (_i32, [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "lrc_rotate_quantize_workspace": (_sz, [_i64, _i64, _i64]),
    "lrc_quantize_rows": (_i32, [_vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "lrc_lowrank_ffn": (_i32, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _i64,
                               _vp, _vp, _vp, _vp, _i64, _vp, _vp, _sz, _vp]),
    "lrc_lowrank_ffn_workspace": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "lrc_ffn_select_channels": (_i32, [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _vp, _i64, _i64,
                                       ctypes.c_float, _i64, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "lrc_ffn_select_channels_workspace": (_sz, [_i64, _i64]),
    "lrc_hybrid_ffn": (_i32, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _vp, _vp,
                              _vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "lrc_hybrid_ffn_workspace": (_sz, [_i64, _i64, _i64, _i64, _i64, _i64]),
    "lrc_status_string": (ctypes.c_char_p, [_i32]),
    "lrc_last_hip_error": (_i32, []),
    "lrc_profile_start": (_i32, []),
    "lrc_profile_stop": (_i32, []),
    "lrc_profile_kernels": (_i32, []),
    "lrc_profile_kernel": (_i32, [_i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(_i64),
                                  ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                  ctypes.POINTER(ctypes.c_double)]),
}


def _load():
    if not os.path.exists(library_path):
        raise ImportError(f"liblrc.so not built at {library_path}; run python curvature_aware_rank_amd/build.py")
    so = ctypes.CDLL(library_path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(so, name)
        fn.restype = res
        fn.argtypes = args
    return so


lib = _load()


class LrcError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib.lrc_status_string(status).decode()
        if status == LRC_EHIP:
            msg += f" (hipError {lib.lrc_last_hip_error()})"
        super().__init__(f"{where}: {msg}")
        self.status = status


def lrc_status_string(status: int) -> str:
    return lib.lrc_status_string(status).decode()


def _check(status: int, where: str):
    if status != LRC_OK:
        raise LrcError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _tensor(t, name, dtype, shape, device=None):
    """Check a GPU tensor's dtype, shape (None entries are free) and device; return it."""
    _dev(t, name)
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if len(shape) != t.dim() or any(want is not None and want != got for want, got in zip(shape, t.shape)):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    return t


def _info(info, device):
    """An optional caller-given int32 (1,) flag on `device`, or a fresh one set to 0."""
    if info is None:
        return torch.zeros(1, dtype=torch.int32, device=device)
    return _tensor(info, "info", torch.int32, (1,), device)


def _workspace(nbytes: int, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return LRC_BF16
    if t.dtype == torch.float32:
        return LRC_F32
    raise ValueError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _rowmajor_ld(t, name):
    if t.dim() != 2 or t.stride(1) != 1 or t.stride(0) < t.shape[1]:
        raise ValueError(f"{name} must be a row-major 2-D tensor")
    return t.stride(0)


def lrc_accumulate_cov(A: torch.Tensor, C: torch.Tensor, quant: bool = False, info=None):
    """C[lower] += sum_t a_t^T a_t over the rows of A (fake-quantised per token if quant).

    info: optional int32 (1,) device flag (sticky LRC_ENONFINITE); a fresh zeroed one is
    made otherwise.  Returns the flag (read it after synchronising)."""
    _dev(A, "A")
    if A.dim() != 2:
        raise ValueError("A must be (n_tokens, d)")
    n, d = A.shape
    _tensor(C, "C", torch.float32, (d, d), A.device)
    lda = _rowmajor_ld(A, "A")
    ldc = _rowmajor_ld(C, "C")
    dt = _dtype_code(A)
    info = _info(info, A.device)
    flags = LRC_COV_QUANT_INT8_TOKEN if quant else 0
    ws = _workspace(lib.lrc_accumulate_cov_workspace(dt, n, d, flags), A.device)
    _check(lib.lrc_accumulate_cov(_ptr(A), dt, n, d, lda, _ptr(C), ldc, flags, _ptr(info), _ptr(ws), ws.numel(),
                                  _stream()), "lrc_accumulate_cov")
    return info


def lrc_whiten_decompose(W: torch.Tensor, rank: int, Xsum=None, n_x: int = 0, Gsum=None, n_g: int = 0,
                         damping: float = 0.0):
    """Whitened truncated decomposition.  W: (d_out, d_in) or (batch, d_out, d_in) fp32;
    Xsum (d_in, d_in) and Gsum (d_out, d_out) fp32 sums shared by the batch, or
    (batch, d_in, d_in) / (batch, d_out, d_out) with one sum per slice (independent
    layers; the token counts n_x, n_g are common), or None for identity.

    Returns (sigma, left, right, info): sigma (batch, k), left (batch, d_out, r),
    right (batch, r, d_in), info (batch,) int32 -- batch dim dropped for 2-D W.  A
    covariance that is not positive definite or an eigensolver at its sweep cap is
    reported in info only (the call does not wait for the GPU)."""
    _dev(W, "W")
    if W.dtype != torch.float32:
        raise ValueError("W must be fp32")
    squeeze = W.dim() == 2
    W3 = W.unsqueeze(0) if squeeze else W
    if W3.dim() != 3 or W3.stride(2) != 1:
        raise ValueError("W must be (d_out, d_in) or (batch, d_out, d_in), row-major")
    batch, d_out, d_in = W3.shape
    ldw, sw = W3.stride(1), W3.stride(0)
    k = min(d_out, d_in)
    dev = W.device
    sigma = torch.empty(batch, k, dtype=torch.float32, device=dev)
    left = torch.empty(batch, d_out, rank, dtype=torch.float32, device=dev)
    right = torch.empty(batch, rank, d_in, dtype=torch.float32, device=dev)
    info = torch.empty(batch, dtype=torch.int32, device=dev)
    def cov_arg(S, name, dim):
        """(pointer tensor, leading dim, slice stride, slices) of a covariance argument"""
        if S is None:
            return None, 0, 0, 0
        if S.dim() == 3 and squeeze:
            raise ValueError(f"{name}: one sum per slice needs a batched W")
        if S.dim() == 3:
            _tensor(S, name, torch.float32, (batch, dim, dim), dev)
            if S.stride(2) != 1 or S.stride(1) < dim or S.stride(0) < dim * S.stride(1):
                raise ValueError(f"{name} must be row-major slices")
            return S, S.stride(1), S.stride(0), batch
        _tensor(S, name, torch.float32, (dim, dim), dev)
        return S, _rowmajor_ld(S, name), 0, 1

    Xs, ldx, sx, nxs = cov_arg(Xsum, "Xsum", d_in)
    Gs, ldg, sg, ngs = cov_arg(Gsum, "Gsum", d_out)
    nb = lib.lrc_whiten_decompose_strided_workspace(d_out, d_in, batch, rank, nxs, ngs)
    ws = _workspace(nb, dev)
    st = lib.lrc_whiten_decompose_strided(_ptr(W3), d_out, d_in, ldw, batch, sw, _ptr(Xs), ldx, sx, int(n_x),
                                          _ptr(Gs), ldg, sg, int(n_g), int(rank), float(damping), _ptr(sigma),
                                          _ptr(left), _ptr(right), _ptr(info), _ptr(ws), ws.numel(), _stream())
    _check(st, "lrc_whiten_decompose")
    if squeeze:
        return sigma[0], left[0], right[0], info
    return sigma, left, right, info


def lrc_score_components(left=None, right=None, sigma=None, A=None, B=None, mode: str = "fisher",
                         scores=None, accumulate: bool = False, finalize: bool = True, n_total=None, info=None):
    """Per-component scores; returns (scores (k,) fp32, info int32 (1,)).

    mode="fisher": needs left (d_out, k), right (k, d_in) fp32, A (n, d_in), B (n, d_out)
    (both bf16 or both fp32).  mode="kfac": needs sigma (k,) fp32 only.  info: optional
    int32 (1,) device flag that receives LRC_ENONFINITE when a score is NaN/Inf (sticky
    over a chunked stream); a fresh zeroed one is made otherwise."""
    if mode == "kfac":
        _dev(sigma, "sigma")
        if sigma.dtype != torch.float32 or sigma.dim() != 1:
            raise ValueError("sigma must be a 1-D fp32 tensor")
        sig = sigma.contiguous()
        k = sig.numel()
        dev = sig.device
        if scores is None:
            scores = torch.empty(k, dtype=torch.float32, device=dev)
        _tensor(scores, "scores", torch.float32, (k,), dev)
        info = _info(info, dev)
        _check(lib.lrc_score_components(None, None, LRC_F32, 0, 1, 1, None, None, _ptr(sig), k,
                                        LRC_SCORE_KFAC, 0, 1, 1, _ptr(scores), _ptr(info), None, 0, _stream()),
               "lrc_score_components")
        return scores, info
    if mode != "fisher":
        raise ValueError("mode is 'fisher' or 'kfac'")
    _dev(left, "left")
    if left.dim() != 2:
        raise ValueError("left must be (d_out, k)")
    d_out, k = left.shape
    dev = left.device
    _tensor(left, "left", torch.float32, (d_out, k), dev)
    _tensor(right, "right", torch.float32, (k, None), dev)
    d_in = right.shape[1]
    _dev(A, "A")
    _dev(B, "B")
    if A.dim() != 2:
        raise ValueError("A must be (n, d_in)")
    n = A.shape[0]
    _tensor(A, "A", A.dtype, (n, d_in), dev)
    _tensor(B, "B", A.dtype, (n, d_out), dev)
    dt = _dtype_code(A)
    if scores is None:
        scores = torch.empty(k, dtype=torch.float32, device=dev)
    _tensor(scores, "scores", torch.float32, (k,), dev)
    info = _info(info, dev)
    # contiguous copies (if any) stay referenced until the call has returned
    a, b, lf, rt = A.contiguous(), B.contiguous(), left.contiguous(), right.contiguous()
    ws = _workspace(lib.lrc_score_components_workspace(n, d_in, d_out, k, LRC_SCORE_FISHER), dev)
    _check(lib.lrc_score_components(_ptr(a), _ptr(b), dt, n, d_in, d_out, _ptr(lf), _ptr(rt), None, k,
                                    LRC_SCORE_FISHER, int(accumulate), int(finalize), int(n_total or n),
                                    _ptr(scores), _ptr(info), _ptr(ws), ws.numel(), _stream()), "lrc_score_components")
    return scores, info


def lrc_allocate_ranks(scores: torch.Tensor, offsets: torch.Tensor, cost: torch.Tensor, budget: int,
                       want_order: bool = True):
    """Global sort-and-truncate.  scores: (M,) fp32; offsets: (n_mat+1,) int64; cost: (n_mat,) int64.

    Returns (order int32 (M,), n_kept int64 (1,), ranks int32 (n_mat,), kept_mask uint8 (M,), info int32 (1,)).
    With want_order=False the library selects the cut without sorting (the same n_kept,
    ranks and mask) and order is None."""
    _dev(scores, "scores")
    dev = scores.device
    n_mat = cost.numel() if isinstance(cost, torch.Tensor) else 0
    _tensor(scores, "scores", torch.float32, (None,), dev)
    _tensor(offsets, "offsets", torch.int64, (n_mat + 1,), dev)
    _tensor(cost, "cost", torch.int64, (n_mat,), dev)
    M = scores.numel()
    sc, offs, cst = scores.contiguous(), offsets.contiguous(), cost.contiguous()
    order = torch.empty(M, dtype=torch.int32, device=dev) if want_order else None
    n_kept = torch.empty(1, dtype=torch.int64, device=dev)
    ranks = torch.empty(n_mat, dtype=torch.int32, device=dev)
    kept = torch.empty(M, dtype=torch.uint8, device=dev)
    info = torch.empty(1, dtype=torch.int32, device=dev)
    ws = _workspace(lib.lrc_allocate_ranks_workspace(n_mat, M), dev)
    _check(lib.lrc_allocate_ranks(_ptr(sc), _ptr(offs), _ptr(cst), n_mat, M, int(budget),
                                  _ptr(order) if want_order else None, _ptr(n_kept),
                                  _ptr(ranks), _ptr(kept), _ptr(info), _ptr(ws), ws.numel(), _stream()),
           "lrc_allocate_ranks")
    return order, n_kept, ranks, kept, info


def lrc_rank_scores(sigma: torch.Tensor, offsets: torch.Tensor, weight: torch.Tensor, mode: str = "unirank",
                    alpha: float = 0.5):
    """Alternative component scores from singular values.  sigma: (M,) fp32, matrices
    concatenated per offsets ((n_mat+1,) int64); weight: (n_mat,) fp32 -- the layer
    importance I_l (mode "unirank") or beta_l (mode "swift", with alpha).

    Returns (scores fp32 (M,), info int32 (1,))."""
    _dev(sigma, "sigma")
    dev = sigma.device
    n_mat = weight.numel() if isinstance(weight, torch.Tensor) else 0
    _tensor(sigma, "sigma", torch.float32, (None,), dev)
    _tensor(offsets, "offsets", torch.int64, (n_mat + 1,), dev)
    _tensor(weight, "weight", torch.float32, (n_mat,), dev)
    flag = {"unirank": LRC_RANKSCORE_UNIRANK, "swift": LRC_RANKSCORE_SWIFT}[mode]
    M = sigma.numel()
    sig, offs, wgt = sigma.contiguous(), offsets.contiguous(), weight.contiguous()
    scores = torch.empty(M, dtype=torch.float32, device=dev)
    info = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib.lrc_rank_scores(_ptr(sig), _ptr(offs), n_mat, M, _ptr(wgt), float(alpha), flag, _ptr(scores),
                               _ptr(info), _stream()), "lrc_rank_scores")
    return scores, info


def lrc_rotate_quantize(left: torch.Tensor, right: torch.Tensor, signs: torch.Tensor, keep_rotated: bool = False):
    """Rotate the factors by a sign-randomised Hadamard matrix and quantise each row to
    int8.  left: (d_out, r) fp32, right: (r, d_in) fp32, signs: (r,) fp32 of +-1.

    Returns (q_left int8, s_left fp32, q_right int8, s_right fp32) and, with
    keep_rotated, the rotated fp32 factors as two more entries."""
    _dev(left, "left")
    if left.dim() != 2:
        raise ValueError("left must be (d_out, r)")
    d_out, r = left.shape
    dev = left.device
    _tensor(left, "left", torch.float32, (d_out, r), dev)
    _tensor(right, "right", torch.float32, (r, None), dev)
    _tensor(signs, "signs", torch.float32, (r,), dev)
    d_in = right.shape[1]
    lf, rt, sg = left.contiguous(), right.contiguous(), signs.contiguous()
    ql = torch.empty(d_out, r, dtype=torch.int8, device=dev)
    sl = torch.empty(d_out, dtype=torch.float32, device=dev)
    qr = torch.empty(r, d_in, dtype=torch.int8, device=dev)
    sr = torch.empty(r, dtype=torch.float32, device=dev)
    lrot = torch.empty(d_out, r, dtype=torch.float32, device=dev) if keep_rotated else None
    rrot = torch.empty(r, d_in, dtype=torch.float32, device=dev) if keep_rotated else None
    ws = _workspace(lib.lrc_rotate_quantize_workspace(d_out, r, d_in), dev)
    _check(lib.lrc_rotate_quantize(_ptr(lf), _ptr(rt), d_out, r, d_in, _ptr(sg), _ptr(ql), _ptr(sl), _ptr(qr), _ptr(sr),
                                   _ptr(lrot) if keep_rotated else None, _ptr(rrot) if keep_rotated else None,
                                   _ptr(ws), ws.numel(), _stream()), "lrc_rotate_quantize")
    return (ql, sl, qr, sr, lrot, rrot) if keep_rotated else (ql, sl, qr, sr)


def lrc_quantize_rows(x: torch.Tensor):
    """Per-row int8 RTN of an fp32 matrix (rows, cols).  Returns (q int8, scale fp32 (rows,))."""
    _dev(x, "x")
    if x.dtype != torch.float32 or x.dim() != 2:
        raise ValueError("x must be a 2-D fp32 tensor")
    x = x.contiguous()
    rows, cols = x.shape
    q = torch.empty(rows, cols, dtype=torch.int8, device=x.device)
    s = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check(lib.lrc_quantize_rows(_ptr(x), rows, cols, cols, _ptr(q), _ptr(s), _stream()), "lrc_quantize_rows")
    return q, s


def lrc_ffn_select_channels(w_gate: torch.Tensor, w_up: torch.Tensor, gate_factors, up_factors,
                            Xsum: torch.Tensor, n_x: int, n_lowrank: int, damping: float = 0.0):
    """Hidden-channel selection of an FFN's hybrid low-rank form.  w_gate, w_up: (d_ff, d)
    fp32; gate_factors, up_factors: (left (d_ff, r), right (r, d)) fp32 from
    lrc_whiten_decompose with the same Xsum (or None for r = 0); Xsum: (d, d) fp32 sum.

    Returns (err fp64 (d_ff,), order int32 (d_ff,), lowrank uint8 (d_ff,), info int32 (1,))."""
    _dev(w_gate, "w_gate")
    if w_gate.dim() != 2:
        raise ValueError("w_gate must be (d_ff, d)")
    d_ff, d = w_gate.shape
    dev = w_gate.device
    _tensor(w_gate, "w_gate", torch.float32, (d_ff, d), dev)
    _tensor(w_up, "w_up", torch.float32, (d_ff, d), dev)
    _tensor(Xsum, "Xsum", torch.float32, (d, d), dev)
    wg, wu = w_gate.contiguous(), w_up.contiguous()
    r = 0
    fac = []
    if gate_factors is not None or up_factors is not None:
        for pair, nm in ((gate_factors, "gate"), (up_factors, "up")):
            if pair is None:
                raise ValueError("give the factors of both gate and up, or of neither")
            left, right = pair
            _tensor(left, f"{nm} left", torch.float32, (d_ff, None), dev)
            _tensor(right, f"{nm} right", torch.float32, (None, d), dev)
            fac += [left.contiguous(), right.contiguous()]
        r = fac[0].shape[1]
        if any(tuple(f.shape) != shp for f, shp in zip(fac, [(d_ff, r), (r, d)] * 2)):
            raise ValueError("factors must be left (d_ff, r) and right (r, d) for both")
    err = torch.empty(d_ff, dtype=torch.float64, device=dev)
    order = torch.empty(d_ff, dtype=torch.int32, device=dev)
    lowrank = torch.empty(d_ff, dtype=torch.uint8, device=dev)
    info = torch.empty(1, dtype=torch.int32, device=dev)
    ws = _workspace(lib.lrc_ffn_select_channels_workspace(d_ff, d), dev)
    ptrs = [_ptr(f) for f in fac] if r > 0 else [None] * 4
    _check(lib.lrc_ffn_select_channels(_ptr(wg), _ptr(wu), d_ff, d, d, ptrs[0], ptrs[1], ptrs[2], ptrs[3], r,
                                       _ptr(Xsum), _rowmajor_ld(Xsum, "Xsum"), int(n_x), float(damping),
                                       int(n_lowrank), _ptr(err), _ptr(order), _ptr(lowrank), _ptr(info), _ptr(ws),
                                       ws.numel(), _stream()), "lrc_ffn_select_channels")
    return err, order, lowrank, info


def _lowrank_factors(gate, up, down, d, dev):
    """Check the int8 factor sets of a low-rank FFN (shapes, dtypes, device) and return
    contiguous copies plus (d_ff, rg, ru, rd)."""
    i8, f32 = torch.int8, torch.float32
    for t in [*gate, *up, *down]:
        _dev(t, "ffn factor")
    if len(gate) != 4 or len(up) != 4 or len(down) != 4:
        raise ValueError("gate, up and down are 4-tuples (q_R, s_R, q_L, s_L)")
    rg, ru = gate[0].shape[0], up[0].shape[0]
    d_ff = gate[2].shape[0]
    rd = down[0].shape[1]
    for (q_r, s_r, q_l, s_l), r, nm in ((gate, rg, "gate"), (up, ru, "up")):
        _tensor(q_r, f"{nm} q_R", i8, (r, d), dev)
        _tensor(s_r, f"{nm} s_R", f32, (r,), dev)
        _tensor(q_l, f"{nm} q_L", i8, (d_ff, r), dev)
        _tensor(s_l, f"{nm} s_L", f32, (d_ff,), dev)
    _tensor(down[0], "down q_Rt", i8, (d_ff, rd), dev)
    _tensor(down[1], "down s_R", f32, (rd,), dev)
    _tensor(down[2], "down q_L", i8, (d, rd), dev)
    _tensor(down[3], "down s_L", f32, (d,), dev)
    return ([t.contiguous() for t in gate], [t.contiguous() for t in up], [t.contiguous() for t in down],
            d_ff, rg, ru, rd)


def lrc_hybrid_ffn(x: torch.Tensor, gate=None, up=None, down=None, dense=None):
    """Hybrid FFN forward: hidden channels [0, n_lr) low-rank (gate, up, down as for
    lrc_lowrank_ffn, or all None when n_lr = 0), the next n_dense dense:
    dense = (q_gd (n_dense, d) int8, s_gd (n_dense,), q_ud, s_ud, q_dd (d, n_dense) int8 --
    W_down's dense columns as rows, s_dd (d,)), or None when n_dense = 0.
    Returns y (n_tok, d) fp32."""
    _dev(x, "x")
    if x.dtype != torch.float32 or x.dim() != 2:
        raise ValueError("x must be (n_tok, d) fp32")
    n_tok, d = x.shape
    dev = x.device
    xc = x.contiguous()
    lr = gate is not None
    if lr != (up is not None) or lr != (down is not None):
        raise ValueError("give gate, up and down together, or none of them")
    if lr:
        g, u, dn, n_lr, rg, ru, rd = _lowrank_factors(gate, up, down, d, dev)
    else:
        g = u = dn = [None] * 4
        rg = ru = rd = n_lr = 0
    if dense is not None:
        if len(dense) != 6:
            raise ValueError("dense is a 6-tuple (q_gd, s_gd, q_ud, s_ud, q_dd, s_dd)")
        _dev(dense[0], "q_gd")
        n_dense = dense[0].shape[0]
        for t, nm, dt, shp in zip(dense, ("q_gd", "s_gd", "q_ud", "s_ud", "q_dd", "s_dd"),
                                  (torch.int8, torch.float32) * 3,
                                  ((n_dense, d), (n_dense,), (n_dense, d), (n_dense,), (d, n_dense), (d,))):
            _tensor(t, nm, dt, shp, dev)
        dd = [t.contiguous() for t in dense]
    else:
        dd = [None] * 6
        n_dense = 0
    y = torch.empty(n_tok, d, dtype=torch.float32, device=dev)
    ws = _workspace(lib.lrc_hybrid_ffn_workspace(n_tok, n_lr, rg, ru, rd, n_dense), dev)
    p = lambda t: None if t is None else _ptr(t)
    _check(lib.lrc_hybrid_ffn(_ptr(xc), n_tok, d, n_lr, p(g[0]), p(g[1]), p(g[2]), p(g[3]), rg, p(u[0]), p(u[1]),
                              p(u[2]), p(u[3]), ru, p(dn[0]), p(dn[1]), p(dn[2]), p(dn[3]), rd, n_dense, p(dd[0]),
                              p(dd[1]), p(dd[2]), p(dd[3]), p(dd[4]), p(dd[5]), _ptr(y), _ptr(ws), ws.numel(),
                              _stream()), "lrc_hybrid_ffn")
    return y


def lrc_lowrank_ffn(x: torch.Tensor, gate, up, down):
    """Low-rank SwiGLU FFN forward with int8 factors.  x: (n_tok, d) fp32.
    gate, up: (q_R (r, d) int8, s_R (r,), q_L (d_ff, r) int8, s_L (d_ff,)).
    down: (q_Rt (d_ff, r_d) int8 -- R_down transposed, s_R (r_d,), q_L (d, r_d) int8, s_L (d,)).
    Returns y (n_tok, d) fp32."""
    _dev(x, "x")
    if x.dtype != torch.float32 or x.dim() != 2:
        raise ValueError("x must be (n_tok, d) fp32")
    n_tok, d = x.shape
    dev = x.device
    xc = x.contiguous()
    g, u, dn, d_ff, rg, ru, rd = _lowrank_factors(gate, up, down, d, dev)
    y = torch.empty(n_tok, d, dtype=torch.float32, device=dev)
    ws = _workspace(lib.lrc_lowrank_ffn_workspace(n_tok, d_ff, rg, ru, rd), dev)
    _check(lib.lrc_lowrank_ffn(_ptr(xc), n_tok, d, d_ff, _ptr(g[0]), _ptr(g[1]), _ptr(g[2]), _ptr(g[3]), rg,
                               _ptr(u[0]), _ptr(u[1]), _ptr(u[2]), _ptr(u[3]), ru, _ptr(dn[0]), _ptr(dn[1]),
                               _ptr(dn[2]), _ptr(dn[3]), rd, _ptr(y), _ptr(ws), ws.numel(), _stream()),
           "lrc_lowrank_ffn")
    return y


def lrc_profile_start() -> None:
    """Start recording HIP events around every instrumented kernel launch (clears totals)."""
    _check(lib.lrc_profile_start(), "lrc_profile_start")


def lrc_profile_stop() -> None:
    """Stop recording; waits for the recorded events and folds their times into the totals."""
    _check(lib.lrc_profile_stop(), "lrc_profile_stop")


def lrc_profile_kernels() -> dict:
    """Totals per kernel name since the last start: launches, total_ms, flops, bytes."""
    out = {}
    for i in range(lib.lrc_profile_kernels()):
        name = ctypes.c_char_p()
        launches = _i64()
        ms, fl, by = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        _check(lib.lrc_profile_kernel(i, ctypes.byref(name), ctypes.byref(launches), ctypes.byref(ms),
                                      ctypes.byref(fl), ctypes.byref(by)), "lrc_profile_kernel")
        out[name.value.decode()] = {"launches": launches.value, "total_ms": ms.value, "flops": fl.value,
                                    "bytes": by.value}
    return out
