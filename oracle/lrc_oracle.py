"""Plain fp64 CPU oracle of the whitened truncated decomposition and rank allocation.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg import this module; the library never does, and this module imports
nothing from the library.  It is written to be read against the pages, not to be
fast: numpy/scipy (LAPACK) in fp64, one step per function, in the pages' order.

Pages (gist.science explainers; the alternative scorers at the end also cite UniRank
2.1 "Local Structural Significance" / "Global Functional Importance" and Swift-SVD
section B "Dynamic Rank Allocation Strategy", item "Hybrid Scoring"; the factor codec
cites LASER section 3 "Hybrid SVD-Quantization for FFNs", item "Quantization", the FFN
channel selection its items "Channel selection" and "Hybrid architecture", and the
low-rank FFN forward cites LASER section 4 "System Implementation"):
  * LASER: Loss-Aware Singular-value Decomposition and Rank Allocation for Efficient
    Low-Precision Vision-Language Models (technical summary, Methodology 1 "loss-aware
    SVD" with the items K-FAC surrogate / Transformation / QAW, Methodology 2
    "cross-layer rank allocation" with the items empirical-Fisher score / global
    optimisation);
  * UniRank: Unified Rank Allocation for Low-Rank LLM Compression (technical summary,
    section 2.1 "Sorting-and-Truncation", paragraph "Aggregation and Truncation");
  * Swift-SVD: Theoretical Optimality Meets Practical Efficiency in Low-Rank LLM
    Compression (technical summary, section 2A: closed-form optimum and incremental
    aggregation of the output covariance).

Orientation.  Weights are stored out x in (y = W x).  The pages write the layer as
Y = X W with W in x out, so their W is our W^T.  Their K-FAC form (G kron X) acting on
the column-major vec of their W, and their whitened weight S_x W S_g, correspond in our
orientation to  W_tilde = L_g^T W L_x  with X = L_x L_x^T and G = L_g L_g^T (lower
Cholesky factors).  The tests pin this against the Kronecker form built explicitly.

Every function is pinned by tests/test_oracle_pins.py (closed forms, invariants,
brute force, hand-derived fixtures under tests/golden/).
"""
from __future__ import annotations

import numpy as np
import scipy.linalg
import scipy.linalg.lapack as lapack

__all__ = [
    "qaw_fake_quant", "covariance_sum", "covariance", "cholesky_lower", "whiten",
    "truncated_svd", "canonical_signs", "back_map", "whiten_decompose",
    "fisher_scores", "kfac_scores", "allocation_keys", "allocate", "kfac_loss",
    "unirank_scores", "swift_layer_scores", "hadamard_rotation", "rotate_factors", "rtn_rows",
    "silu", "lowrank_ffn", "hybrid_ffn", "ffn_channel_errors", "select_channels",
]


# ---------------------------------------------------------------------------
# a0: quantisation-aware whitening input (LASER, Methodology 1, item QAW)
# ---------------------------------------------------------------------------
def qaw_fake_quant(a):
    """Per-token symmetric int8 fake quantisation, emulated exactly in float32.

    LASER (Methodology 1, QAW) estimates the K-FAC factors from quantised calibration
    activations.  The pages do not fix the quantiser; the reading used here is
    symmetric per token, levels -127..127, scale s_t = fl32(max_j |a_tj| / 127),
    q = clamp(round_half_even(fl32(a / s_t)), -127, 127), a_hat = fl32(q * s_t); an
    all-zero token stays zero.  Returns (q as int8, s as float32, a_hat as float32).
    """
    a = np.asarray(a, dtype=np.float32)
    m = np.max(np.abs(a), axis=1) if a.shape[1] else np.zeros(a.shape[0], np.float32)
    s = (m / np.float32(127.0)).astype(np.float32)
    q = np.zeros(a.shape, dtype=np.float32)
    nz = s > 0
    ratio = (a[nz] / s[nz, None]).astype(np.float32)
    q[nz] = np.clip(np.rint(ratio), -127.0, 127.0)
    a_hat = (q * s[:, None]).astype(np.float32)
    return q.astype(np.int8), s, a_hat


# ---------------------------------------------------------------------------
# a1: covariance streaming (LASER Methodology 1 K-FAC factors; Swift-SVD 2A
#     incremental aggregation)
# ---------------------------------------------------------------------------
def covariance_sum(a, block: int = 8192):
    """Raw second-moment sum  sum_t a_t^T a_t  in fp64 (inputs widened exactly).

    Swift-SVD (2A) aggregates the covariance one batch at a time; summing row blocks
    here is that aggregation, with fp64 accumulation."""
    a = np.asarray(a)
    d = a.shape[1]
    c = np.zeros((d, d), dtype=np.float64)
    for t0 in range(0, a.shape[0], block):
        blk = a[t0:t0 + block].astype(np.float64)
        c += blk.T @ blk
    return c


def covariance(a):
    """X = A^T A / N (LASER Methodology 1: activation / gradient covariance on the calibration set)."""
    n = np.asarray(a).shape[0]
    return covariance_sum(a) / float(n)


# ---------------------------------------------------------------------------
# a2: Cholesky factors (LASER Methodology 1, item Transformation)
# ---------------------------------------------------------------------------
def cholesky_lower(x):
    """Lower Cholesky factor of x with LAPACK dpotrf.  Returns (L, info).

    info = 0 on success; info = k > 0 when the leading minor of order k is not
    positive definite (then L is not usable).  No damping is added here."""
    x = np.asarray(x, dtype=np.float64)
    c, info = lapack.dpotrf(x, lower=1, clean=1)
    return np.tril(c), int(info)


# ---------------------------------------------------------------------------
# a3: whitening (LASER Methodology 1, item Transformation)
# ---------------------------------------------------------------------------
def whiten(w, lx=None, lg=None):
    """W_tilde = L_g^T W L_x  (identity for an absent factor)."""
    wt = np.asarray(w, dtype=np.float64)
    if lx is not None:
        wt = wt @ lx
    if lg is not None:
        wt = lg.T @ wt
    return wt


# ---------------------------------------------------------------------------
# a4: decomposition of the whitened weight
# ---------------------------------------------------------------------------
def truncated_svd(wt):
    """Thin SVD of the whitened weight (LAPACK dgesdd), singular values descending.

    The pages only say that the whitened weight is decomposed by SVD; any backward-
    stable thin SVD is that definition.  dgesdd is used because the host's dgesvd
    takes minutes at 4096 x 4096."""
    u, s, vt = scipy.linalg.svd(wt, full_matrices=False, lapack_driver="gesdd")
    order = np.argsort(-s, kind="stable")
    return u[:, order], s[order], vt[order, :]


def canonical_signs(u, vt, d_out, d_in):
    """Fix the sign of each singular pair (pages silent; reading of this library).

    The eigen-decomposed side is the smaller one: the left (output) side when
    d_out <= d_in, else the right (input) side.  Each pair (u_i, v_i) is flipped so
    that the largest-magnitude entry of that side's vector is positive; on a tie the
    lowest index decides."""
    u = u.copy()
    vt = vt.copy()
    left_side = d_out <= d_in
    for i in range(u.shape[1]):
        vec = u[:, i] if left_side else vt[i, :]
        j = int(np.argmax(np.abs(vec)))
        if vec[j] < 0:
            u[:, i] = -u[:, i]
            vt[i, :] = -vt[i, :]
    return u, vt


# ---------------------------------------------------------------------------
# a5: back to weight space (LASER Methodology 1, Transformation: factors mapped back)
# ---------------------------------------------------------------------------
def back_map(u, s, vt, r, lx=None, lg=None):
    """Left = L_g^-T U_r S_r^1/2 (d_out x r);  Right = S_r^1/2 V_r^T L_x^-1 (r x d_in).

    The square-root split of the singular values between the two factors is this
    library's reading (the pages are silent); Left @ Right does not depend on it."""
    sq = np.sqrt(s[:r])
    left = u[:, :r] * sq[None, :]
    right_t = vt[:r, :].T * sq[None, :]
    if lg is not None:
        left = scipy.linalg.solve_triangular(lg, left, trans="T", lower=True)
    if lx is not None:
        right_t = scipy.linalg.solve_triangular(lx, right_t, trans="T", lower=True)
    return left, right_t.T


def whiten_decompose(w, xsum=None, n_x=None, gsum=None, n_g=None, rank=None, damping=0.0):
    """The whole decomposition of one weight, as the pages define it.

    X = Xsum / n_x (+ damping I), G = Gsum / n_g (+ damping I); absent => identity.
    Cholesky -> whitening -> SVD -> sign fix -> back-map to rank r.
    Returns a dict with sigma (all k, descending), left, right, the whitened singular
    vectors u, vt, the factors lx, lg and info (0, or the failing Cholesky pivot,
    1-based; 'info_side' says which factor failed)."""
    w = np.asarray(w, dtype=np.float64)
    d_out, d_in = w.shape
    k = min(d_out, d_in)
    r = k if rank is None else int(rank)
    out = {"info": 0, "info_side": None}
    lx = lg = None
    if xsum is not None:
        x = np.asarray(xsum, dtype=np.float64)
        x = np.tril(x) + np.tril(x, -1).T
        x = x / float(n_x) + damping * np.eye(d_in)
        lx, info = cholesky_lower(x)
        if info:
            out.update(info=info, info_side="x")
            return out
    if gsum is not None:
        g = np.asarray(gsum, dtype=np.float64)
        g = np.tril(g) + np.tril(g, -1).T
        g = g / float(n_g) + damping * np.eye(d_out)
        lg, info = cholesky_lower(g)
        if info:
            out.update(info=info, info_side="g")
            return out
    wt = whiten(w, lx, lg)
    u, s, vt = truncated_svd(wt)
    u, vt = canonical_signs(u, vt, d_out, d_in)
    left, right = back_map(u, s, vt, r, lx, lg)
    out.update(sigma=s, left=left, right=right, u=u, vt=vt, lx=lx, lg=lg, wt=wt, k=k, r=r)
    return out


# ---------------------------------------------------------------------------
# a6: component scores (LASER Methodology 2, empirical-Fisher importance score)
# ---------------------------------------------------------------------------
def fisher_scores(a, b, left, right):
    """Empirical-Fisher contribution of each singular component.

    LASER (Methodology 2) scores a component by its contribution to the
    empirical-Fisher quadratic loss, which couples the component's size with its
    alignment to the calibration gradients in the original parameter space.  Reading:
    per-token gradient samples grad_t = b_t a_t^T (b_t: output gradient, a_t: input
    activation), component Delta_i = left_i right_i^T, and
        s_i = 1/2 * mean_t <grad_t, Delta_i>^2 = 1/(2N) sum_t (b_t . left_i)^2 (a_t . right_i)^2.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    n = a.shape[0]
    p = a @ np.asarray(right, dtype=np.float64).T     # N x k : a_t . right_i
    q = b @ np.asarray(left, dtype=np.float64)        # N x k : b_t . left_i
    return (p * p * q * q).sum(axis=0) / (2.0 * n)


def kfac_scores(sigma):
    """Without gradients: the K-FAC loss of dropping component i alone, 1/2 sigma_i^2."""
    s = np.asarray(sigma, dtype=np.float64)
    return 0.5 * s * s


# ---------------------------------------------------------------------------
# a7: global sort-and-truncate (LASER Methodology 2 global optimisation; UniRank 2.1
#     Aggregation and Truncation)
# ---------------------------------------------------------------------------
def allocation_keys(scores, cost_per_item):
    """Score per parameter cost, fp64(score) / fp64(cost) with IEEE rounding (Python float)."""
    return [float(np.float64(s)) / float(c) for s, c in zip(scores, cost_per_item)]


def allocate(scores_per_matrix, costs, budget):
    """Greedy global allocation under a parameter budget.

    All components of all matrices are pooled and sorted by score per parameter cost,
    highest first (LASER Methodology 2); one component of an m x n matrix costs m + n
    parameters and components are taken in sorted order until the budget is reached
    (UniRank 2.1).  Readings: equal keys keep (matrix id, component index) order; the
    kept set is the longest sorted prefix whose total cost is <= budget; a matrix's
    rank is the number of its kept components.

    scores_per_matrix: list of 1-D float32 arrays; costs: list of ints; budget: int.
    Returns (order, n_kept, ranks, kept_mask) with order a list of global item ids.
    A score is an importance (a sum of squares, or half a squared singular value), so
    NaN, infinite and negative scores are rejected, as are costs that are not positive."""
    mat, idx, sc, cst = [], [], [], []
    for m, s in enumerate(scores_per_matrix):
        if int(costs[m]) <= 0:
            raise ValueError("cost must be positive")
        s = np.asarray(s, dtype=np.float32)
        for i, v in enumerate(s.tolist()):
            if v != v or v in (float("inf"), float("-inf")) or v < 0.0:
                raise ValueError("score must be finite and non-negative")
            mat.append(m)
            idx.append(i)
            sc.append(v)
            cst.append(int(costs[m]))
    keys = allocation_keys(sc, cst)
    order = sorted(range(len(keys)), key=lambda j: (-keys[j], mat[j], idx[j]))
    total = 0
    n_kept = 0
    for j in order:
        if total + cst[j] > budget:
            break
        total += cst[j]
        n_kept += 1
    kept = np.zeros(len(keys), dtype=np.uint8)
    ranks = np.zeros(len(scores_per_matrix), dtype=np.int32)
    for j in order[:n_kept]:
        kept[j] = 1
        ranks[mat[j]] += 1
    return np.asarray(order, dtype=np.int64), n_kept, ranks, kept


# ---------------------------------------------------------------------------
# objective (LASER Methodology 1, K-FAC surrogate) -- used by the pins
# ---------------------------------------------------------------------------
def kfac_loss(dw, x, g):
    """1/2 vec(dW_p)^T (G kron X) vec(dW_p) with the pages' orientation dW_p = dW^T
    (in x out) and column-major vec, the Kronecker product built explicitly."""
    dwp = np.asarray(dw, dtype=np.float64).T
    v = dwp.reshape(-1, order="F")
    k = np.kron(np.asarray(g, dtype=np.float64), np.asarray(x, dtype=np.float64))
    return 0.5 * float(v @ k @ v)


# ---------------------------------------------------------------------------
# alternative component scores for the same allocator
# ---------------------------------------------------------------------------
def unirank_scores(sigmas_per_matrix, importance):
    """UniRank (2.1 Sorting-and-Truncation, "Aggregation and Truncation"): the score of
    singular triplet i of matrix l is the layer's global functional importance I_l times
    the triplet's local structural significance, its share of the squared singular-value
    energy sigma_{l,i}^2 / ||Sigma_l||_F^2.  I_l is supplied by the caller (the pages
    measure it as one minus the mean input/output cosine similarity of the layer on
    calibration data).  A matrix whose singular values are all zero scores 0.
    Returns one fp64 array per matrix."""
    out = []
    for sig, il in zip(sigmas_per_matrix, importance):
        s2 = np.asarray(sig, dtype=np.float64) ** 2
        total = float(np.sum(s2))
        out.append(float(il) * s2 / total if total > 0.0 else np.zeros_like(s2))
    return out


def swift_layer_scores(sigmas_per_matrix, beta, alpha):
    """Swift-SVD (section B, Hybrid Scoring): the compressibility score of layer l at
    rank k is beta_l^alpha * log(e + eps*_{k,l})^(1 - alpha), where beta_l is the
    caller's layer importance and eps*_{k,l} the theoretical loss of the closed-form
    rank-k solution, i.e. the energy of the discarded singular values,
    sum_{j > k} sigma_{l,j}^2.  Entry k - 1 of matrix l's array is the score at rank k
    (k = 1 .. number of singular values).  Returns one fp64 array per matrix."""
    out = []
    for sig, b in zip(sigmas_per_matrix, beta):
        s2 = np.asarray(sig, dtype=np.float64) ** 2
        eps = np.array([float(np.sum(s2[k:])) for k in range(1, len(s2) + 1)], dtype=np.float64)
        out.append(float(b) ** alpha * np.log(np.e + eps) ** (1.0 - alpha))
    return out


# ---------------------------------------------------------------------------
# factor codec (LASER, 3. Hybrid SVD-Quantization for FFNs, item Quantization)
# ---------------------------------------------------------------------------
def hadamard_rotation(r, signs):
    """The orthogonal rotation inserted between the low-rank factors to smooth outliers.
    The pages do not fix it; the reading used here is a sign-randomised Hadamard matrix
    R = H_r diag(signs) / sqrt(r), with H_r the Sylvester Hadamard matrix (r a power of
    two) and signs a caller-supplied vector of +-1."""
    h = scipy.linalg.hadamard(int(r)).astype(np.float64)
    return h * np.asarray(signs, dtype=np.float64)[None, :] / np.sqrt(float(r))


def rotate_factors(left, right, signs):
    """left' = left R and right' = R^T right, so left' right' = left right (R orthogonal).
    left: d_out x r, right: r x d_in.  The products are taken in fp64 and rounded once to
    fp32 (the values the quantiser then sees)."""
    rot = hadamard_rotation(np.asarray(left).shape[1], signs)
    lr = np.asarray(left, dtype=np.float64) @ rot
    rr = rot.T @ np.asarray(right, dtype=np.float64)
    return lr.astype(np.float32), rr.astype(np.float32)


def rtn_rows(x):
    """Round-to-nearest int8 quantisation of each row (one output channel per row) of an
    fp32 matrix.  The pages name RTN without its parameters; the reading used here is the
    same symmetric quantiser as qaw_fake_quant, per row: scale = fl32(max|row| / 127),
    q = clamp(round_half_even(fl32(x / scale)), -127, 127), an all-zero row gives zeros
    with scale 0.  Returns (q int8, scale float32)."""
    q, s, _ = qaw_fake_quant(np.asarray(x, dtype=np.float32))
    return q, s


# ---------------------------------------------------------------------------
# low-rank FFN forward (LASER, 4. System Implementation)
# ---------------------------------------------------------------------------
def silu(z):
    """SiLU(z) = z / (1 + exp(-z)), the gate nonlinearity of the SwiGLU FFN."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def lowrank_ffn(x, gate, up, down):
    """Forward pass of a SwiGLU FFN whose three weights are replaced by their low-rank
    factors, as the pages' fused decode kernels run it: the input projection to the
    latent space, the latent-to-hidden expansion, SwiGLU, and the down projection,
    with the int8 factors dequantised on the fly.  The reading: y = W_down (SiLU(W_gate x)
    * (W_up x)) with W ~ L R for each of gate, up, down; every factor is int8 with one
    scale per row, L = q_L * s_L[:, None], R = q_R * s_R[:, None].
    x: n_tok x d.  gate, up: (q_R (r x d), s_R, q_L (d_ff x r), s_L); down: (q_R
    (r_d x d_ff), s_R, q_L (d x r_d), s_L).  Returns y: n_tok x d in fp64."""
    def deq(q, sc):
        return np.asarray(q, dtype=np.float64) * np.asarray(sc, dtype=np.float64)[:, None]

    def apply(f, v):
        q_r, s_r, q_l, s_l = f
        return (v @ deq(q_r, s_r).T) @ deq(q_l, s_l).T

    xv = np.asarray(x, dtype=np.float64)
    h = silu(apply(gate, xv)) * apply(up, xv)
    return apply(down, h)


def hybrid_ffn(x, gate=None, up=None, down=None, dense=None):
    """Forward pass of an FFN in the hybrid form (LASER, 3. Hybrid SVD-Quantization for
    FFNs, item "Hybrid architecture"): the selected hidden channels go through the
    low-rank factors, the rest keep dense (int8, per-row scale) rows.  Reading: the
    channels are ordered low-rank first; the FFN is the sum of the two channel groups'
    contributions, y = lowrank_ffn(x, gate, up, down) + Wd_dense (SiLU(Wg_dense x) *
    (Wu_dense x)).  dense = (q_gd (n_dense x d), s_gd, q_ud, s_ud, q_dd (d x n_dense), s_dd)
    with each matrix = q * s[:, None]; either group may be absent (None).
    Returns y: n_tok x d in fp64."""
    xv = np.asarray(x, dtype=np.float64)
    y = np.zeros_like(xv)
    if gate is not None:
        y = y + lowrank_ffn(xv, gate, up, down)
    if dense is not None:
        wg, wu, wd = (np.asarray(dense[i], np.float64) * np.asarray(dense[i + 1], np.float64)[:, None]
                      for i in (0, 2, 4))
        y = y + (silu(xv @ wg.T) * (xv @ wu.T)) @ wd.T
    return y


# ---------------------------------------------------------------------------
# FFN hybrid channel selection (LASER, 3. Hybrid SVD-Quantization for FFNs, items
# "Channel selection" and "Hybrid architecture")
# ---------------------------------------------------------------------------
def ffn_channel_errors(w_gate, w_up, gate_factors, up_factors, xsum, n_x, damping=0.0):
    """Reconstruction error of every hidden channel under the temporary low-rank form of
    the gate and up projections.  The pages call the channels with a low reconstruction
    error "SVD-friendly"; the reading here measures a channel's error the way the
    method measures loss, in the activation-weighted space: the expected squared error
    of the channel's two pre-activations under the calibration distribution,
        err[h] = sum over P in (gate, up) of dW_P[h] X dW_P[h]^T,  dW_P = W_P - Left_P Right_P,
    with X = Xsum / n_x + damping I (the covariance the decompositions used).
    w_gate, w_up: d_ff x d; *_factors: (Left d_ff x r, Right r x d) or None (r = 0).
    Returns err (d_ff,) in fp64."""
    x = np.asarray(xsum, dtype=np.float64)
    x = np.tril(x) + np.tril(x, -1).T
    x = x / float(n_x) + damping * np.eye(x.shape[0])
    err = 0.0
    for w, fac in ((w_gate, gate_factors), (w_up, up_factors)):
        dw = np.asarray(w, dtype=np.float64)
        if fac is not None:
            dw = dw - np.asarray(fac[0], dtype=np.float64) @ np.asarray(fac[1], dtype=np.float64)
        err = err + np.einsum("hi,ij,hj->h", dw, x, dw)
    return err


def select_channels(err, n_lowrank):
    """The n_lowrank channels with the smallest error take the low-rank branch, the rest
    stay dense (the pages: the SVD-friendly channels are compressed).  Ties go to the
    lower channel index.  Returns (order: channels by ascending error, lowrank: 0/1 mask)."""
    err = [float(v) for v in err]
    order = sorted(range(len(err)), key=lambda h: (err[h], h))
    lowrank = np.zeros(len(err), dtype=np.uint8)
    for h in order[:n_lowrank]:
        lowrank[h] = 1
    return np.array(order, dtype=np.int64), lowrank
