"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same
seeded inputs, at sizes the oracle finishes in seconds (several tiles, ragged tails).

Tolerances (floating point) follow from the arithmetic, see each test; integer and
index results are compared bit for bit.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24     # fp32 unit roundoff


@pytest.fixture(scope="module")
def lrc():
    import curvature_aware_rank_amd as m
    return m


def dev():
    return torch.device("cuda:0")


def to_np(t):
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


def lower(c):
    return np.tril(c)


def bf16_stream(n, d, exponent, seed, outlier_frac=0.0):
    return synth.activation_stream(n, d, exponent, seed, outlier_frac=outlier_frac, dtype=torch.bfloat16,
                                   device="cpu")


# ----------------------------------------------------------------------------- a1 covariance
@pytest.mark.parametrize("n,d", [(700, 8), (1000, 300), (4100, 520), (130, 1100), (2000, 4000), (64, 1100)])
def test_cov_bf16_exact_on_small_integers(lrc, n, d):
    """bf16 inputs in {-3..3}: every product and partial sum is an integer below 2^24, so
    fp32 accumulation is exact in any order -> bit-exact against the oracle.  Catches a
    dropped, repeated or misplaced token, channel or tile.  The last two shapes have few
    token steps per tile, so each tile is one split that the SYRK adds to C itself."""
    g = torch.Generator().manual_seed(n * 7 + d)
    a = torch.randint(-3, 4, (n, d), generator=g).to(torch.bfloat16)
    c = torch.zeros(d, d, dtype=torch.float32, device=dev())
    lrc.lrc_accumulate_cov(a.to(dev()), c)
    want = lower(oracle.covariance_sum(to_np(a)))
    got = lower(to_np(c))
    assert np.array_equal(got, want)
    # the strict upper triangle is left untouched
    assert np.all(np.triu(to_np(c), 1) == 0)


@pytest.mark.parametrize("n,d", [(4096, 256), (3000, 520)])
def test_cov_bf16_gaussian(lrc, n, d):
    """fp32 accumulation of exact bf16 products: per-entry error modelled as
    sqrt(depth) * u * (|A|^T |A|)_ij with depth = n (+splits), times a safety factor 10."""
    a = bf16_stream(n, d, 1.0, 1234 + d, outlier_frac=0.01)
    c = torch.zeros(d, d, dtype=torch.float32, device=dev())
    lrc.lrc_accumulate_cov(a.to(dev()), c)
    an = to_np(a).astype(np.float64)
    want = an.T @ an
    absmag = np.abs(an).T @ np.abs(an)
    tol = 10 * math.sqrt(n + 64) * U32 * absmag + 1e-30
    err = np.abs(lower(to_np(c)) - lower(want))
    assert np.all(err <= lower(tol)), float(np.max(err / lower(tol + 1e-300)))


def test_cov_streaming_chunks_match_one_shot(lrc):
    """Swift-SVD 2A aggregation: summing chunks equals one pass up to rounding, and the
    same chunking twice gives the same bits."""
    a = bf16_stream(5000, 264, 1.0, 77).to(dev())
    c1 = torch.zeros(264, 264, device=dev())
    lrc.lrc_accumulate_cov(a, c1)
    c2 = torch.zeros(264, 264, device=dev())
    for t0 in range(0, 5000, 1234):
        lrc.lrc_accumulate_cov(a[t0:t0 + 1234], c2)
    c3 = torch.zeros(264, 264, device=dev())
    for t0 in range(0, 5000, 1234):
        lrc.lrc_accumulate_cov(a[t0:t0 + 1234], c3)
    assert torch.equal(c2, c3)
    ref = to_np(c1).astype(np.float64)
    np.testing.assert_allclose(np.tril(to_np(c2)), np.tril(ref), rtol=1e-5, atol=1e-5 * np.abs(ref).max())


@pytest.mark.parametrize("n,d", [(1000, 96), (4096, 256)])
def test_cov_fp32(lrc, n, d):
    a = synth.activation_stream(n, d, 1.2, 99 + d, dtype=torch.float32)
    c = torch.zeros(d, d, device=dev())
    lrc.lrc_accumulate_cov(a.to(dev()), c)
    an = to_np(a).astype(np.float64)
    absmag = np.abs(an).T @ np.abs(an)
    tol = 10 * math.sqrt(n) * U32 * absmag + 2 * U32 * np.abs(an.T @ an)
    err = np.abs(lower(to_np(c)) - lower(an.T @ an))
    assert np.all(err <= lower(tol))


# ----------------------------------------------------------------------------- a0 QAW
@pytest.mark.parametrize("d", [136, 4000])
def test_qaw_cov_exact_with_power_of_two_scales(lrc, d):
    """Rows whose max |a| is 127 * 2^e have an exact scale s = 2^e, so q, s^2 q (one bf16
    term, the low term is 0) and every product are exact; with 48 tokens, |values| <= 127
    and s >= 1/4 every partial sum is a multiple of 1/16 below 2^20, so fp32 accumulation
    is exact in any order and the GPU must equal the oracle bit for bit.  At 4000 channels
    each tile is one split, added to C by the SYRK itself."""
    g = torch.Generator().manual_seed(5)
    n = 48
    a = torch.randint(-7, 8, (n, d), generator=g).float()
    a[:, 3] = 127.0                                   # row max exactly 127 -> s = 1
    scale = 2.0 ** torch.randint(-2, 1, (n, 1), generator=g).float()
    a = a * scale
    a[17] = 0.0                                       # an all-zero token
    a = a.to(torch.bfloat16)                          # exact
    c = torch.zeros(d, d, device=dev())
    lrc.lrc_accumulate_cov(a.to(dev()), c, quant=True)
    _, _, ahat = oracle.qaw_fake_quant(to_np(a))
    assert np.array_equal(lower(to_np(c)), lower(oracle.covariance_sum(ahat)))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_qaw_cov_gaussian(lrc, dtype):
    """Products q_i (s^2 q_j) with s^2 q_j carried as bf16 hi + lo (relative 2^-16) against
    fl32(q s) products in fp64: tolerance 2^-15 |A_hat|^T |A_hat| + accumulation term."""
    n, d = 3000, 200
    a = synth.activation_stream(n, d, 1.0, 4242, outlier_frac=0.02, dtype=dtype)
    c = torch.zeros(d, d, device=dev())
    lrc.lrc_accumulate_cov(a.to(dev()), c, quant=True)
    _, _, ahat = oracle.qaw_fake_quant(to_np(a).astype(np.float32))
    ah = ahat.astype(np.float64)
    absmag = np.abs(ah).T @ np.abs(ah)
    tol = (2.0 ** -15 + 10 * math.sqrt(n) * U32) * absmag
    err = np.abs(lower(to_np(c)) - lower(ah.T @ ah))
    assert np.all(err <= lower(tol) + 1e-30)


# ----------------------------------------------------------------------------- a2..a5
def _decompose_case(lrc, d_out, d_in, n, rank, two_sided, seed, dtype=torch.float32, quant=False):
    a = synth.activation_stream(n, d_in, 1.2, seed, dtype=dtype)
    b = synth.activation_stream(n, d_out, 1.2, seed + 1, dtype=dtype) if two_sided else None
    w = synth.weight(d_out, d_in, seed + 2)
    xs = torch.zeros(d_in, d_in, device=dev())
    lrc.lrc_accumulate_cov(a.to(dev()), xs, quant=quant)
    gs = None
    if two_sided:
        gs = torch.zeros(d_out, d_out, device=dev())
        lrc.lrc_accumulate_cov(b.to(dev()), gs)
    sig, left, right, info = lrc.lrc_whiten_decompose(w.to(dev()), rank, xs, n, gs, n if two_sided else 0)
    an = to_np(a).astype(np.float32)
    if quant:
        an = oracle.qaw_fake_quant(an)[2]
    ref = oracle.whiten_decompose(to_np(w), oracle.covariance_sum(an), n,
                                  oracle.covariance_sum(to_np(b)) if two_sided else None, n if two_sided else None,
                                  rank=rank)
    return dict(a=an, b=None if b is None else to_np(b), w=to_np(w), sig=to_np(sig), left=to_np(left),
                right=to_np(right), info=to_np(info), ref=ref, n=n)


def _check_decomposition(case, rank, sig_rtol=1e-4, angle_tol=1e-3):
    ref, sig = case["ref"], case["sig"].astype(np.float64)
    s_ref = ref["sigma"]
    assert np.all(case["info"] == 0)
    # retained singular values: relative error (stated accuracy 1e-4)
    rel = np.abs(sig[:rank] - s_ref[:rank]) / s_ref[:rank]
    assert rel.max() <= sig_rtol, rel.max()
    # every sigma (discarded tail included): absolute error within 1e-4 sigma_1 -- the
    # tail's relative accuracy is out of an fp32 whitened weight's reach, its absolute
    # accuracy is not; and the same in sigma^2, against sigma_1^2
    assert np.max(np.abs(sig - s_ref)) <= 1e-4 * s_ref[0]
    assert np.max(np.abs(sig ** 2 - s_ref ** 2)) <= 1e-5 * s_ref[0] ** 2
    # K-FAC loss of the truncation (the objective, independent of signs and rotations)
    x = oracle.covariance(case["a"])
    dw = case["w"].astype(np.float64) - case["left"].astype(np.float64) @ case["right"].astype(np.float64)
    lx = np.linalg.cholesky(x)
    if case["b"] is not None:
        lg = np.linalg.cholesky(oracle.covariance(case["b"]))
        loss = 0.5 * np.linalg.norm(lg.T @ dw @ lx) ** 2
    else:
        loss = 0.5 * np.linalg.norm(dw @ lx) ** 2
    want = 0.5 * np.sum(s_ref[rank:] ** 2)
    assert abs(loss - want) <= 1e-3 * want + 1e-6 * 0.5 * s_ref[0] ** 2
    # leading subspaces where the spectral gap exceeds 1e-3 sigma_1 (whitened coordinates)
    lg_ = ref["lg"]
    lx_ = ref["lx"]
    u_gpu = case["left"].astype(np.float64)
    v_gpu = case["right"].astype(np.float64).T
    u_gpu = (lg_.T @ u_gpu) if lg_ is not None else u_gpu          # = U~ S^1/2
    v_gpu = (lx_.T @ v_gpu) if lx_ is not None else v_gpu           # = V~ S^1/2
    for j in range(1, rank + 1):
        if j < len(s_ref) and s_ref[j - 1] - s_ref[j] <= 1e-3 * s_ref[0]:
            continue
        for g, r in ((u_gpu[:, :j], ref["u"][:, :j]), (v_gpu[:, :j], ref["vt"][:j].T)):
            q, _ = np.linalg.qr(g)
            cosines = np.linalg.svd(q.T @ r, compute_uv=False)
            ang = np.arccos(np.clip(cosines.min(), -1, 1))
            assert ang <= angle_tol, (j, ang)


@pytest.fixture(params=["jacobi", "tridiag"])
def solver(request):
    """Run a decomposition test through each eigensolver of the library."""
    old = os.environ.get("LRC_EIGENSOLVER")
    os.environ["LRC_EIGENSOLVER"] = request.param
    yield request.param
    if old is None:
        del os.environ["LRC_EIGENSOLVER"]
    else:
        os.environ["LRC_EIGENSOLVER"] = old


def test_decompose_two_sided_fp32_config0_shape(lrc, solver):
    """The single-linear-layer workload: 256 x 256, 4096 fp32 tokens, two-sided, r = 64."""
    case = _decompose_case(lrc, 256, 256, 4096, 64, True, 11)
    _check_decomposition(case, 64)
    # signs follow the canonical rule on the output side (d_out <= d_in): compare
    # factor columns whose singular value is isolated by > 1e-3 sigma_1
    s = case["ref"]["sigma"]
    ref_left = case["ref"]["left"]
    for i in range(64):
        gap = min(s[i - 1] - s[i] if i else np.inf, s[i] - s[i + 1])
        if gap > 1e-3 * s[0]:
            np.testing.assert_allclose(case["left"][:, i], ref_left[:, i], rtol=0,
                                       atol=2e-3 * np.abs(ref_left[:, i]).max())


@pytest.mark.parametrize("d_out,d_in,rank", [(100, 150, 30), (150, 100, 40), (64, 64, 64), (300, 200, 7),
                                             (33, 1, 1), (257, 301, 40)])
def test_decompose_ragged_shapes(lrc, solver, d_out, d_in, rank):
    case = _decompose_case(lrc, d_out, d_in, 2000, rank, True, 23 + d_out)
    _check_decomposition(case, rank)


def test_decompose_activation_only_bf16(lrc, solver):
    case = _decompose_case(lrc, 320, 256, 3000, 64, False, 31, dtype=torch.bfloat16)
    _check_decomposition(case, 64)


def test_decompose_qaw_two_sided(lrc, solver):
    case = _decompose_case(lrc, 192, 128, 3000, 64, True, 41, dtype=torch.bfloat16, quant=True)
    _check_decomposition(case, 64)


def test_decompose_batched_heads(lrc):
    """Batched slices sharing one X (the per-head workload at small size)."""
    heads, hd, d_in, n, rank = 6, 24, 200, 3000, 10
    a = synth.activation_stream(n, d_in, 1.0, 55, outlier_frac=0.02, dtype=torch.bfloat16)
    w = synth.weight(heads * hd, d_in, 56)
    xs = torch.zeros(d_in, d_in, device=dev())
    lrc.lrc_accumulate_cov(a.to(dev()), xs)
    w3 = w.view(heads, hd, d_in).to(dev())
    sig, left, right, info = lrc.lrc_whiten_decompose(w3, rank, xs, n)
    assert torch.all(info == 0)
    an = to_np(a)
    xsum = oracle.covariance_sum(an)
    for h in range(heads):
        ref = oracle.whiten_decompose(to_np(w)[h * hd:(h + 1) * hd], xsum, n, rank=rank)
        case = dict(a=an, b=None, w=to_np(w)[h * hd:(h + 1) * hd], sig=to_np(sig[h]), left=to_np(left[h]),
                    right=to_np(right[h]), info=to_np(info[h:h + 1]), ref=ref, n=n)
        _check_decomposition(case, rank)


def test_decompose_batched_large_slices_take_tridiagonal_route(lrc, monkeypatch):
    """A batch of slices with k >= 384 (e.g. projections sharing one input covariance) is
    solved slice after slice by the tridiagonal solver: each slice gives the same bits as
    decomposing it alone, and matches the oracle."""
    monkeypatch.delenv("LRC_EIGENSOLVER", raising=False)
    batch, d_out, d_in, n, rank = 3, 400, 520, 3000, 50
    a = synth.activation_stream(n, d_in, 1.0, 61, dtype=torch.bfloat16)
    ws = [synth.weight(d_out, d_in, 62 + b) for b in range(batch)]
    xs = torch.zeros(d_in, d_in, device=dev())
    lrc.lrc_accumulate_cov(a.to(dev()), xs)
    w3 = torch.stack(ws).to(dev())
    sig, left, right, info = lrc.lrc_whiten_decompose(w3, rank, xs, n)
    assert torch.all(info == 0)
    for b in range(batch):
        s1, l1, r1, i1 = lrc.lrc_whiten_decompose(w3[b], rank, xs, n)
        assert torch.equal(sig[b], s1) and torch.equal(left[b], l1) and torch.equal(right[b], r1)
    an = to_np(a)
    ref = oracle.whiten_decompose(to_np(ws[1]), oracle.covariance_sum(an), n, rank=rank)
    case = dict(a=an, b=None, w=to_np(ws[1]), sig=to_np(sig[1]), left=to_np(left[1]), right=to_np(right[1]),
                info=to_np(info[1:2]), ref=ref, n=n)
    _check_decomposition(case, rank)


def test_decompose_batched_ragged_two_sided_large_grid(lrc):
    """40 two-sided slices of 301 x 517 share both covariances: the whitening products
    (W Lx, then Lg^T (W Lx)) run as batched launches with sizes that are not multiples of 4
    (scalar loads, ragged tile edges in every slice).  Slices checked against the oracle:
    the first and the last."""
    batch, d_out, d_in, n, rank = 40, 301, 517, 2000, 40
    a = synth.activation_stream(n, d_in, 1.2, 71, dtype=torch.float32)
    b = synth.activation_stream(n, d_out, 1.2, 72, dtype=torch.float32)
    ws = [synth.weight(d_out, d_in, 73 + i) for i in range(batch)]
    xs = torch.zeros(d_in, d_in, device=dev())
    gs = torch.zeros(d_out, d_out, device=dev())
    lrc.lrc_accumulate_cov(a.to(dev()), xs)
    lrc.lrc_accumulate_cov(b.to(dev()), gs)
    sig, left, right, info = lrc.lrc_whiten_decompose(torch.stack(ws).to(dev()), rank, xs, n, gs, n)
    assert torch.all(info == 0)
    an, bn = to_np(a), to_np(b)
    xsum, gsum = oracle.covariance_sum(an), oracle.covariance_sum(bn)
    for i in (0, batch - 1):
        ref = oracle.whiten_decompose(to_np(ws[i]), xsum, n, gsum, n, rank=rank)
        case = dict(a=an, b=bn, w=to_np(ws[i]), sig=to_np(sig[i]), left=to_np(left[i]), right=to_np(right[i]),
                    info=to_np(info[i:i + 1]), ref=ref, n=n)
        _check_decomposition(case, rank)


@pytest.mark.parametrize("d_out,d_in,rank,two_sided", [(400, 520, 50, False), (150, 100, 30, True)])
def test_decompose_slices_with_their_own_covariances(lrc, d_out, d_in, rank, two_sided, monkeypatch):
    """Independent layers in one call: slice b is whitened with its own X (and G) sums.
    Every slice gives the same bits as a call of its own on the same eigensolver route
    (tridiagonal at k = 400; block Jacobi, forced for the single calls too, at k = 100),
    and one slice is checked against the oracle."""
    monkeypatch.setenv("LRC_EIGENSOLVER", "tridiag" if min(d_out, d_in) >= 384 else "jacobi")
    batch, n = 3, 2500
    streams_a = [synth.activation_stream(n, d_in, 1.0 + 0.1 * b, 80 + b, dtype=torch.bfloat16) for b in range(batch)]
    streams_b = [synth.activation_stream(n, d_out, 1.3, 90 + b, dtype=torch.bfloat16) for b in range(batch)]
    w3 = torch.stack([synth.weight(d_out, d_in, 95 + b) for b in range(batch)]).to(dev())
    xs = torch.zeros(batch, d_in, d_in, device=dev())
    gs = torch.zeros(batch, d_out, d_out, device=dev()) if two_sided else None
    for b in range(batch):
        lrc.lrc_accumulate_cov(streams_a[b].to(dev()), xs[b])
        if two_sided:
            lrc.lrc_accumulate_cov(streams_b[b].to(dev()), gs[b])
    sig, left, right, info = lrc.lrc_whiten_decompose(w3, rank, xs, n, gs, n if two_sided else 0)
    assert torch.all(info == 0)
    for b in range(batch):
        s1, l1, r1, i1 = lrc.lrc_whiten_decompose(w3[b], rank, xs[b], n, gs[b] if two_sided else None,
                                                 n if two_sided else 0)
        assert int(i1[0]) == 0
        assert torch.equal(sig[b], s1) and torch.equal(left[b], l1) and torch.equal(right[b], r1), b
    an = to_np(streams_a[2])
    bn = to_np(streams_b[2]) if two_sided else None
    ref = oracle.whiten_decompose(to_np(w3[2]), oracle.covariance_sum(an), n,
                                  oracle.covariance_sum(bn) if two_sided else None, n if two_sided else None,
                                  rank=rank)
    case = dict(a=an, b=bn, w=to_np(w3[2]), sig=to_np(sig[2]), left=to_np(left[2]), right=to_np(right[2]),
                info=to_np(info[2:3]), ref=ref, n=n)
    _check_decomposition(case, rank)


def test_decompose_slices_own_covariance_not_positive_definite(lrc, monkeypatch):
    """A per-slice covariance that is not positive definite is reported in that slice's
    info only (the first failing pivot); the other slices are unaffected, bit for bit
    (single calls on the batch's block-Jacobi route)."""
    monkeypatch.setenv("LRC_EIGENSOLVER", "jacobi")
    batch, d, n, rank = 3, 96, 1000, 12
    xs = torch.zeros(batch, d, d, device=dev())
    for b in range(batch):
        lrc.lrc_accumulate_cov(synth.activation_stream(n, d, 1.0, 100 + b, dtype=torch.bfloat16).to(dev()), xs[b])
    xs[1, 40, :] = 0.0
    xs[1, :, 40] = 0.0          # pivot 41 of slice 1 is zero
    w3 = torch.stack([synth.weight(64, d, 110 + b) for b in range(batch)]).to(dev())
    sig, left, right, info = lrc.lrc_whiten_decompose(w3, rank, xs, n)
    assert to_np(info).tolist() == [0, 41, 0]
    for b in (0, 2):
        s1, l1, r1, i1 = lrc.lrc_whiten_decompose(w3[b], rank, xs[b], n)
        assert int(i1[0]) == 0
        assert torch.equal(sig[b], s1) and torch.equal(left[b], l1) and torch.equal(right[b], r1)


def test_decompose_identity_covariances_is_plain_svd(lrc, solver):
    """X = G = I (identity sums with count 1): plain truncated SVD of W (Eckart-Young)."""
    w = synth.weight(96, 130, 3)
    eye_in = torch.eye(130, device=dev())
    eye_out = torch.eye(96, device=dev())
    sig, left, right, info = lrc.lrc_whiten_decompose(w.to(dev()), 20, eye_in, 1, eye_out, 1)
    s = np.linalg.svd(to_np(w).astype(np.float64), compute_uv=False)
    np.testing.assert_allclose(to_np(sig), s, rtol=1e-5, atol=1e-6 * s[0])
    wr = to_np(left).astype(np.float64) @ to_np(right).astype(np.float64)
    np.testing.assert_allclose(np.linalg.norm(to_np(w) - wr) ** 2, np.sum(s[20:] ** 2), rtol=1e-4)


@pytest.mark.parametrize("side", ["x", "g"])
def test_decompose_not_positive_definite(lrc, side):
    """A negative pivot is reported (info = pivot, or d_in + pivot for G), never patched.
    The failure is found on the device: the call itself returns normally."""
    d_out, d_in, n = 40, 70, 500
    a = synth.activation_stream(n, d_in, 1.0, 8, dtype=torch.float32)
    b = synth.activation_stream(n, d_out, 1.0, 9, dtype=torch.float32)
    an, bn = to_np(a).astype(np.float64), to_np(b).astype(np.float64)
    xs = torch.tensor(an.T @ an, dtype=torch.float32, device=dev())
    gs = torch.tensor(bn.T @ bn, dtype=torch.float32, device=dev())
    p = 37 if side == "x" else 21
    (xs if side == "x" else gs)[p, p] = -1.0
    w = synth.weight(d_out, d_in, 10).to(dev())
    _, _, _, info = lrc.lrc_whiten_decompose(w, 5, xs, n, gs, n)
    ref = oracle.whiten_decompose(to_np(w), to_np(xs), n, to_np(gs), n, rank=5)
    assert ref["info_side"] == side and ref["info"] == p + 1
    want = p + 1 if side == "x" else d_in + p + 1
    assert int(info[0]) == want
    # batched slices: every slice reports the shared covariance's pivot
    w3 = torch.stack([w, 2 * w, -w])
    _, _, _, info3 = lrc.lrc_whiten_decompose(w3, 5, xs, n, gs, n)
    assert to_np(info3).tolist() == [want] * 3


def test_jacobi_sweep_cap_reports_no_convergence(lrc, monkeypatch):
    """The Jacobi solver enqueues a fixed number of sweeps; an item still rotating after
    the last one is reported with info = -1 (forced here by a cap of one sweep through the
    library's test override), one that converged within the cap with 0."""
    w = synth.weight(96, 130, 21).to(dev())
    a = synth.activation_stream(2000, 130, 1.0, 22, dtype=torch.bfloat16).to(dev())
    xs = torch.zeros(130, 130, device=dev())
    lrc.lrc_accumulate_cov(a, xs)
    monkeypatch.setenv("LRC_EIGENSOLVER", "jacobi")
    monkeypatch.setenv("LRC_JACOBI_MAX_SWEEPS", "1")
    _, _, _, info = lrc.lrc_whiten_decompose(w, 10, xs, 2000)
    assert int(info[0]) == -1
    # a diagonal Gram needs no rotation: converged in the first sweep
    eye = torch.eye(130, device=dev())
    wd = torch.zeros(96, 130, device=dev())
    wd[torch.arange(96), torch.arange(96)] = torch.linspace(3.0, 1.0, 96, device=dev())
    _, _, _, info = lrc.lrc_whiten_decompose(wd, 10, eye, 1)
    assert int(info[0]) == 0
    monkeypatch.delenv("LRC_JACOBI_MAX_SWEEPS")
    sig, _, _, info = lrc.lrc_whiten_decompose(w, 10, xs, 2000)
    assert int(info[0]) == 0


@pytest.mark.parametrize("solver_name,k", [("tridiag", 600), ("jacobi", 200)])
def test_decompose_does_not_wait_for_the_gpu(lrc, monkeypatch, solver_name, k):
    """The library only enqueues: with the stream busy for about a second, the call
    returns at once and an event recorded right after it is still pending."""
    import time
    monkeypatch.setenv("LRC_EIGENSOLVER", solver_name)
    w = synth.weight(k, k, 31).to(dev())
    a = synth.activation_stream(3000, k, 1.0, 32, dtype=torch.bfloat16).to(dev())
    xs = torch.zeros(k, k, device=dev())
    lrc.lrc_accumulate_cov(a, xs)
    sig0, _, _, _ = lrc.lrc_whiten_decompose(w, 16, xs, 3000)    # warm-up (module load, workspace)
    big = torch.randn(4096, 4096, device=dev())
    torch.cuda.synchronize()
    t_busy = time.perf_counter()
    for _ in range(8):
        big @ big
    torch.cuda.synchronize()
    per_mm = (time.perf_counter() - t_busy) / 8
    reps = max(8, int(1.0 / per_mm))
    for _ in range(reps):                                       # ~1 s of queued GPU work
        big @ big
    t0 = time.perf_counter()
    sig, left, right, info = lrc.lrc_whiten_decompose(w, 16, xs, 3000)
    t_call = time.perf_counter() - t0
    ev = torch.cuda.Event()
    ev.record()
    pending = not ev.query()
    torch.cuda.synchronize()
    assert pending, f"the stream had drained when the call returned ({t_call * 1e3:.1f} ms)"
    assert t_call < 0.5 * reps * per_mm, (t_call, reps * per_mm)
    assert int(info[0]) == 0 and torch.equal(sig, sig0)


def test_decompositions_on_two_streams_match_sequential(lrc):
    """Independent decompositions issued on two streams at once (each with its own
    buffers) give the same bits as one after another: no kernel may depend on the order
    or timing in which its workgroups are dispatched.  A kernel that reads an entry which
    another of its own workgroups writes goes wrong only when some workgroups start late,
    as they do while another stream's kernels hold compute units: this is the case that
    shows it at the attention projection's size."""
    d, n, r = 4096, 8192, 256
    a = synth.activation_stream(n, d, 1.0, 91, dtype=torch.bfloat16).to(dev())
    w = synth.weight(d, d, 92).to(dev())
    cov = torch.zeros(d, d, device=dev())
    lrc.lrc_accumulate_cov(a, cov)
    ref = [t.clone() for t in lrc.lrc_whiten_decompose(w, r, cov, n)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    covs = [cov.clone(), cov.clone()]
    torch.cuda.synchronize()
    outs = []
    for k in range(6):
        with torch.cuda.stream(streams[k % 2]):
            outs.append(lrc.lrc_whiten_decompose(w, r, covs[k % 2], n))
    torch.cuda.synchronize()
    for k, out in enumerate(outs):
        for got, want, name in zip(out, ref, ("sigma", "left", "right", "info")):
            assert torch.equal(got, want), f"call {k} (stream {k % 2}): {name} differs from the sequential result"


def test_whole_path_on_three_streams_matches_sequential(lrc):
    """Three independent pipelines (covariance, a tridiagonal and a Jacobi-batched
    decomposition, Fisher scores, allocation) run at the same time on three streams, each
    enqueued by its own host thread, give the same bits as one after another."""
    import threading
    d_out, d_in, n, r = 700, 900, 4000, 64

    def inputs(seed):
        a = synth.activation_stream(n, d_in, 1.0, seed, dtype=torch.bfloat16).to(dev())
        b = synth.activation_stream(n, d_out, 1.3, seed + 1, dtype=torch.bfloat16).to(dev())
        w = synth.weight(d_out, d_in, seed + 2).to(dev())
        heads = synth.weight(8 * 32, d_in, seed + 3).to(dev()).view(8, 32, d_in)
        return a, b, w, heads

    def pipeline(a, b, w, heads):
        xs = torch.zeros(d_in, d_in, device=dev())
        ci = lrc.lrc_accumulate_cov(a, xs)
        sig, left, right, info = lrc.lrc_whiten_decompose(w, r, xs, n)
        hs, _, _, hinfo = lrc.lrc_whiten_decompose(heads, 8, xs, n)
        sc, si = lrc.lrc_score_components(left, right, A=a, B=b)
        pool = torch.cat([sc, hs.reshape(-1)])
        offs = torch.tensor([0, r] + [r + 32 * (h + 1) for h in range(8)], dtype=torch.int64, device=dev())
        cost = torch.tensor([d_out + d_in] + [32 + d_in] * 8, dtype=torch.int64, device=dev())
        order, n_kept, ranks, mask, ainfo = lrc.lrc_allocate_ranks(pool, offs, cost, 40 * (d_out + d_in))
        return [xs, sig, left, right, info, hs, hinfo, sc, order, n_kept, ranks, mask, ci, si, ainfo]

    data = [inputs(100 + 10 * i) for i in range(3)]
    torch.cuda.synchronize()
    ref = []
    for x in data:
        ref.append([t.clone() for t in pipeline(*x)])
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    got = [None] * 3

    def feed(i):
        torch.cuda.set_device(dev())
        with torch.cuda.stream(streams[i]):
            got[i] = pipeline(*data[i])

    threads = [threading.Thread(target=feed, args=(i,)) for i in range(3)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for i in range(3):
        assert int(ref[i][4][0]) == 0 and int(ref[i][14][0]) == 0
        for k, (g, want) in enumerate(zip(got[i], ref[i])):
            assert torch.equal(g, want), f"pipeline {i}: output {k} differs from the sequential run"


def test_cov_and_scores_flag_nonfinite_inputs(lrc):
    """A NaN or Inf in the tokens reaches the covariance diagonal (a sum of squares) and
    every Fisher score (sums of non-negative terms): both calls set LRC_ENONFINITE in their
    info; clean inputs leave it 0, and the flag is sticky over a chunked stream."""
    for dtype in (torch.bfloat16, torch.float32):
        a = synth.activation_stream(700, 96, 1.0, 61, dtype=dtype).to(dev())
        c = torch.zeros(96, 96, device=dev())
        info = lrc.lrc_accumulate_cov(a, c)
        assert int(info[0]) == 0
        bad = a.clone()
        bad[123, 45] = float("nan")
        info = torch.zeros(1, dtype=torch.int32, device=dev())
        lrc.lrc_accumulate_cov(bad, torch.zeros(96, 96, device=dev()), info=info)
        assert int(info[0]) == lrc.LRC_ENONFINITE
        lrc.lrc_accumulate_cov(a, torch.zeros(96, 96, device=dev()), info=info)   # sticky
        assert int(info[0]) == lrc.LRC_ENONFINITE
        bad = a.clone()
        bad[5, 95] = float("inf")
        info = lrc.lrc_accumulate_cov(bad, torch.zeros(96, 96, device=dev()), quant=True)
        assert int(info[0]) == lrc.LRC_ENONFINITE
        b = synth.activation_stream(700, 64, 1.5, 62, dtype=dtype).to(dev())
        g = torch.Generator().manual_seed(63)
        left = torch.randn(64, 40, generator=g).to(dev())
        right = torch.randn(40, 96, generator=g).to(dev())
        _, info = lrc.lrc_score_components(left, right, A=a, B=b)
        assert int(info[0]) == 0
        bb = b.clone()
        bb[9, 3] = float("nan")
        s, info = lrc.lrc_score_components(left, right, A=a, B=bb)
        assert int(info[0]) == lrc.LRC_ENONFINITE and torch.isnan(s).all()
    _, info = lrc.lrc_score_components(sigma=torch.tensor([1.0, float("inf")], device=dev()), mode="kfac")
    assert int(info[0]) == lrc.LRC_ENONFINITE


def test_cov_single_split_flags_nonfinite(lrc):
    """The SYRK that adds its tiles to C itself (one split: few tokens, many tiles) checks
    the diagonal as the split reduction does: a NaN in channel 3999 sets LRC_ENONFINITE,
    clean tokens leave info 0, and the entries away from that channel stay finite."""
    a = synth.activation_stream(100, 4000, 1.0, 64, dtype=torch.bfloat16).to(dev())
    c = torch.zeros(4000, 4000, device=dev())
    info = lrc.lrc_accumulate_cov(a, c)
    assert int(info[0]) == 0
    bad = a.clone()
    bad[7, 3999] = float("nan")
    c = torch.zeros(4000, 4000, device=dev())
    info = lrc.lrc_accumulate_cov(bad, c)
    assert int(info[0]) == lrc.LRC_ENONFINITE
    assert torch.isnan(c[3999, 3999]) and torch.isfinite(c[:3999, :3999]).all()


def test_decompose_deterministic(lrc, solver):
    w = synth.weight(128, 200, 5).to(dev())
    a = synth.activation_stream(1500, 200, 1.0, 6, dtype=torch.bfloat16).to(dev())
    xs = torch.zeros(200, 200, device=dev())
    lrc.lrc_accumulate_cov(a, xs)
    r1 = lrc.lrc_whiten_decompose(w, 32, xs, 1500)
    r2 = lrc.lrc_whiten_decompose(w, 32, xs, 1500)
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)


def _spectrum_weight(d_out, d_in, sigmas, seed):
    """W = U diag(sigmas) V^T with Haar U, V (fp32)."""
    u = synth.haar_rotation(d_out, seed)[:, :len(sigmas)].double()
    v = synth.haar_rotation(d_in, seed + 1)[:, :len(sigmas)].double()
    return ((u * torch.tensor(sigmas, dtype=torch.float64)) @ v.T).float()


@pytest.mark.parametrize("mult", [8, 200])
def test_decompose_repeated_singular_values(lrc, mult):
    """A block of `mult` equal singular values: inverse iteration orthogonalises within the
    cluster, by one wave (8) or by a whole workgroup (200, above the one-wave limit of 32).
    Checked: sigma, the truncation loss, the leading subspaces outside the cluster and the
    orthonormality of the cluster's whitened singular vectors."""
    d = 600
    sig = np.linspace(2.0, 0.5, d)
    sig[100:100 + mult] = sig[100]      # stays descending; the cluster sits at 100 .. 100 + mult - 1
    w = _spectrum_weight(d, d, sig, 77 + mult)
    eye = torch.eye(d, device=dev())
    rank = 150 + mult
    s_gpu, left, right, info = lrc.lrc_whiten_decompose(w.to(dev()), rank, eye, 1)
    assert int(info[0]) == 0
    s_ref = np.linalg.svd(to_np(w).astype(np.float64), compute_uv=False)
    np.testing.assert_allclose(to_np(s_gpu), s_ref, rtol=1e-5, atol=1e-6 * s_ref[0])
    wr = to_np(left).astype(np.float64) @ to_np(right).astype(np.float64)
    np.testing.assert_allclose(np.linalg.norm(to_np(w).astype(np.float64) - wr) ** 2, np.sum(s_ref[rank:] ** 2),
                               rtol=1e-4)
    u_ref = np.linalg.svd(to_np(w).astype(np.float64))[0]
    for j in (50, rank):
        q, _ = np.linalg.qr(to_np(left).astype(np.float64)[:, :j])
        cosines = np.linalg.svd(q.T @ u_ref[:, :j], compute_uv=False)
        assert np.arccos(np.clip(cosines.min(), -1, 1)) <= 1e-3
    # G = I: Left = U S^1/2, so U = Left S^-1/2 must be orthonormal, cluster included
    u = to_np(left).astype(np.float64) / np.sqrt(to_np(s_gpu)[:rank].astype(np.float64))
    assert np.abs(u.T @ u - np.eye(rank)).max() <= 1e-4


def test_decompose_batched_clusters_equal_single_calls(lrc, monkeypatch):
    """Three 600 x 600 slices solved together by the tridiagonal route (the eigenvalues and
    the inverse iteration of all slices in one launch per kernel): slice 0 has a cluster of
    8 equal singular values (one-wave orthogonalisation), slice 1 one of 200 (a workgroup
    per cluster), slice 2 none.  Each slice equals its own call bit for bit."""
    monkeypatch.setenv("LRC_EIGENSOLVER", "tridiag")
    d, rank = 600, 350
    ws = []
    for b, mult in enumerate((8, 200, 1)):
        sig = np.linspace(2.0, 0.5, d)
        sig[100:100 + mult] = sig[100]
        ws.append(_spectrum_weight(d, d, sig, 177 + b))
    w3 = torch.stack(ws).to(dev())
    eye = torch.eye(d, device=dev())
    sig, left, right, info = lrc.lrc_whiten_decompose(w3, rank, eye, 1)
    assert torch.all(info == 0)
    for b in range(3):
        s1, l1, r1, i1 = lrc.lrc_whiten_decompose(w3[b], rank, eye, 1)
        assert int(i1[0]) == 0
        assert torch.equal(sig[b], s1) and torch.equal(left[b], l1) and torch.equal(right[b], r1), b
    # the 200-member cluster's whitened vectors are orthonormal (G = I: U = Left S^-1/2)
    u = to_np(left[1]).astype(np.float64) / np.sqrt(to_np(sig[1])[:rank].astype(np.float64))
    assert np.abs(u.T @ u - np.eye(rank)).max() <= 1e-4


def test_decompose_default_solver_mid_size(lrc):
    """A single Gram takes the tridiagonal route by default (here k = 600, ragged panels)."""
    case = _decompose_case(lrc, 640, 600, 4000, 100, False, 91, dtype=torch.bfloat16)
    _check_decomposition(case, 100)


# ----------------------------------------------------------------------------- a6 scores
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("n,d_out,d_in,k", [(1000, 70, 90, 50), (4096, 256, 128, 128), (65, 16, 300, 16),
                                             (1000, 72, 88, 50), (777, 200, 136, 300), (513, 1024, 64, 129),
                                             (2100, 264, 520, 600), (20000, 64, 64, 2048)])
def test_fisher_scores(lrc, dtype, n, d_out, d_in, k):
    """Same synthetic factors and streams into both sides.  fp32 projections then
    squares: relative error per token term ~ 4 * sqrt(d) u on well-scaled terms; the sum
    of non-negative terms keeps that relative bound -> rtol 2e-4.  bf16 activations with
    widths a multiple of 8 take the MFMA kernel, whose factors are split into two bf16
    parts (residual <= 2^-16 of each factor entry): the projection error grows to about
    2^-16 relative, 4 of which reach the product of squares, still inside 2e-4.  The
    shapes cover ragged token, component and reduction tiles of both kernels, up to 79
    token tiles by 16 component tiles."""
    a = synth.activation_stream(n, d_in, 1.0, 300 + n, dtype=dtype)
    b = synth.activation_stream(n, d_out, 1.5, 301 + n, dtype=dtype)
    g = torch.Generator().manual_seed(k)
    left = torch.randn(d_out, k, generator=g)
    right = torch.randn(k, d_in, generator=g)
    got, info = lrc.lrc_score_components(left.to(dev()), right.to(dev()), A=a.to(dev()), B=b.to(dev()))
    assert int(info[0]) == 0
    want = oracle.fisher_scores(to_np(a), to_np(b), left.numpy(), right.numpy())
    np.testing.assert_allclose(to_np(got), want, rtol=2e-4)


@pytest.mark.parametrize("d_out,d_in", [(40, 60), (48, 64)])
def test_fisher_scores_streamed_chunks(lrc, d_out, d_in):
    n, k = 3000, 30
    a = synth.activation_stream(n, d_in, 1.0, 1, dtype=torch.bfloat16).to(dev())
    b = synth.activation_stream(n, d_out, 1.5, 2, dtype=torch.bfloat16).to(dev())
    g = torch.Generator().manual_seed(3)
    left = torch.randn(d_out, k, generator=g).to(dev())
    right = torch.randn(k, d_in, generator=g).to(dev())
    one, _ = lrc.lrc_score_components(left, right, A=a, B=b)
    s = torch.empty(k, device=dev())
    cuts = [0, 1000, 2100, 3000]
    for i in range(3):
        lrc.lrc_score_components(left, right, A=a[cuts[i]:cuts[i + 1]], B=b[cuts[i]:cuts[i + 1]], scores=s,
                                 accumulate=i > 0, finalize=i == 2, n_total=n)
    np.testing.assert_allclose(to_np(s), to_np(one), rtol=1e-5)


def test_kfac_scores(lrc):
    sig = torch.rand(77) * 3
    got, info = lrc.lrc_score_components(sigma=sig.to(dev()), mode="kfac")
    assert int(info[0]) == 0
    np.testing.assert_allclose(to_np(got), oracle.kfac_scores(sig.numpy()), rtol=2 * U32 * 4)


# ----------------------------------------------------------------------------- a7 allocation
def _alloc_case(lrc, scores_list, costs, budget, want_order=True):
    """The allocation of a pool on the device and by the oracle.  With want_order False the
    library selects the cut without sorting and the returned order is None."""
    offs = np.concatenate([[0], np.cumsum([len(s) for s in scores_list])]).astype(np.int64)
    flat = np.concatenate(scores_list).astype(np.float32) if scores_list else np.zeros(0, np.float32)
    order, n_kept, ranks, kept, info = lrc.lrc_allocate_ranks(
        torch.tensor(flat, device=dev()), torch.tensor(offs, device=dev()),
        torch.tensor(np.asarray(costs, np.int64), device=dev()), budget, want_order=want_order)
    ref = oracle.allocate(scores_list, costs, budget)
    return (to_np(order) if want_order else None, int(to_np(n_kept)[0]), to_np(ranks), to_np(kept),
            int(to_np(info)[0])), ref


def _same_order(got, ref):
    return got[0] is None or got[0].tolist() == ref[0].tolist()


WANT_ORDER = pytest.mark.parametrize("want_order", [True, False], ids=["sort", "select"])


@WANT_ORDER
def test_allocate_golden_fixture(lrc, want_order):
    got, ref = _alloc_case(lrc, [np.array([10, 1], np.float32), np.array([16, 8, 8, 0.8], np.float32)], [5, 8], 22,
                           want_order)
    assert got[4] == 0
    assert ref[0].tolist() == [0, 2, 3, 4, 1, 5] and _same_order(got, ref)
    assert got[1] == 3 and got[2].tolist() == [1, 2] and got[3].tolist() == [1, 0, 1, 1, 0, 0]


@WANT_ORDER
@pytest.mark.parametrize("seed", range(6))
def test_allocate_bit_exact_random(lrc, seed, want_order):
    """Identical fp32 score arrays into both sides: order, n_kept, ranks and mask equal."""
    rng = np.random.default_rng(seed)
    nm = int(rng.integers(1, 40))
    sizes = rng.integers(0, 700, nm)
    costs = [int(c) for c in rng.integers(1, 20000, nm)]
    lst = []
    for m in range(nm):
        s = (rng.standard_exponential(sizes[m]) ** 3).astype(np.float32)
        if seed % 2:       # force many exact key ties across matrices and within
            s = np.round(s * 4).astype(np.float32) * np.float32(costs[m] % 7 + 1)
        lst.append(s)
    total = sum(int(c) * int(z) for c, z in zip(costs, sizes))
    budget = int(rng.integers(0, total + 1)) if total else 0
    got, ref = _alloc_case(lrc, lst, costs, budget, want_order)
    assert got[4] == 0
    assert _same_order(got, ref)
    assert got[1] == ref[1]
    assert got[2].tolist() == ref[2].tolist()
    assert got[3].tolist() == ref[3].tolist()


@WANT_ORDER
def test_allocate_large_ties(lrc, want_order):
    """Tens of thousands of items (several sort tiles), keys drawn from 50 values."""
    rng = np.random.default_rng(9)
    lst = [rng.integers(0, 50, 9000).astype(np.float32) for _ in range(7)]
    costs = [8192, 8192, 8192, 8192, 15104, 15104, 15104]
    got, ref = _alloc_case(lrc, lst, costs, 200_000_000, want_order)
    assert _same_order(got, ref) and got[1] == ref[1] and got[2].tolist() == ref[2].tolist()
    assert got[3].tolist() == ref[3].tolist()


@WANT_ORDER
def test_allocate_many_tiles_skewed(lrc, want_order):
    """About a million items (hundreds of sort tiles and a ragged last tile): half the keys
    share one value, the rest are spread over a few hundred values, so whole tiles fall
    into one digit and the stable order of equal keys spans tiles."""
    rng = np.random.default_rng(21)
    sizes = rng.integers(20000, 50000, 30)
    costs = [int(c) for c in rng.integers(1000, 16000, 30)]
    lst = []
    for m in range(30):
        s = rng.integers(0, 300, sizes[m]).astype(np.float32) * np.float32(0.25)
        s[rng.random(sizes[m]) < 0.5] = np.float32(costs[m])   # key exactly 1.0
        lst.append(s)
    total = sum(c * int(z) for c, z in zip(costs, sizes))
    got, ref = _alloc_case(lrc, lst, costs, total // 3, want_order)
    assert got[4] == 0
    assert _same_order(got, ref)
    assert got[1] == ref[1] and got[2].tolist() == ref[2].tolist() and got[3].tolist() == ref[3].tolist()


def test_allocate_runs_of_tiles_per_workgroup(lrc):
    """A pool of 20 million items, large enough that each sort workgroup takes a run of
    several tiles (its digit counts carry from tile to tile): 224 matrices, half the scores
    from 64 values (ties inside and across tiles and workgroups), half uniform.  The
    reference order is the oracle's keys (checked against allocation_keys on a sample)
    sorted by a stable library sort: key descending, global item id ascending."""
    rng = np.random.default_rng(31)
    n_mat, per = 224, 89286
    m_items = n_mat * per
    costs = np.where(np.arange(n_mat) % 7 < 4, 8192, 15104).astype(np.int64)
    s = rng.random(m_items, dtype=np.float32)
    tied = rng.random(m_items) < 0.5
    s[tied] = rng.integers(0, 64, int(tied.sum())).astype(np.float32) * np.float32(1.0 / 64)
    cost_item = np.repeat(costs, per)
    budget = int(0.6 * int(cost_item.sum()))
    offs = np.arange(0, m_items + 1, per, dtype=np.int64)
    order, n_kept, ranks, kept, info = lrc.lrc_allocate_ranks(
        torch.tensor(s, device=dev()), torch.tensor(offs, device=dev()), torch.tensor(costs, device=dev()), budget)
    assert int(to_np(info)[0]) == 0
    key = s.astype(np.float64) / cost_item.astype(np.float64)
    smp = rng.integers(0, m_items, 5000)
    assert np.array_equal(np.asarray(oracle.allocation_keys(s[smp].tolist(), cost_item[smp].tolist())), key[smp])
    ref_order = np.lexsort((np.arange(m_items), -key))
    assert np.array_equal(to_np(order).astype(np.int64), ref_order)
    csum = np.cumsum(cost_item[ref_order])
    ref_kept = int(np.searchsorted(csum, budget, side="right"))
    assert int(to_np(n_kept)[0]) == ref_kept
    mask = np.zeros(m_items, np.uint8)
    mask[ref_order[:ref_kept]] = 1
    assert np.array_equal(to_np(kept), mask)
    assert np.array_equal(to_np(ranks), np.bincount(ref_order[:ref_kept] // per, minlength=n_mat).astype(np.int32))
    # the selection without an order reaches the same cut on the same pool
    _, n_kept2, ranks2, kept2, info2 = lrc.lrc_allocate_ranks(
        torch.tensor(s, device=dev()), torch.tensor(offs, device=dev()), torch.tensor(costs, device=dev()), budget,
        want_order=False)
    assert int(to_np(info2)[0]) == 0 and int(to_np(n_kept2)[0]) == ref_kept
    assert np.array_equal(to_np(kept2), mask) and np.array_equal(to_np(ranks2), to_np(ranks))


def test_allocate_select_64m_items(lrc):
    """The benchmark's scaled pool, 16384 matrices x 4096 uniform scores (67,108,864 items,
    costs 8192 and 15104, 60% budget), both ways: the sort and the order-free selection
    give the same n_kept, ranks and mask, and the kept set is checked against the plain
    definition on the host: every kept (key, id) lies below every excluded one in the
    order (key descending, id ascending), the kept cost fits the budget and adding the
    first excluded item would not."""
    n_mat, per = 16384, 4096
    m_items = n_mat * per
    costs = np.where(np.arange(n_mat) % 2 == 0, 8192, 15104).astype(np.int64)
    g = torch.Generator(device=dev()).manual_seed(64)
    sc = torch.rand(m_items, generator=g, device=dev())
    offs = torch.arange(0, m_items + 1, per, dtype=torch.int64, device=dev())
    cost_item = np.repeat(costs, per)
    budget = int(0.6 * int(cost_item.sum()))
    order, n_kept, ranks, kept, info = lrc.lrc_allocate_ranks(sc, offs, torch.tensor(costs, device=dev()), budget)
    _, n_kept2, ranks2, kept2, info2 = lrc.lrc_allocate_ranks(sc, offs, torch.tensor(costs, device=dev()), budget,
                                                              want_order=False)
    assert int(to_np(info)[0]) == 0 == int(to_np(info2)[0])
    nk = int(to_np(n_kept)[0])
    assert nk == int(to_np(n_kept2)[0])
    mask = to_np(kept).astype(bool)
    assert np.array_equal(mask, to_np(kept2).astype(bool)) and np.array_equal(to_np(ranks), to_np(ranks2))
    del order
    key = to_np(sc).astype(np.float64) / cost_item.astype(np.float64)
    assert int(mask.sum()) == nk
    kept_cost = int(cost_item[mask].sum())
    assert kept_cost <= budget
    kk, ek = key[mask], key[~mask]
    lo = kk.min()
    assert ek.max() <= lo
    ids = np.arange(m_items)
    tie_ex = ids[~mask][ek == lo]
    if tie_ex.size:   # excluded items with the smallest kept key come after every kept one
        assert tie_ex.min() > ids[mask][kk == lo].max()
    first_ex = tie_ex.min() if tie_ex.size else ids[~mask][ek == ek.max()].min()
    assert kept_cost + int(cost_item[first_ex]) > budget
    assert np.array_equal(to_np(ranks), mask.reshape(n_mat, per).sum(1).astype(np.int32))


@WANT_ORDER
def test_allocate_edge_cases(lrc, want_order):
    # zero budget keeps nothing, a budget above the total keeps everything
    lst = [np.array([1, 2, 3], np.float32), np.zeros(0, np.float32), np.array([5], np.float32)]
    got, ref = _alloc_case(lrc, lst, [3, 4, 5], 0, want_order)
    assert got[1] == 0 == ref[1] and got[2].tolist() == [0, 0, 0] and got[3].tolist() == [0, 0, 0, 0]
    got, ref = _alloc_case(lrc, lst, [3, 4, 5], 10 ** 12, want_order)
    assert got[1] == 4 == ref[1] and got[2].tolist() == [3, 0, 1] and got[3].tolist() == [1, 1, 1, 1]
    # a budget equal to the total keeps everything, one less drops the last in the order
    got, ref = _alloc_case(lrc, lst, [3, 4, 5], 14, want_order)
    assert got[1] == 4 == ref[1]
    got, ref = _alloc_case(lrc, lst, [3, 4, 5], 13, want_order)
    assert got[1] == ref[1] and got[3].tolist() == ref[3].tolist()
    # -0.0 and +0.0 are the same key; equal keys are kept in id order
    got, ref = _alloc_case(lrc, [np.array([0.0, -0.0, 0.0], np.float32)], [2], 4, want_order)
    assert ref[0].tolist() == [0, 1, 2] and _same_order(got, ref)
    assert got[1] == 2 and got[3].tolist() == [1, 1, 0]
    # every score zero (one key over the whole pool), several sort tiles
    got, ref = _alloc_case(lrc, [np.zeros(5000, np.float32), np.zeros(3000, np.float32)], [7, 7], 7 * 4321,
                           want_order)
    assert got[1] == 4321 == ref[1] and got[2].tolist() == [4321, 0] and got[3].tolist() == ref[3].tolist()
    # no items at all
    got, ref = _alloc_case(lrc, [np.zeros(0, np.float32)], [3], 10, want_order)
    assert got[1] == 0 and got[2].tolist() == [0]


@WANT_ORDER
@pytest.mark.parametrize("bad", [float("nan"), float("inf"), float("-inf"), -1.0])
def test_allocate_rejects_invalid_scores(lrc, bad, want_order):
    """A score that is NaN, infinite or negative is rejected (LRC_ENONFINITE) and nothing is
    kept, like the oracle's allocator, which raises on the same input."""
    flat = torch.tensor([1.0, bad, 2.0], device=dev())
    offs = torch.tensor([0, 3], dtype=torch.int64, device=dev())
    _, n_kept, ranks, kept, info = lrc.lrc_allocate_ranks(flat, offs,
                                                          torch.tensor([4], dtype=torch.int64, device=dev()), 10,
                                                          want_order=want_order)
    assert int(info[0]) == lrc.LRC_ENONFINITE
    assert int(n_kept[0]) == 0 and int(ranks[0]) == 0 and int(kept.sum()) == 0
    with pytest.raises(ValueError):
        oracle.allocate([to_np(flat)], [4], 10)


@WANT_ORDER
def test_allocate_rejects_bad_cost(lrc, want_order):
    flat = torch.tensor([1.0, 2.0, 2.0], device=dev())
    offs = torch.tensor([0, 3], dtype=torch.int64, device=dev())
    _, n_kept, ranks, kept, info = lrc.lrc_allocate_ranks(flat, offs,
                                                          torch.tensor([0], dtype=torch.int64, device=dev()), 10,
                                                          want_order=want_order)
    assert int(info[0]) == lrc.LRC_EINVAL
    assert int(n_kept[0]) == 0 and int(ranks[0]) == 0 and int(kept.sum()) == 0


# ----------------------------------------------------------------------------- alternative scorers
def _rank_score_case(lrc, sizes, mode, alpha, seed, zero_matrix=None):
    rng = np.random.default_rng(seed)
    sig = []
    for m, z in enumerate(sizes):
        s = np.sort(rng.gamma(0.7, 2.0, z))[::-1].astype(np.float32)
        if m == zero_matrix:
            s[:] = 0
        sig.append(s)
    weight = rng.uniform(0.2, 3.0, len(sizes)).astype(np.float32)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    flat = np.concatenate(sig) if sig else np.zeros(0, np.float32)
    got, info = lrc.lrc_rank_scores(torch.tensor(flat, device=dev()), torch.tensor(offs, device=dev()),
                                    torch.tensor(weight, device=dev()), mode=mode, alpha=alpha)
    if mode == "unirank":
        ref = oracle.unirank_scores(sig, weight.astype(np.float64))
    else:
        ref = oracle.swift_layer_scores(sig, weight.astype(np.float64), float(np.float32(alpha)))
    ref = np.concatenate(ref) if ref else np.zeros(0)
    return to_np(got), ref, int(to_np(info)[0]), sig, weight, offs


@pytest.mark.parametrize("mode,alpha", [("unirank", 0.0), ("swift", 0.5), ("swift", 0.0), ("swift", 1.0)])
def test_rank_scores_match_oracle(lrc, mode, alpha):
    """fp64 sums on the device, fp32 outputs: within 2 fp32 ulps of the fp64 oracle.  Sizes
    cover empty and one-element matrices, segments shorter than a workgroup and a matrix
    longer than a workgroup's 256 threads (several elements per thread)."""
    got, ref, info, *_ = _rank_score_case(lrc, [5, 0, 1, 300, 4096, 17, 11008], mode, alpha, 3, zero_matrix=5)
    assert info == 0
    np.testing.assert_allclose(got, ref, rtol=2.5e-7, atol=1e-37)


def test_rank_scores_unirank_feed_the_allocator(lrc):
    """UniRank scores go straight into the global sort-and-truncate: the allocation of the
    GPU's fp32 scores matches the oracle allocator on the same scores bit for bit."""
    sizes = [64, 128, 96, 200]
    got, ref, info, sig, weight, offs = _rank_score_case(lrc, sizes, "unirank", 0.0, 8)
    assert info == 0
    costs = [256, 384, 300, 520]
    lst = [got[offs[m]:offs[m + 1]] for m in range(len(sizes))]
    order, n_kept, ranks, kept, ainfo = lrc.lrc_allocate_ranks(
        torch.tensor(got, device=dev()), torch.tensor(offs, device=dev()),
        torch.tensor(np.asarray(costs, np.int64), device=dev()), 40000)
    o = oracle.allocate(lst, costs, 40000)
    assert int(to_np(ainfo)[0]) == 0
    assert to_np(order).tolist() == o[0].tolist() and int(to_np(n_kept)[0]) == o[1]
    assert to_np(ranks).tolist() == o[2].tolist()


def test_rank_scores_reject_bad_inputs(lrc):
    sig = torch.tensor([2.0, float("nan"), 1.0], device=dev())
    offs = torch.tensor([0, 3], dtype=torch.int64, device=dev())
    _, info = lrc.lrc_rank_scores(sig, offs, torch.tensor([1.0], device=dev()))
    assert int(info[0]) == lrc.LRC_ENONFINITE
    sig = torch.tensor([2.0, 1.0, 1.0], device=dev())
    _, info = lrc.lrc_rank_scores(sig, offs, torch.tensor([-1.0], device=dev()))
    assert int(info[0]) == lrc.LRC_EINVAL
    _, info = lrc.lrc_rank_scores(sig, offs, torch.tensor([0.0], device=dev()), mode="swift")
    assert int(info[0]) == lrc.LRC_EINVAL
    _, info = lrc.lrc_rank_scores(sig, torch.tensor([0, 2], dtype=torch.int64, device=dev()),
                                  torch.tensor([1.0], device=dev()))
    assert int(info[0]) == lrc.LRC_EINVAL


# ----------------------------------------------------------------------------- factor codec
@pytest.mark.parametrize("d_out,r,d_in", [(96, 64, 40), (300, 1024, 257), (5, 1, 3), (64, 2048, 128),
                                         (40, 4096, 130), (24, 8192, 77)])
def test_rotate_quantize(lrc, d_out, r, d_in):
    """The rotated factors are the fp64 products rounded once to fp32: they match the
    oracle's within one fp32 rounding (the two sides sum in different orders).  The int8
    codes and scales are a decision taken in fp32 on those values, so they are checked bit
    for bit against the oracle's quantiser applied to the GPU's own rotated factors.
    The shapes include an outlier channel, r = 1, ragged d_out / d_in and the largest
    ranks (4096, 8192: rows of 32 and 64 KB in LDS)."""
    g = torch.Generator().manual_seed(r + d_in)
    left = torch.randn(d_out, r, generator=g)
    left[:, r // 3] *= 40.0      # an outlier channel, the case the rotation is for
    right = torch.randn(r, d_in, generator=g)
    signs = (torch.randint(0, 2, (r,), generator=g) * 2 - 1).float()
    ql, sl, qr, sr, lrot, rrot = lrc.lrc_rotate_quantize(left.to(dev()), right.to(dev()), signs.to(dev()),
                                                          keep_rotated=True)
    ref_l, ref_r = oracle.rotate_factors(left.numpy(), right.numpy(), signs.numpy())
    np.testing.assert_allclose(to_np(lrot), ref_l, rtol=2.4e-7, atol=1e-30)
    np.testing.assert_allclose(to_np(rrot), ref_r, rtol=2.4e-7, atol=1e-30)
    for q, s, rot in ((ql, sl, lrot), (qr, sr, rrot)):
        oq, os_ = oracle.rtn_rows(to_np(rot))
        assert np.array_equal(to_np(q), oq) and np.array_equal(to_np(s), os_)
    # the rotation spreads the outlier: left's largest magnitude falls
    if r > 1:
        assert np.abs(to_np(lrot)).max() < np.abs(left.numpy()).max()


def test_quantize_rows_bit_exact(lrc):
    """Dense branch: per-row RTN of the input itself, bit for bit with the oracle (ties
    to even and an all-zero row included)."""
    x = torch.randn(70, 333, generator=torch.Generator().manual_seed(5)) * 3
    x[4] = 0
    x[7, :4] = torch.tensor([127.0, 0.5, 1.5, -2.5])   # scale 1: exact halves round to even
    x[7, 4:] = 0
    q, s = lrc.lrc_quantize_rows(x.to(dev()))
    oq, os_ = oracle.rtn_rows(x.numpy())
    assert np.array_equal(to_np(q), oq) and np.array_equal(to_np(s), os_)


# ----------------------------------------------------------------------------- low-rank FFN
def _ffn_factor(g, rows, cols):
    q = torch.randint(-127, 128, (rows, cols), generator=g, dtype=torch.int8)
    s = (torch.rand(rows, generator=g) * 0.004 + 0.001).float()
    return q, s


@pytest.mark.parametrize("n_tok,d,d_ff,rg,ru,rd", [(1, 256, 688, 64, 48, 32), (5, 128, 300, 32, 32, 16),
                                                   (9, 4096, 11008, 2048, 2048, 2048)])
def test_lowrank_ffn(lrc, n_tok, d, d_ff, rg, ru, rd):
    """fp32 products and sums against the fp64 oracle.  Each output is a chain of four
    dot products of at most 11008 terms; the per-lane partial sums (<= 172 terms) and the
    fixed trees keep the rounding error near 200 u of the summed magnitudes, and for these
    random factors the summed magnitudes stay within ~30x of the outputs' largest, so the
    bound is 200 * 2^-24 * 30 ~ 4e-4 of max|y|; the observed error is far below it."""
    g = torch.Generator().manual_seed(d_ff + n_tok)
    gate = (*_ffn_factor(g, rg, d), *_ffn_factor(g, d_ff, rg))
    up = (*_ffn_factor(g, ru, d), *_ffn_factor(g, d_ff, ru))
    qrd, srd = _ffn_factor(g, rd, d_ff)
    qld, sld = _ffn_factor(g, d, rd)
    x = torch.randn(n_tok, d, generator=g) * 4
    y = lrc.lrc_lowrank_ffn(x.to(dev()), [t.to(dev()) for t in gate], [t.to(dev()) for t in up],
                            [qrd.t().contiguous().to(dev()), srd.to(dev()), qld.to(dev()), sld.to(dev())])
    ref = oracle.lowrank_ffn(x.numpy(), [t.numpy() for t in gate], [t.numpy() for t in up],
                             (qrd.numpy(), srd.numpy(), qld.numpy(), sld.numpy()))
    err = np.abs(to_np(y) - ref).max() / np.abs(ref).max()
    assert err < 4e-4, err




@pytest.mark.parametrize("n_tok,d,n_lr,n_dense,r", [(1, 256, 344, 336, 64), (5, 128, 160, 144, 32),
                                                    (3, 128, 0, 96, 0), (2, 128, 300, 0, 32),
                                                    (9, 4096, 5504, 5504, 2048)])
def test_hybrid_ffn(lrc, n_tok, d, n_lr, n_dense, r):
    """Hybrid FFN (low-rank channels first, then dense ones) against the fp64 oracle, at
    the low-rank FFN's bound (4e-4 of max|y|: the dense channels add one more dot product
    of d terms and one of n_dense terms per output, each with a fixed-order fp32 sum);
    either group may be empty."""
    g = torch.Generator().manual_seed(n_lr + 7 * n_dense + n_tok)
    lr = dn = None
    if n_lr:
        gate = (*_ffn_factor(g, r, d), *_ffn_factor(g, n_lr, r))
        up = (*_ffn_factor(g, r, d), *_ffn_factor(g, n_lr, r))
        qrd, srd = _ffn_factor(g, r, n_lr)
        qld, sld = _ffn_factor(g, d, r)
        lr = (gate, up, (qrd, srd, qld, sld))
    if n_dense:
        dn = (*_ffn_factor(g, n_dense, d), *_ffn_factor(g, n_dense, d), *_ffn_factor(g, d, n_dense))
    x = torch.randn(n_tok, d, generator=g) * 4
    to = lambda ts: [t.to(dev()) for t in ts]
    if lr:
        gate, up, (qrd, srd, qld, sld) = lr
        args = (to(gate), to(up), [qrd.t().contiguous().to(dev()), srd.to(dev()), qld.to(dev()), sld.to(dev())])
    else:
        args = (None, None, None)
    y = lrc.lrc_hybrid_ffn(x.to(dev()), *args, dense=to(dn) if dn else None)
    npy = lambda ts: [t.numpy() for t in ts]
    ref = oracle.hybrid_ffn(x.numpy(), *(npy(f) for f in lr) if lr else (None, None, None),
                            dense=npy(dn) if dn else None)
    err = np.abs(to_np(y) - ref).max() / np.abs(ref).max()
    assert err < 4e-4, err


# ----------------------------------------------------------------------------- FFN channel selection
def _ffn_sel_inputs(d_ff, d, r, n, seed, dup=False):
    """Seeded gate/up weights, a power-law calibration stream and the oracle's own rank-r
    factors (fp32) as the inputs both sides receive."""
    rng = np.random.default_rng(seed)
    q, rr = np.linalg.qr(rng.standard_normal((d, d)))
    q = q * np.sign(np.diag(rr))
    lam = np.arange(1, d + 1, dtype=np.float64) ** -1.0
    a = ((rng.standard_normal((n, d)) * np.sqrt(lam)) @ q.T).astype(np.float32)
    wg = (rng.standard_normal((d_ff, d)) / math.sqrt(d)).astype(np.float32)
    wu = (rng.standard_normal((d_ff, d)) / math.sqrt(d)).astype(np.float32)
    if dup:   # repeated channels: equal errors, ordered by index
        wg[7::11] = wg[3]
        wu[7::11] = wu[3]
    xs = oracle.covariance_sum(a).astype(np.float32)
    fac = []
    for w in (wg, wu):
        if r == 0:
            fac.append(None)
            continue
        res = oracle.whiten_decompose(w, xs.astype(np.float64), n, rank=r, damping=1e-3)
        left = res["left"].astype(np.float32)
        if dup:
            left[7::11] = left[3]
        fac.append((left, res["right"].astype(np.float32)))
    return wg, wu, fac, xs


@pytest.mark.parametrize("d_ff,d,r,n_low", [(300, 96, 24, 120), (257, 64, 0, 100), (1100, 256, 128, 550),
                                            (130, 80, 60, 0), (130, 80, 40, 130)])
def test_ffn_select_channels(lrc, d_ff, d, r, n_low):
    """Per-channel errors against the fp64 oracle (its quadratic form dW X dW^T, not the
    library's ||dW L_x||^2).  The GPU forms D = W - Left Right and E = D L_x in fp32
    (MFMA, sums of <= 256 products: relative error of an entry ~ sqrt(k) u = 16 u against
    the summed magnitudes, which stay within a few times |E| for these inputs) and sums
    E^2 in fp64, so err is within ~1e-5 relative; the bound is 5e-5.  The order and the
    selection are a decision in fp64 on the GPU's errors: bit-exact against the oracle's
    rule applied to them."""
    n, damping = 2000, 1e-3
    wg, wu, fac, xs = _ffn_sel_inputs(d_ff, d, r, n, seed=d_ff + r)
    t = lambda x: torch.from_numpy(x).to(dev())
    err, order, low, info = lrc.lrc_ffn_select_channels(
        t(wg), t(wu), None if r == 0 else (t(fac[0][0]), t(fac[0][1])), None if r == 0 else (t(fac[1][0]), t(fac[1][1])),
        t(xs), n, n_low, damping)
    assert int(info.item()) == 0
    ref = oracle.ffn_channel_errors(wg, wu, fac[0], fac[1], xs, n, damping)
    np.testing.assert_allclose(to_np(err), ref, rtol=5e-5)
    o_ord, o_low = oracle.select_channels(to_np(err), n_low)
    assert np.array_equal(to_np(order).astype(np.int64), o_ord)
    assert np.array_equal(to_np(low), o_low)


def test_ffn_select_channels_ties_and_failure(lrc):
    """Repeated channels give bit-equal errors (row-independent arithmetic) and are
    ordered by index; a covariance that is not positive definite is reported (info =
    the failing pivot), not patched."""
    d_ff, d, r, n = 140, 64, 16, 1000
    wg, wu, fac, xs = _ffn_sel_inputs(d_ff, d, r, n, seed=7, dup=True)
    t = lambda x: torch.from_numpy(x).to(dev())
    err, order, low, info = lrc.lrc_ffn_select_channels(t(wg), t(wu), (t(fac[0][0]), t(fac[0][1])),
                                                        (t(fac[1][0]), t(fac[1][1])), t(xs), n, 60, 1e-3)
    e = to_np(err)
    assert np.all(e[7::11] == e[3])
    o_ord, o_low = oracle.select_channels(e, 60)
    assert np.array_equal(to_np(order).astype(np.int64), o_ord) and np.array_equal(to_np(low), o_low)
    bad = np.zeros((d, d), dtype=np.float32)
    _, _, _, info = lrc.lrc_ffn_select_channels(t(wg), t(wu), None, None, t(bad), n, 10, 0.0)
    assert int(info.item()) == 1          # the first pivot of the zero covariance, found on the device
