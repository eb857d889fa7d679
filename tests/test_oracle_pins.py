"""Pins of the fp64 oracle to facts fixed outside itself (CPU only).

Each test ties one oracle function to a closed form, an invariant, a brute-force
construction or a hand-derived fixture (tests/golden/), chosen so that a plausible
slip (a transposed factor, a dropped 1/2, a wrong vec order, a wrong tie-break) fails.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from tests.conftest import read_golden

RNG = np.random.default_rng(20260602)


def _spd_stream(n, d, exponent, rng):
    q, r = np.linalg.qr(rng.standard_normal((d, d)))
    q = q * np.sign(np.diag(r))
    lam = np.arange(1, d + 1, dtype=np.float64) ** (-exponent)
    return (rng.standard_normal((n, d)) * np.sqrt(lam)) @ q.T


# --------------------------------------------------------------------------- QAW
def test_qaw_golden_rows():
    for line in read_golden("qaw_rows.txt"):
        parts = dict(p.strip().split(":", 1) for p in line.split("|"))
        a = np.array([float(v) for v in parts["a"].split()], dtype=np.float32)[None, :]
        q, s, ah = oracle.qaw_fake_quant(a)
        assert s[0] == np.float32(float(parts["s"]))
        assert q[0].tolist() == [int(v) for v in parts["q"].split()]
        assert ah[0].tolist() == [float(v) for v in parts["ahat"].split()]


def test_qaw_invariants():
    a = (RNG.standard_normal((64, 37)) * np.exp(RNG.standard_normal((64, 1)))).astype(np.float32)
    a[5] = 0.0
    q, s, ah = oracle.qaw_fake_quant(a)
    assert q.dtype == np.int8 and np.all(np.abs(q.astype(int)) <= 127)
    nz = np.any(a != 0, axis=1)
    assert np.all(np.max(np.abs(q[nz].astype(int)), axis=1) == 127)
    assert np.all(q[~nz] == 0) and np.all(ah[~nz] == 0)
    # |a_hat - a| <= s/2 up to the fp32 roundings of a/s and q*s
    err = np.abs(ah.astype(np.float64) - a.astype(np.float64))
    bound = s[:, None].astype(np.float64) * (0.5 + 1e-5) + 1e-6 * np.abs(a)
    assert np.all(err <= bound)


# --------------------------------------------------------------------------- covariance
def test_covariance_is_mean_outer_product():
    a = RNG.standard_normal((7, 4)).astype(np.float32)
    brute = np.zeros((4, 4))
    for t in range(7):
        v = a[t].astype(np.float64)
        for i in range(4):
            for j in range(4):
                brute[i, j] += v[i] * v[j]
    np.testing.assert_allclose(oracle.covariance(a), brute / 7, rtol=1e-14, atol=1e-15)
    # chunked aggregation (Swift-SVD 2A) equals one-shot
    np.testing.assert_allclose(oracle.covariance_sum(a, block=3), brute, rtol=1e-14, atol=1e-14)


# --------------------------------------------------------------------------- Cholesky
def test_cholesky_golden():
    g = {ln.split(":")[0]: ln.split(":", 1)[1] for ln in read_golden("cholesky_cases.txt")}

    def mat(txt):
        return np.array([[float(v) for v in row.split()] for row in txt.split(";")])

    l, info = oracle.cholesky_lower(mat(g["pd_x"]))
    assert info == 0
    np.testing.assert_allclose(l, mat(g["pd_l"]), atol=1e-15)
    _, info = oracle.cholesky_lower(mat(g["notpd_x"]))
    assert info == int(g["notpd_info"])


def test_cholesky_reconstructs():
    x = oracle.covariance(RNG.standard_normal((50, 9)))
    l, info = oracle.cholesky_lower(x)
    assert info == 0 and np.allclose(np.triu(l, 1), 0)
    np.testing.assert_allclose(l @ l.T, x, rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------- decomposition
@pytest.mark.parametrize("shape", [(6, 6), (5, 8), (8, 3)])
def test_identity_whitening_is_plain_truncated_svd(shape):
    """X = G = I: the method reduces to a plain truncated SVD of W, and Eckart-Young
    (named by UniRank 2.1) fixes the truncation error."""
    d_out, d_in = shape
    w = RNG.standard_normal(shape)
    r = 2
    res = oracle.whiten_decompose(w, np.eye(d_in), 1, np.eye(d_out), 1, rank=r)
    # singular values from a different route: symmetric eigenvalues of W^T W
    ev = np.sort(np.linalg.eigvalsh(w.T @ w))[::-1][: min(shape)]
    np.testing.assert_allclose(res["sigma"] ** 2, np.maximum(ev, 0), rtol=1e-10, atol=1e-12)
    wr = res["left"] @ res["right"]
    assert np.linalg.matrix_rank(wr, tol=1e-9) == r
    np.testing.assert_allclose(np.linalg.norm(w - wr) ** 2, np.sum(res["sigma"][r:] ** 2), rtol=1e-10)


@pytest.mark.parametrize("d_out,d_in,r", [(3, 2, 1), (2, 4, 1), (4, 4, 2), (3, 5, 2), (2, 2, 0)])
def test_kfac_loss_equals_discarded_whitened_energy_bruteforce(d_out, d_in, r):
    """LASER Methodology 1: with the K-FAC surrogate 1/2 vec(dW)^T (G kron X) vec(dW),
    truncating the SVD of the whitened weight costs 1/2 * sum of the discarded
    sigma_tilde^2.  The Kronecker product is built explicitly (d_in*d_out <= 20)."""
    a = _spd_stream(300, d_in, 1.0, RNG)
    b = _spd_stream(300, d_out, 1.3, RNG)
    w = RNG.standard_normal((d_out, d_in))
    xs, gs = oracle.covariance_sum(a), oracle.covariance_sum(b)
    res = oracle.whiten_decompose(w, xs, 300, gs, 300, rank=r)
    x, g = xs / 300, gs / 300
    dw = w - (res["left"] @ res["right"] if r else 0.0)
    loss = oracle.kfac_loss(dw, x, g)
    np.testing.assert_allclose(loss, 0.5 * np.sum(res["sigma"][r:] ** 2), rtol=1e-10)
    # dropping one component alone costs exactly its K-FAC score 1/2 sigma_i^2
    full = oracle.whiten_decompose(w, xs, 300, gs, 300, rank=min(d_out, d_in))
    for i in range(min(d_out, d_in)):
        comp = np.outer(full["left"][:, i], full["right"][i])
        np.testing.assert_allclose(oracle.kfac_loss(comp, x, g), oracle.kfac_scores(full["sigma"])[i],
                                   rtol=1e-9)


def test_kfac_loss_orientation_would_catch_swap():
    """A swapped whitening (L_x on the left side) must not satisfy the identity: this
    keeps the brute-force pin sensitive to the orientation reading."""
    d_out, d_in = 3, 3
    a = _spd_stream(200, d_in, 1.0, RNG)
    b = _spd_stream(200, d_out, 1.3, RNG)
    w = RNG.standard_normal((d_out, d_in))
    x, g = oracle.covariance(a), oracle.covariance(b)
    lx, _ = oracle.cholesky_lower(x)
    lg, _ = oracle.cholesky_lower(g)
    wrong = lx.T @ w @ lg
    u, s, vt = np.linalg.svd(wrong)
    wr = np.linalg.solve(lx.T, u[:, :1] * s[:1]) @ np.linalg.solve(lg.T, vt[:1].T).T
    assert abs(oracle.kfac_loss(w - wr, x, g) - 0.5 * np.sum(s[1:] ** 2)) > 1e-6


def test_swift_svd_closed_form_and_optimality():
    """Swift-SVD 2A: with G = I, the optimum of ||A W^T - A W_k^T|| is W V_k V_k^T in the
    pages' orientation, V_k the top-k eigenvectors of the aggregated output covariance
    C = sum_t y_t^T y_t; its loss is the discarded eigen-energy (the theoretical
    minimum), and no other rank-k weight does better."""
    n, d_out, d_in, r = 400, 6, 7, 3
    a = _spd_stream(n, d_in, 1.2, RNG)
    w = RNG.standard_normal((d_out, d_in))
    res = oracle.whiten_decompose(w, oracle.covariance_sum(a), n, None, None, rank=r)
    y = a @ w.T                              # outputs, tokens x d_out
    c = np.zeros((d_out, d_out))
    for t0 in range(0, n, 64):               # incremental aggregation
        c += y[t0:t0 + 64].T @ y[t0:t0 + 64]
    ev, evec = np.linalg.eigh(c)
    ev, evec = ev[::-1], evec[:, ::-1]
    np.testing.assert_allclose(ev[: min(d_out, d_in)] / n, res["sigma"] ** 2, rtol=1e-10)
    wk = evec[:, :r] @ evec[:, :r].T @ w
    wr = res["left"] @ res["right"]
    np.testing.assert_allclose(wr, wk, rtol=1e-8, atol=1e-10)
    loss = np.linalg.norm(y - a @ wr.T) ** 2
    np.testing.assert_allclose(loss, n * np.sum(res["sigma"][r:] ** 2), rtol=1e-9)
    for _ in range(20):
        w2 = RNG.standard_normal((d_out, r)) @ RNG.standard_normal((r, d_in))
        assert np.linalg.norm(y - a @ w2.T) ** 2 >= loss * (1 - 1e-12)


@pytest.mark.parametrize("d_out,d_in", [(5, 7), (7, 5), (6, 6)])
def test_back_map_invariants(d_out, d_in):
    """The back-mapped factors are G- and X-orthogonal with the singular values on the
    diagonal, and whiten back to the truncated whitened SVD."""
    a = _spd_stream(500, d_in, 1.1, RNG)
    b = _spd_stream(500, d_out, 1.4, RNG)
    w = RNG.standard_normal((d_out, d_in))
    r = 3
    res = oracle.whiten_decompose(w, oracle.covariance_sum(a), 500, oracle.covariance_sum(b), 500, rank=r)
    x, g = oracle.covariance(a), oracle.covariance(b)
    left, right, s = res["left"], res["right"], res["sigma"]
    np.testing.assert_allclose(left.T @ g @ left, np.diag(s[:r]), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(right @ x @ right.T, np.diag(s[:r]), rtol=1e-9, atol=1e-11)
    lx, lg = res["lx"], res["lg"]
    wt_r = lg.T @ (left @ right) @ lx
    u, vt = res["u"], res["vt"]
    np.testing.assert_allclose(wt_r, (u[:, :r] * s[:r]) @ vt[:r], rtol=1e-9, atol=1e-11)


def test_canonical_signs_rule():
    w = RNG.standard_normal((4, 6))
    res = oracle.whiten_decompose(w, None, None, None, None, rank=4)
    for i in range(4):
        v = res["u"][:, i]
        assert v[np.argmax(np.abs(v))] > 0
    res = oracle.whiten_decompose(w.T.copy(), None, None, None, None, rank=4)
    for i in range(4):
        v = res["vt"][i]
        assert v[np.argmax(np.abs(v))] > 0


def test_cholesky_failure_reported_not_patched():
    a = RNG.standard_normal((3, 5))      # 3 tokens, 5 channels: X is singular
    res = oracle.whiten_decompose(RNG.standard_normal((4, 5)), oracle.covariance_sum(a), 3, rank=1)
    assert res["info"] > 0 and res["info_side"] == "x" and "sigma" not in res


# --------------------------------------------------------------------------- scores
@pytest.mark.parametrize("d_out,d_in", [(2, 3), (3, 2), (2, 2)])
def test_fisher_score_equals_empirical_fisher_quadratic_bruteforce(d_out, d_in):
    """LASER Methodology 2: the score is the component's contribution to the
    empirical-Fisher quadratic 1/2 vec(D)^T F vec(D), F = mean_t g_t g_t^T with the
    per-token gradient g_t = vec(b_t a_t^T).  F is built explicitly."""
    n = 40
    a = RNG.standard_normal((n, d_in))
    b = RNG.standard_normal((n, d_out))
    w = RNG.standard_normal((d_out, d_in))
    res = oracle.whiten_decompose(w, oracle.covariance_sum(a), n, oracle.covariance_sum(b), n)
    k = min(d_out, d_in)
    f = np.zeros((d_out * d_in, d_out * d_in))
    for t in range(n):
        gt = np.outer(b[t], a[t]).reshape(-1)
        f += np.outer(gt, gt)
    f /= n
    want = []
    for i in range(k):
        dlt = np.outer(res["left"][:, i], res["right"][i]).reshape(-1)
        want.append(0.5 * dlt @ f @ dlt)
    np.testing.assert_allclose(oracle.fisher_scores(a, b, res["left"], res["right"]), want, rtol=1e-10)


def test_fisher_score_expectation_is_kfac_score():
    """With independent Gaussian activations and gradients the empirical-Fisher score
    of component i concentrates on the K-FAC score 1/2 sigma_i^2 (the empirical-Fisher
    quadratic factorises in expectation into G kron X)."""
    n, d_out, d_in = 60000, 5, 4
    a = _spd_stream(n, d_in, 1.0, RNG)
    b = _spd_stream(n, d_out, 1.5, RNG)
    w = RNG.standard_normal((d_out, d_in))
    res = oracle.whiten_decompose(w, oracle.covariance_sum(a), n, oracle.covariance_sum(b), n)
    ratio = oracle.fisher_scores(a, b, res["left"], res["right"]) / oracle.kfac_scores(res["sigma"])
    assert np.all(np.abs(ratio - 1) < 0.1), ratio


# --------------------------------------------------------------------------- allocation
def test_allocate_golden():
    g = {ln.split(":")[0]: ln.split(":", 1)[1].split() for ln in read_golden("alloc_example.txt")}
    costs = [int(v) for v in g["costs"]]
    scores = [np.array([float(v) for v in g["scores0"]], np.float32),
              np.array([float(v) for v in g["scores1"]], np.float32)]
    order, n_kept, ranks, kept = oracle.allocate(scores, costs, int(g["budget"][0]))
    assert order.tolist() == [int(v) for v in g["order"]]
    assert n_kept == int(g["n_kept"][0])
    assert ranks.tolist() == [int(v) for v in g["ranks"]]
    assert kept.tolist() == [int(v) for v in g["kept_mask"]]


def test_allocate_invariants_random():
    for trial in range(30):
        nm = int(RNG.integers(1, 5))
        costs = [int(c) for c in RNG.integers(3, 12, nm)]
        scores = []
        for m in range(nm):
            s = RNG.choice([0.5, 1.0, 2.0, 3.0], size=int(RNG.integers(1, 6))).astype(np.float32)
            scores.append(s * np.float32(costs[m]) / np.float32(4.0))   # many exact ties
        tot = sum(c * len(s) for c, s in zip(costs, scores))
        budget = int(RNG.integers(0, tot + 5))
        order, n_kept, ranks, kept = oracle.allocate(scores, costs, budget)
        mat = np.concatenate([[m] * len(s) for m, s in enumerate(scores)]).astype(int)
        idx = np.concatenate([np.arange(len(s)) for s in scores]).astype(int)
        key = np.concatenate([s.astype(np.float64) / c for s, c in zip(scores, costs)])
        cost = np.array([costs[m] for m in mat])
        assert sorted(order.tolist()) == list(range(len(mat)))
        for p, q in zip(order[:-1], order[1:]):
            assert (key[p] > key[q]) or (key[p] == key[q] and (mat[p], idx[p]) < (mat[q], idx[q]))
        used = int(cost[order[:n_kept]].sum())
        assert used <= budget
        if n_kept < len(order):
            assert used + cost[order[n_kept]] > budget
        assert ranks.tolist() == np.bincount(mat[kept.astype(bool)], minlength=nm).tolist()


def test_allocate_equal_costs_is_optimal_subset():
    """Equal costs: the kept set is the top-K scores, hence it minimises the summed
    K-FAC loss of the discarded components over every subset of the same size."""
    scores = [RNG.random(4).astype(np.float32), RNG.random(3).astype(np.float32)]
    costs = [7, 7]
    flat = np.concatenate(scores).astype(np.float64)
    for budget in range(0, 7 * 7 + 1, 3):
        _, n_kept, _, kept = oracle.allocate(scores, costs, budget)
        assert n_kept == min(budget // 7, 7)
        best = min(flat.sum() - flat[list(c)].sum() for c in itertools.combinations(range(7), n_kept))
        np.testing.assert_allclose(flat.sum() - flat[kept.astype(bool)].sum(), best, rtol=1e-12)


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf, -0.5])
def test_allocate_rejects_invalid_scores(bad):
    """Importance scores are non-negative finite numbers (sums of squares, or half a
    squared singular value): anything else is rejected rather than sorted."""
    with pytest.raises(ValueError):
        oracle.allocate([np.array([1.0, bad], np.float32)], [3], 10)


def test_allocate_accepts_negative_zero_and_rejects_bad_cost():
    order, n_kept, _, _ = oracle.allocate([np.array([-0.0, 1.0], np.float32)], [3], 10)
    assert order.tolist() == [1, 0] and n_kept == 2
    with pytest.raises(ValueError):
        oracle.allocate([np.array([1.0], np.float32)], [0], 10)


# ----------------------------------------------------------------------------- alternative scorers
def _rank_score_fixture():
    rows = []
    for ln in read_golden("rank_scores.txt"):
        head, sig, want = (part.split() for part in ln.split("|"))
        rows.append((head[0], [float(x) for x in head[1:]], np.array(sig, float), np.array(want, float)))
    return rows


def test_rank_scores_golden():
    """Hand-worked values (tests/golden/rank_scores.txt, 7 significant digits)."""
    for kind, par, sig, want in _rank_score_fixture():
        if kind == "unirank":
            got = oracle.unirank_scores([sig], [par[0]])[0]
        else:
            got = oracle.swift_layer_scores([sig], [par[0]], par[1])[0]
        np.testing.assert_allclose(got, want, rtol=1e-6)


def test_unirank_scores_sum_to_importance():
    """Energy shares sum to one, so a matrix's scores sum to its importance I_l; they are
    proportional to sigma^2; I_l = 0 or an all-zero spectrum scores zero."""
    sig = [np.sort(RNG.random(n))[::-1] for n in (5, 1, 12)]
    imp = [0.3, 2.0, 0.0]
    out = oracle.unirank_scores(sig, imp)
    for s, i, o in zip(sig, imp, out):
        np.testing.assert_allclose(o.sum(), i, rtol=1e-14, atol=1e-300)
        if i > 0:
            np.testing.assert_allclose(o / o[0], s ** 2 / s[0] ** 2, rtol=1e-14)
    assert np.all(oracle.unirank_scores([np.zeros(4)], [1.0])[0] == 0.0)


def test_swift_discarded_energy_is_the_truncation_residual():
    """eps*_k of the score is the theoretical loss of the rank-k optimum: by
    Eckart-Young-Mirsky it equals ||M - M_k||_F^2 for the truncated SVD M_k, computed
    here by reconstruction from numpy's SVD.  With alpha = 0 the score is log(e + eps*)."""
    m = RNG.standard_normal((9, 6))
    u, sv, vt = np.linalg.svd(m, full_matrices=False)
    got = oracle.swift_layer_scores([sv], [1.7], 0.0)[0]
    for k in range(1, len(sv) + 1):
        resid = m - (u[:, :k] * sv[:k]) @ vt[:k]
        np.testing.assert_allclose(got[k - 1], np.log(np.e + np.sum(resid ** 2)), rtol=1e-12)


def test_swift_limits_and_monotone():
    """alpha = 1 gives beta at every rank; at full rank nothing is discarded, so the score
    is beta^alpha; the score never grows with the rank (less is discarded)."""
    sv = np.sort(RNG.random(7) * 3)[::-1]
    np.testing.assert_allclose(oracle.swift_layer_scores([sv], [2.5], 1.0)[0], 2.5, rtol=1e-15)
    for a in (0.0, 0.3, 0.8):
        s = oracle.swift_layer_scores([sv], [2.5], a)[0]
        np.testing.assert_allclose(s[-1], 2.5 ** a, rtol=1e-15)
        assert np.all(np.diff(s) <= 0)


# ----------------------------------------------------------------------------- factor codec
def test_rotation_golden():
    g = {ln.split(":")[0]: np.array(ln.split(":", 1)[1].split(), float) for ln in read_golden("hadamard_rotation.txt")}
    lr, rr = oracle.rotate_factors(np.array([[1.0, 2.0]], np.float32), np.array([[1.0], [2.0]], np.float32), [1, -1])
    np.testing.assert_allclose(lr[0], g["left"], rtol=1e-7)
    np.testing.assert_allclose(rr[:, 0], g["right"], rtol=1e-7)


def test_rotation_is_orthogonal_and_keeps_the_product():
    """R R^T = I; left' right' = left right up to the fp32 rounding of the factors."""
    r = 64
    signs = RNG.choice([-1.0, 1.0], r)
    rot = oracle.hadamard_rotation(r, signs)
    np.testing.assert_allclose(rot @ rot.T, np.eye(r), atol=1e-14)
    left = RNG.standard_normal((10, r)).astype(np.float32)
    right = RNG.standard_normal((r, 7)).astype(np.float32)
    lr, rr = oracle.rotate_factors(left, right, signs)
    prod = left.astype(np.float64) @ right.astype(np.float64)
    np.testing.assert_allclose(lr.astype(np.float64) @ rr.astype(np.float64), prod,
                               atol=64 * 2 ** -23 * np.abs(prod).max())


def test_rotation_spreads_an_outlier():
    """A row with one spike of size M (the outlier channels the rotation smooths) becomes
    a row whose every entry has magnitude M / sqrt(r): its max drops by sqrt(r)."""
    r = 256
    x = np.zeros((1, r), np.float32)
    x[0, 37] = 50.0
    lr, _ = oracle.rotate_factors(x, np.zeros((r, 1), np.float32), RNG.choice([-1.0, 1.0], r))
    np.testing.assert_allclose(np.abs(lr[0]), 50.0 / 16.0, rtol=1e-7)


def test_rtn_rows_is_the_token_quantiser_per_row():
    """Per-row RTN equals the QAW quantiser applied to rows: codes within +-127, each
    non-zero row reaches 127, reconstruction error within half a step."""
    x = RNG.standard_normal((6, 33)).astype(np.float32) * np.float32(3.0)
    x[2] = 0
    q, s = oracle.rtn_rows(x)
    assert q.dtype == np.int8 and np.all(np.abs(q.astype(int)) <= 127)
    for i in range(6):
        if i == 2:
            assert s[i] == 0 and np.all(q[i] == 0)
        else:
            assert np.abs(q[i].astype(int)).max() == 127
            assert np.all(np.abs(q[i].astype(np.float32) * s[i] - x[i]) <= s[i] / 2 * (1 + 1e-6))


# ----------------------------------------------------------------------------- low-rank FFN
def _int8_factor(rng, rows, cols):
    return rng.integers(-127, 128, (rows, cols)).astype(np.int8), rng.uniform(0.001, 0.02, rows).astype(np.float32)


def test_lowrank_ffn_golden():
    y = np.array(read_golden("lowrank_ffn.txt")[0].split(":")[1].split(), float)
    half = np.array([0.5], np.float32)
    gate = (np.array([[2, 4]], np.int8), half, np.array([[2], [0]], np.int8), np.array([0.5, 0.5], np.float32))
    up = (np.array([[2, 0]], np.int8), half, np.array([[2], [2]], np.int8), np.array([0.5, 0.5], np.float32))
    down = (np.array([[2, 2]], np.int8), half, np.array([[2], [4]], np.int8), np.array([0.5, 0.5], np.float32))
    np.testing.assert_allclose(oracle.lowrank_ffn(np.ones((1, 2)), gate, up, down)[0], y, rtol=1e-12)


def test_lowrank_ffn_equals_the_dense_ffn_of_the_product():
    """With each weight built explicitly as L R, the factored forward equals the dense
    SwiGLU FFN y = W_down (SiLU(W_gate x) * W_up x), evaluated here elementwise."""
    rng = np.random.default_rng(4)
    d, dff, r = 12, 20, 5
    g = (*_int8_factor(rng, r, d), *_int8_factor(rng, dff, r))
    u = (*_int8_factor(rng, r, d), *_int8_factor(rng, dff, r))
    dn = (*_int8_factor(rng, r, dff), *_int8_factor(rng, d, r))

    def dense(f):
        return (f[2].astype(np.float64) * f[3][:, None]) @ (f[0].astype(np.float64) * f[1][:, None])

    wg, wu, wd = dense(g), dense(u), dense(dn)
    x = rng.standard_normal((3, d))
    want = np.zeros((3, d))
    for t in range(3):
        zg, zu = wg @ x[t], wu @ x[t]
        h = np.array([z / (1.0 + math.exp(-z)) * v for z, v in zip(zg, zu)])
        want[t] = wd @ h
    np.testing.assert_allclose(oracle.lowrank_ffn(x, g, u, dn), want, rtol=1e-12, atol=1e-12)


def test_hybrid_ffn_equals_the_dense_ffn_of_the_assembled_weights():
    """Hybrid form: the full weights are assembled channel by channel (rows of W_gate and
    W_up, columns of W_down: low-rank channels from L R, dense ones from q * s), and the
    plain dense SwiGLU FFN of those weights, token by token, must equal the hybrid
    forward; with either group empty it reduces to the other one alone."""
    rng = np.random.default_rng(6)
    d, n_lr, n_dn, r = 10, 7, 5, 3
    g = (*_int8_factor(rng, r, d), *_int8_factor(rng, n_lr, r))
    u = (*_int8_factor(rng, r, d), *_int8_factor(rng, n_lr, r))
    dn = (*_int8_factor(rng, r, n_lr), *_int8_factor(rng, d, r))
    dense = (*_int8_factor(rng, n_dn, d), *_int8_factor(rng, n_dn, d), *_int8_factor(rng, d, n_dn))

    def lr(f):
        return (f[2].astype(np.float64) * f[3][:, None]) @ (f[0].astype(np.float64) * f[1][:, None])

    def rows(q, s):
        return q.astype(np.float64) * s.astype(np.float64)[:, None]

    wg = np.vstack([lr(g), rows(dense[0], dense[1])])
    wu = np.vstack([lr(u), rows(dense[2], dense[3])])
    wd = np.hstack([lr(dn), rows(dense[4], dense[5])])
    x = rng.standard_normal((4, d))
    want = np.zeros((4, d))
    for t in range(4):
        zg, zu = wg @ x[t], wu @ x[t]
        want[t] = wd @ np.array([z / (1.0 + math.exp(-z)) * v for z, v in zip(zg, zu)])
    np.testing.assert_allclose(oracle.hybrid_ffn(x, g, u, dn, dense), want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.hybrid_ffn(x, g, u, dn, None), oracle.lowrank_ffn(x, g, u, dn), rtol=1e-14)
    only_dense = np.zeros((4, d))
    for t in range(4):
        zg, zu = rows(dense[0], dense[1]) @ x[t], rows(dense[2], dense[3]) @ x[t]
        only_dense[t] = rows(dense[4], dense[5]) @ (zg / (1.0 + np.exp(-zg)) * zu)
    np.testing.assert_allclose(oracle.hybrid_ffn(x, dense=dense), only_dense, rtol=1e-12, atol=1e-12)


def test_silu_values():
    np.testing.assert_allclose(oracle.silu([0.0, 1.0, -1.0, 30.0]),
                               [0.0, 0.7310585786300049, -0.2689414213699951, 30.0], rtol=1e-12)


# --------------------------------------------------------------------------- FFN channel selection
@pytest.mark.parametrize("d_ff,d,r", [(7, 4, 2), (9, 5, 0), (6, 6, 3)])
def test_ffn_channel_error_is_the_mean_squared_preactivation_error(d_ff, d, r):
    """LASER 3, item Channel selection: a hidden channel's reconstruction error (reading:
    the expected squared error of its gate and up pre-activations over the calibration
    tokens) equals, token by token, the mean of (dW_gate a_t)_h^2 + (dW_up a_t)_h^2."""
    n = 200
    a = _spd_stream(n, d, 1.0, RNG)
    wg, wu = RNG.standard_normal((d_ff, d)), RNG.standard_normal((d_ff, d))
    xs = oracle.covariance_sum(a)
    fg = fu = None
    if r:
        rg = oracle.whiten_decompose(wg, xs, n, rank=r)
        ru = oracle.whiten_decompose(wu, xs, n, rank=r)
        fg, fu = (rg["left"], rg["right"]), (ru["left"], ru["right"])
    err = oracle.ffn_channel_errors(wg, wu, fg, fu, xs, n)
    dg = wg - (fg[0] @ fg[1] if r else 0.0)
    du = wu - (fu[0] @ fu[1] if r else 0.0)
    brute = np.zeros(d_ff)
    for t in range(n):
        brute += (dg @ a[t]) ** 2 + (du @ a[t]) ** 2
    np.testing.assert_allclose(err, brute / n, rtol=1e-10)
    # damping adds damping * ||dW[h]||^2 per projection
    errd = oracle.ffn_channel_errors(wg, wu, fg, fu, xs, n, damping=0.25)
    np.testing.assert_allclose(errd, err + 0.25 * (np.sum(dg ** 2, axis=1) + np.sum(du ** 2, axis=1)),
                               rtol=1e-10)


def test_ffn_channel_errors_sum_to_the_discarded_whitened_energy():
    """Summed over the channels, one projection's errors are its whitened truncation
    error (Eckart-Young in the whitened space): sum of the discarded sigma_tilde^2; at
    full rank every error vanishes."""
    n, d_ff, d, r = 300, 12, 8, 3
    a = _spd_stream(n, d, 1.2, RNG)
    xs = oracle.covariance_sum(a)
    wg, wu = RNG.standard_normal((d_ff, d)), RNG.standard_normal((d_ff, d))
    rg = oracle.whiten_decompose(wg, xs, n, rank=r)
    ru = oracle.whiten_decompose(wu, xs, n, rank=r)
    zero = np.zeros_like(wu)
    eg = oracle.ffn_channel_errors(wg, zero, (rg["left"], rg["right"]), None, xs, n)
    eu = oracle.ffn_channel_errors(zero, wu, None, (ru["left"], ru["right"]), xs, n)
    np.testing.assert_allclose(eg.sum(), np.sum(rg["sigma"][r:] ** 2), rtol=1e-10)
    np.testing.assert_allclose(eu.sum(), np.sum(ru["sigma"][r:] ** 2), rtol=1e-10)
    both = oracle.ffn_channel_errors(wg, wu, (rg["left"], rg["right"]), (ru["left"], ru["right"]), xs, n)
    np.testing.assert_allclose(both, eg + eu, rtol=1e-12)
    full_g = oracle.whiten_decompose(wg, xs, n, rank=d)
    full_u = oracle.whiten_decompose(wu, xs, n, rank=d)
    e0 = oracle.ffn_channel_errors(wg, wu, (full_g["left"], full_g["right"]), (full_u["left"], full_u["right"]), xs, n)
    assert np.max(np.abs(e0)) <= 1e-20 * np.max(oracle.ffn_channel_errors(wg, wu, None, None, xs, n))


def test_select_channels_rule():
    """The n smallest errors take the low-rank branch; equal errors go by channel index.
    Hand-derived: errors (0.5, 0.25, 0.5, 0, 0.25) order as 3, 1, 4, 0, 2."""
    order, low = oracle.select_channels([0.5, 0.25, 0.5, 0.0, 0.25], 3)
    assert order.tolist() == [3, 1, 4, 0, 2]
    assert low.tolist() == [0, 1, 0, 1, 1]
    order, low = oracle.select_channels([0.5, 0.25, 0.5, 0.0, 0.25], 0)
    assert low.sum() == 0
    order, low = oracle.select_channels([0.5, 0.25, 0.5, 0.0, 0.25], 5)
    assert low.sum() == 5
    err = RNG.random(50)
    err[10:20] = err[5]                          # ties
    order, low = oracle.select_channels(err, 17)
    assert sorted(order.tolist()) == list(range(50))
    assert low.sum() == 17
    assert np.max(err[low == 1]) <= np.min(err[low == 0])
    keys = [(err[h], h) for h in order]
    assert keys == sorted(keys)
