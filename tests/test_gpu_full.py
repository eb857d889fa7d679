"""GPU parity at the workloads' real widths (LLaMA-7B-class projections).

The HIP path runs at full size; the oracle checks sampled outputs it can compute one
by one (covariance entries as column dot products), or full results where its fp64
LAPACK run stays within about a minute on host cores.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

U32 = 2.0 ** -24
_T0 = [0.0]
_CAP = [None]


@pytest.fixture(autouse=True)
def _progress_past_capture(capsys):
    """These tests run for minutes: their progress lines go to the terminal even while
    pytest captures output (a run that prints nothing for minutes looks hung)."""
    _CAP[0] = capsys
    yield
    _CAP[0] = None


def step(msg):
    """Progress line for long full-size runs."""
    import time
    now = time.perf_counter()
    if not _T0[0]:
        _T0[0] = now
    line = f"  [{now - _T0[0]:7.1f}s] {msg}"
    if _CAP[0] is not None:
        with _CAP[0].disabled():
            print(line, flush=True)
    else:
        print(line, flush=True)


@pytest.fixture(scope="module")
def lrc():
    import curvature_aware_rank_amd as m
    return m


def dev():
    return torch.device("cuda:0")


def host(t):
    return t.detach().float().cpu().numpy()


def sampled_cov_check(c_gpu, a_host, rng, n_samples=1000, extra_bound=0.0):
    """Entries (i >= j) of the GPU covariance sum against fp64 column dot products."""
    d = a_host.shape[1]
    i = rng.integers(0, d, n_samples)
    j = rng.integers(0, d, n_samples)
    i, j = np.maximum(i, j), np.minimum(i, j)
    c = host(c_gpu)
    n = a_host.shape[0]
    worst = 0.0
    for ii, jj in zip(i, j):
        x = a_host[:, ii].astype(np.float64)
        y = a_host[:, jj].astype(np.float64)
        want = float(x @ y)
        mag = float(np.abs(x) @ np.abs(y))
        tol = (10 * math.sqrt(n) * U32 + extra_bound) * mag
        err = abs(float(c[ii, jj]) - want)
        worst = max(worst, err / tol)
    step(f"sampled covariance entries: worst error / tolerance = {worst:.3f}")
    assert worst <= 1.0, worst


def check_decomposition(sig, left, right, w, ref, rank, two_sided=False):
    """Decomposition at full size against the oracle's fp64 SVD route:
    * retained sigma relative error <= 1e-4, every sigma (tail included) within
      1e-4 sigma_1 absolute, and sigma^2 within 1e-5 sigma_1^2;
    * the K-FAC loss of the truncation;
    * principal angles <= 1e-3 rad between the leading left and right subspaces (whitened
      coordinates) wherever the spectral gap exceeds 1e-3 sigma_1;
    * isolated components (gap > 1e-3 sigma_1 on both sides): Left columns and Right rows
      elementwise (signs are canonical on both sides), within 2e-3 of the largest entry.
    Returns (subspaces checked, isolated components checked)."""
    s_ref = ref["sigma"]
    sig = sig.astype(np.float64)
    rel = np.abs(sig[:rank] - s_ref[:rank]) / s_ref[:rank]
    assert rel.max() <= 1e-4, rel.max()
    tail = np.abs(sig - s_ref).max() / s_ref[0]
    assert tail <= 1e-4, tail
    assert np.max(np.abs(sig ** 2 - s_ref ** 2)) <= 1e-5 * s_ref[0] ** 2
    step(f"sigma: retained rel {rel.max():.2e}, all |d sigma| / sigma_1 {tail:.2e}")
    lx, lg = ref["lx"], ref["lg"] if two_sided else None
    l64, r64 = left.astype(np.float64), right.astype(np.float64)
    dw = w.astype(np.float64) - l64 @ r64
    m = dw @ lx
    if lg is not None:
        m = lg.T @ m
    loss = 0.5 * np.linalg.norm(m) ** 2
    want = 0.5 * np.sum(s_ref[rank:] ** 2)
    assert abs(loss - want) <= 1e-3 * want + 1e-6 * 0.5 * s_ref[0] ** 2, (loss, want)
    u_gpu = lg.T @ l64 if lg is not None else l64          # = U~ S^1/2
    v_gpu = lx.T @ r64.T                                    # = V~ S^1/2
    checked = 0
    for jx in range(1, rank + 1):
        if jx < len(s_ref) and s_ref[jx - 1] - s_ref[jx] <= 1e-3 * s_ref[0]:
            continue
        for g, rr in ((u_gpu[:, :jx], ref["u"][:, :jx]), (v_gpu[:, :jx], ref["vt"][:jx].T)):
            q, _ = np.linalg.qr(g)
            cosines = np.linalg.svd(q.T @ rr, compute_uv=False)
            assert np.arccos(np.clip(cosines.min(), -1, 1)) <= 1e-3, jx
        checked += 1
    iso = [i for i in range(rank)
           if (i == 0 or s_ref[i - 1] - s_ref[i] > 1e-3 * s_ref[0]) and s_ref[i] - s_ref[i + 1] > 1e-3 * s_ref[0]]
    for i in iso:
        for got, want_v in ((l64[:, i], ref["left"][:, i]), (r64[i], ref["right"][i])):
            np.testing.assert_allclose(got, want_v, rtol=0, atol=2e-3 * np.abs(want_v).max())
    step(f"subspaces checked at {checked} gaps, {len(iso)} isolated components elementwise")
    return checked, len(iso)


def test_attention_projection_full(lrc):
    """4096 x 4096 weight, 65536 bf16 tokens with 1% outlier channels, G = I, r = 1024."""
    n, d, r = 65536, 4096, 1024
    rng = np.random.default_rng(1)
    a = synth.activation_stream(n, d, 1.0, 31, outlier_frac=0.01, dtype=torch.bfloat16, device=dev())
    w = synth.weight(d, d, 35, device=dev())
    cov = torch.zeros(d, d, device=dev())
    lrc.lrc_accumulate_cov(a, cov)
    sig, left, right, info = lrc.lrc_whiten_decompose(w, r, cov, n)
    assert int(info[0]) == 0
    step("GPU covariance + decomposition done")
    ah = host(a)
    sampled_cov_check(cov, ah, rng)
    x64 = oracle.covariance_sum(ah)
    step("oracle covariance done")
    ref = oracle.whiten_decompose(host(w), x64, n, rank=r)
    step("oracle decomposition done")
    checked, iso = check_decomposition(host(sig), host(left), host(right), host(w), ref, r)
    assert checked >= 10 and iso >= 10


@pytest.mark.parametrize("which", ["up", "down"])
def test_ffn_two_sided_qaw(lrc, which):
    """The FFN pair at full width, two-sided with int8-QAW activations, rank 2048 (half of
    min(d_out, d_in)): up 11008 x 4096 (the Gram on the 4096-wide input side) and down
    4096 x 11008 (output side; 11008-wide activation covariance and Cholesky).  16384
    tokens keep the oracle's fp64 covariances and SVD near a minute."""
    n, r = 16384, 2048
    cs = synth.workload_spec("ffn_pair_11008x4096", n_tokens=n)
    m = cs.matrices[0 if which == "up" else 1]
    a = synth.stream(cs, m.a_stream, device=dev())
    b = synth.stream(cs, m.b_stream, device=dev())
    w = synth.weight(m.d_out, m.d_in, 45 if which == "up" else 46, device=dev())
    xs = torch.zeros(m.d_in, m.d_in, device=dev())
    gs = torch.zeros(m.d_out, m.d_out, device=dev())
    ia = lrc.lrc_accumulate_cov(a, xs, quant=True)
    ib = lrc.lrc_accumulate_cov(b, gs)
    sig, left, right, info = lrc.lrc_whiten_decompose(w, r, xs, n, gs, n)
    assert int(info[0]) == 0 and int(ia[0]) == 0 and int(ib[0]) == 0
    step(f"GPU two-sided QAW decomposition of {which} done")
    ahat = oracle.qaw_fake_quant(host(a))[2]
    del a
    xsum = oracle.covariance_sum(ahat)
    del ahat
    gsum = oracle.covariance_sum(host(b))
    del b
    step("oracle covariances done")
    ref = oracle.whiten_decompose(host(w), xsum, n, gsum, n, rank=r)
    step("oracle decomposition done")
    checked, iso = check_decomposition(host(sig), host(left), host(right), host(w), ref, r, two_sided=True)
    assert checked >= 1


def test_ffn_full_token_covariances_sampled(lrc):
    """All 131072 tokens: QAW activation covariance (4096) and gradient covariance
    (11008), sampled entries against the oracle."""
    cs = synth.workload_spec("ffn_pair_11008x4096")
    rng = np.random.default_rng(2)
    a = synth.stream(cs, "a_up", device=dev())
    xs = torch.zeros(4096, 4096, device=dev())
    lrc.lrc_accumulate_cov(a, xs, quant=True)
    ahat = oracle.qaw_fake_quant(host(a))[2]
    del a
    sampled_cov_check(xs, ahat, rng, n_samples=1500, extra_bound=2.0 ** -15)
    del ahat
    b = synth.stream(cs, "b_up", device=dev())
    gs = torch.zeros(11008, 11008, device=dev())
    lrc.lrc_accumulate_cov(b, gs)
    sampled_cov_check(gs, host(b), rng, n_samples=1500)


def test_heads_full_allocation(lrc):
    """32 K heads + 32 V heads (128 x 4096 slices), one shared X from 65536 tokens,
    K-FAC scores, global allocation at 40% of the dense parameters."""
    n, d, hd = 65536, 4096, 128
    a = synth.activation_stream(n, d, 1.0, 131, outlier_frac=0.01, dtype=torch.bfloat16, device=dev())
    wk = synth.weight(d, d, 137, device=dev())
    wv = synth.weight(d, d, 139, device=dev())
    w3 = torch.cat([wk, wv], 0).view(64, hd, d)
    cov = torch.zeros(d, d, device=dev())
    lrc.lrc_accumulate_cov(a, cov)
    sig, left, right, info = lrc.lrc_whiten_decompose(w3, hd, cov, n)
    assert torch.all(info == 0)
    step("GPU 64-head batched decomposition done")
    scores = torch.cat([lrc.lrc_score_components(sigma=sig[h].contiguous(), mode="kfac")[0] for h in range(64)])
    offs = torch.arange(0, 64 * hd + 1, hd, dtype=torch.int64, device=dev())
    cost = torch.full((64,), hd + d, dtype=torch.int64, device=dev())
    budget = int(0.4 * 2 * d * d)
    order, n_kept, ranks, kept, ainfo = lrc.lrc_allocate_ranks(scores, offs, cost, budget)
    assert int(ainfo[0]) == 0
    sc = host(scores)
    lst = [sc[h * hd:(h + 1) * hd] for h in range(64)]
    ref_alloc = oracle.allocate(lst, [hd + d] * 64, budget)
    assert host(order).astype(np.int64).tolist() == ref_alloc[0].tolist()
    assert int(n_kept[0]) == ref_alloc[1] and host(ranks).tolist() == ref_alloc[2].tolist()
    step("allocation bit-exact on identical scores")
    # decompositions of sampled heads against the oracle (shared Cholesky factor)
    x64 = oracle.covariance_sum(host(a)) / n
    lx, inf = oracle.cholesky_lower(x64)
    assert inf == 0
    wh = host(w3)
    s_gpu = host(sig)
    ref_scores = []
    for h in range(64):
        s = np.linalg.svd(wh[h].astype(np.float64) @ lx, compute_uv=False)
        ref_scores.append(oracle.kfac_scores(s))
        rel = np.abs(s_gpu[h][:64] - s[:64]) / s[:64]
        assert rel.max() <= 1e-4, (h, rel.max())
        assert np.max(np.abs(s_gpu[h].astype(np.float64) ** 2 - s ** 2)) <= 1e-5 * s[0] ** 2
    # end to end: the oracle's own fp64 scores give the same kept set except inside the
    # band of components whose key lies within the score error of the cut key
    step("64 head spectra checked")
    ref_own = oracle.allocate([x.astype(np.float32) for x in ref_scores], [hd + d] * 64, budget)
    flat_ref = np.concatenate(ref_scores)
    kept_gpu = host(kept).astype(bool)
    kept_ref = ref_own[3].astype(bool)
    diff = np.nonzero(kept_gpu != kept_ref)[0]
    if len(diff):
        cut = flat_ref[ref_own[0][ref_own[1] - 1]]
        band = np.abs(flat_ref[diff] - cut) <= 1e-4 * cut
        assert band.all(), (len(diff), int(band.sum()))


def fisher_error_bound(s_gpu, s_ref, sig_gpu, sig_ref):
    """Per-component bound on |s_gpu - s_ref| for the empirical-Fisher scores of one matrix
    (every component kept).  Two sources:
    * the projections and sums (bf16 activations exact, factors split hi/lo, fp32 sums):
      1e-3 of the score itself;
    * the singular vectors: both sides decompose the same whitened weight up to a
      perturbation E of norm eta * sigma_1, which turns component i's vectors by an angle
      up to eta sigma_1 / gap_i (Wedin), mixing it with its neighbours; the score, a
      product of two squared projections, then moves by up to ~8 such angles times the
      larger of the neighbouring scores.  eta is taken as 10x the largest sigma error
      (a sigma moves by at most ||E||, so that error bounds ||E|| from below).
    Returns (bound, eta, gap/sigma_1)."""
    s1 = sig_ref[0]
    eta = max(10.0 * np.abs(sig_gpu.astype(np.float64) - sig_ref).max() / s1, 1e-7)
    k = len(s_ref)
    gap = np.full(k, np.inf)
    gap[:-1] = np.minimum(gap[:-1], sig_ref[:-1] - sig_ref[1:])
    gap[1:] = np.minimum(gap[1:], sig_ref[:-1] - sig_ref[1:])
    ang = np.minimum(1.0, eta * s1 / np.maximum(gap, 1e-300))
    nb = s_ref.copy()
    nb[1:] = np.maximum(nb[1:], s_ref[:-1])
    nb[:-1] = np.maximum(nb[:-1], s_ref[1:])
    return 1e-3 * s_ref + 8.0 * ang * nb, eta, gap / s1


def test_decoder_stack_full(lrc):
    """The 32-layer decoder stack end to end on the GPU: per layer four activation streams
    and seven gradient streams of 32768 tokens (covariance scale x0.1..x10 per layer),
    activation-only whitening of q, k, v, o, gate, up and down with every component
    computed, empirical-Fisher scores of all 917,504 components, and one global
    sort-and-truncate at 60% of the dense parameter count.
    (i) The allocation is bit-exact against the oracle's allocator on the GPU's scores.
    (ii) Layer 0 against the oracle: its seven decompositions (at the ranks the allocation
    gave them), every one of its 28,672 Fisher scores within fisher_error_bound, and the
    allocation of the layer's own pool from the oracle's fp64 scores, which may differ
    from the GPU's only inside the band of components whose key lies within the measured
    score error of the cut key."""
    cs = synth.workload_spec("decoder_stack_32_layers")
    n = cs.n_tokens
    all_scores, costs, sizes, infos = [], [], [], []
    layer0 = {}
    for layer in range(32):
        streams = {key: synth.stream(cs, key, layer=layer, device=dev())
                   for key in ("attn_in", "o_in", "mlp_in", "down_in")}
        covs = {}
        for key, a in streams.items():
            c = torch.zeros(a.shape[1], a.shape[1], device=dev())
            infos.append(lrc.lrc_accumulate_cov(a, c))
            covs[key] = c
        if layer == 0:
            layer0["streams"] = {key: host(a) for key, a in streams.items()}
        for mi, m in enumerate(cs.matrices):
            w = synth.weight(m.d_out, m.d_in, 1000 + 10 * layer + mi, device=dev())
            k = min(m.d_out, m.d_in)
            sig, left, right, info = lrc.lrc_whiten_decompose(w, k, covs[m.a_stream], n)
            b = synth.stream(cs, m.b_stream, layer=layer, device=dev())
            s, sinfo = lrc.lrc_score_components(left, right, A=streams[m.a_stream], B=b)
            infos += [info, sinfo]
            all_scores.append(s)
            costs.append(m.d_out + m.d_in)
            sizes.append(k)
            if layer == 0:
                layer0[m.name] = dict(w=host(w), b=host(b), sig=host(sig), left=host(left), right=host(right),
                                      s=host(s))
            del b, left, right
        del streams, covs
        torch.cuda.synchronize()
        step(f"layer {layer}: 4 covariances, 7 decompositions, 7 x 4096 Fisher scores")
    assert all(int(i.max()) == 0 and int(i.min()) == 0 for i in infos)
    scores = torch.cat(all_scores)
    assert scores.numel() == 917504
    offs_h = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    offs = torch.tensor(offs_h, dtype=torch.int64, device=dev())
    cost_t = torch.tensor(costs, dtype=torch.int64, device=dev())
    dense = 32 * sum(m.d_out * m.d_in for m in cs.matrices)
    budget = int(0.6 * dense)
    assert budget == 3885603225
    order, n_kept, ranks, kept, ainfo = lrc.lrc_allocate_ranks(scores, offs, cost_t, budget)
    torch.cuda.synchronize()
    assert int(ainfo[0]) == 0
    step(f"GPU allocation: {int(n_kept[0])} of 917504 components kept")
    # (i) bit-exact on the same fp32 score array
    sc = host(scores)
    lst = [sc[offs_h[i]:offs_h[i + 1]] for i in range(len(sizes))]
    ref = oracle.allocate(lst, costs, budget)
    assert host(order).astype(np.int64).tolist() == ref[0].tolist()
    assert int(n_kept[0]) == ref[1]
    assert host(ranks).tolist() == ref[2].tolist()
    assert np.array_equal(host(kept).astype(np.uint8), ref[3])
    step("(i) allocation bit-exact against the oracle on the GPU's 917504 scores")
    # (ii) layer 0 against the oracle
    ranks0 = host(ranks)[:7]
    s_gpu0, s_ref0 = [], []
    for mi, m in enumerate(cs.matrices):
        d = layer0[m.name]
        a = layer0["streams"][m.a_stream]
        refd = oracle.whiten_decompose(d["w"], oracle.covariance_sum(a), n, rank=min(m.d_out, m.d_in))
        r_m = max(int(ranks0[mi]), 1)
        check_decomposition(d["sig"], d["left"][:, :r_m], d["right"][:r_m], d["w"],
                            dict(refd, left=refd["left"][:, :r_m], right=refd["right"][:r_m]), r_m)
        f_ref = oracle.fisher_scores(a, d["b"], refd["left"], refd["right"])
        bound, eta, gap = fisher_error_bound(d["s"], f_ref, d["sig"], refd["sigma"])
        err = np.abs(d["s"].astype(np.float64) - f_ref)
        well = gap > 100 * eta
        step(f"layer 0 {m.name}: rank {r_m}; eta {eta:.1e}; Fisher error / bound max {np.max(err / bound):.3f}; "
             f"{int(well.sum())} components with gap > 100 eta sigma_1, their max relative error "
             f"{np.max(err[well] / f_ref[well]) if well.any() else 0.0:.2e}")
        assert np.all(err <= bound), (m.name, int(np.argmax(err / bound)), float(np.max(err / bound)))
        s_gpu0.append(d["s"])
        s_ref0.append(f_ref)
    # the layer's own pool at 60% of its dense parameters: GPU scores vs the oracle's
    costs0 = [m.d_out + m.d_in for m in cs.matrices]
    budget0 = int(0.6 * sum(m.d_out * m.d_in for m in cs.matrices))
    g_alloc = oracle.allocate(s_gpu0, costs0, budget0)
    o_alloc = oracle.allocate([x.astype(np.float32) for x in s_ref0], costs0, budget0)
    flat_ref = np.concatenate(s_ref0)
    flat_gpu = np.concatenate(s_gpu0).astype(np.float64)
    cost_item = np.concatenate([np.full(len(x), c, dtype=np.float64) for x, c in zip(s_ref0, costs0)])
    key_ref = flat_ref / cost_item
    cut = key_ref[o_alloc[0][o_alloc[1] - 1]]
    near = np.abs(key_ref - cut) <= 0.5 * cut
    delta = float(np.max(np.abs(flat_gpu[near] - flat_ref[near]) / flat_ref[near]))
    diff = np.nonzero(g_alloc[3] != o_alloc[3])[0]
    band = np.abs(key_ref[diff] - cut) <= 2.0 * delta * cut
    step(f"(ii) layer 0 pool: {len(diff)} components allocated differently from the oracle's own scores, "
         f"all within {2 * delta:.2e} of the cut key: {bool(band.all())}")
    assert band.all(), (len(diff), int(band.sum()))


def test_ffn_channel_selection_full(lrc):
    """FFN pair width: gate and up 11008 x 4096 at rank 2048 (the pages' rank ratio 0.5),
    the covariance of a power-law 4096-wide stream.  Sampled channels' errors against the
    oracle's quadratic form dW[h] X dW[h]^T (fp64, one channel at a time); the order and
    selection bit-exact against the oracle's rule on the GPU's errors.  The factors are
    seeded fp32 matrices (the selection step takes any factors; their optimality is the
    decomposition's business)."""
    d_ff, d, r, n = 11008, 4096, 2048, 16384
    rng = np.random.default_rng(11)
    step("inputs")
    a = synth.activation_stream(n, d, 1.0, 51, dtype=torch.bfloat16, device=dev())
    xs = torch.zeros(d, d, device=dev())
    lrc.lrc_accumulate_cov(a, xs)
    xs_np = xs.cpu().numpy()
    del a
    wg = rng.standard_normal((d_ff, d), dtype=np.float32) / np.float32(64.0)
    wu = rng.standard_normal((d_ff, d), dtype=np.float32) / np.float32(64.0)
    fac = [(rng.standard_normal((d_ff, r), dtype=np.float32) / np.float32(64.0),
            rng.standard_normal((r, d), dtype=np.float32) / np.float32(64.0)) for _ in range(2)]
    t = lambda x: torch.from_numpy(x).to(dev())
    step("select on the GPU")
    err, order, low, info = lrc.lrc_ffn_select_channels(t(wg), t(wu), (t(fac[0][0]), t(fac[0][1])),
                                                        (t(fac[1][0]), t(fac[1][1])), xs, n, d_ff // 2, 1e-3)
    assert int(info.item()) == 0
    e = err.cpu().numpy()
    step("oracle on sampled channels")
    hs = rng.choice(d_ff, 24, replace=False)
    x = np.tril(xs_np.astype(np.float64))
    x = x + np.tril(x, -1).T
    x = x / n + 1e-3 * np.eye(d)
    for h in hs:
        tot = 0.0
        for w, (lf, rf) in zip((wg, wu), fac):
            dw = w[h].astype(np.float64) - lf[h].astype(np.float64) @ rf.astype(np.float64)
            tot += dw @ x @ dw
        np.testing.assert_allclose(e[h], tot, rtol=5e-5)
    o_ord, o_low = oracle.select_channels(e, d_ff // 2)
    assert np.array_equal(order.cpu().numpy().astype(np.int64), o_ord)
    assert np.array_equal(low.cpu().numpy(), o_low)
    step("done")
