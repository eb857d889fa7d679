"""The allocation-free allocator entry point (lrc_allocate_ranks_noalloc) against the
workspace entry point (lrc_allocate_ranks), both called through the C ABI on the same
inputs: identical order, n_kept, ranks, kept_mask and info (integer results, bit for
bit), on two calls in a row with the second on a smaller pool, and the size limit
reported as LRC_EWORKSPACE; and the same entry point without the order (the selected cut)
against the sort."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lrc():
    import curvature_aware_rank_amd as m
    return m


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _inputs(rng, n_mat, per_max, dev, tie_heavy):
    sizes = rng.integers(0, per_max, n_mat)
    costs = rng.integers(1000, 16000, n_mat).astype(np.int64)
    scores = (rng.standard_exponential(int(sizes.sum())) ** 2).astype(np.float32)
    if tie_heavy:
        scores = np.round(scores * 8).astype(np.float32)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    budget = int(0.5 * float((costs * sizes).sum()))
    return (torch.tensor(scores, device=dev), torch.tensor(offs, device=dev), torch.tensor(costs, device=dev),
            n_mat, int(sizes.sum()), budget)


def _outputs(M, n_mat, dev):
    return (torch.full((max(M, 1),), -1, dtype=torch.int32, device=dev), torch.full((1,), -1, dtype=torch.int64,
            device=dev), torch.full((n_mat,), -1, dtype=torch.int32, device=dev),
            torch.full((max(M, 1),), 9, dtype=torch.uint8, device=dev), torch.full((1,), -1, dtype=torch.int32,
                                                                                  device=dev))


def _run_both(lrc, inp, dev):
    scores, offs, cost, n_mat, M, budget = inp
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ref = _outputs(M, n_mat, dev)
    ws = torch.empty(max(int(lrc.lib.lrc_allocate_ranks_workspace(n_mat, M)), 1), dtype=torch.uint8, device=dev)
    st = lrc.lib.lrc_allocate_ranks(_p(scores), _p(offs), _p(cost), n_mat, M, budget, *[_p(t) for t in ref],
                                    _p(ws), ws.numel(), stream)
    assert st == 0
    got = _outputs(M, n_mat, dev)
    torch.cuda.synchronize()
    st = lrc.lib.lrc_allocate_ranks_noalloc(_p(scores), _p(offs), _p(cost), n_mat, M, budget, *[_p(t) for t in got],
                                            stream)
    assert st == 0
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    return ref


def test_noalloc_matches_workspace_entry_point(lrc):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(5)
    # the decoder stack's pool size first (917,504 items in 224 matrices), then a smaller one
    big = _inputs(rng, 224, 8192, dev, tie_heavy=True)
    assert big[4] > 800_000
    r1 = _run_both(lrc, big, dev)
    assert int(r1[4][0]) == 0 and int(r1[1][0]) > 0
    small = _inputs(rng, 9, 700, dev, tie_heavy=False)
    r2 = _run_both(lrc, small, dev)
    assert int(r2[4][0]) == 0


def test_noalloc_without_order_matches_sort(lrc):
    """order = NULL (the cut selected without sorting) through the allocation-free entry
    point: n_kept, ranks, kept_mask and info equal the workspace entry point's sort, on
    two calls in a row with the second on a smaller pool."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(6)
    for inp in (_inputs(rng, 224, 8192, dev, tie_heavy=True), _inputs(rng, 9, 700, dev, tie_heavy=False)):
        scores, offs, cost, n_mat, M, budget = inp
        ref = _run_both(lrc, inp, dev)
        got = _outputs(M, n_mat, dev)
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        st = lrc.lib.lrc_allocate_ranks_noalloc(_p(scores), _p(offs), _p(cost), n_mat, M, budget, None,
                                                *[_p(t) for t in got[1:]], stream)
        assert st == 0
        torch.cuda.synchronize()
        assert int(got[0][0]) == -1   # order untouched
        for a, b in zip(ref[1:], got[1:]):
            assert torch.equal(a, b)


def test_noalloc_limit(lrc):
    dev = torch.device("cuda:0")
    cap = int(lrc.lib.lrc_allocate_ranks_noalloc_max_items())
    assert cap == 1 << 21
    scores = torch.zeros(1, device=dev)
    offs = torch.tensor([0, cap + 1], dtype=torch.int64, device=dev)
    cost = torch.ones(1, dtype=torch.int64, device=dev)
    outs = _outputs(1, 1, dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # rejected on the host before any kernel could read past the one-element buffers
    assert lrc.lib.lrc_allocate_ranks_noalloc(_p(scores), _p(offs), _p(cost), 1, cap + 1, 10,
                                              *[_p(t) for t in outs], stream) == lrc.LRC_EWORKSPACE
