"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/lrc.h declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "curvature_aware_rank_amd", "liblrc.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="liblrc.so not built")

EINVAL, EDTYPE, EWORKSPACE = 1, 2, 3
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation returns first


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "lrc.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lrc_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import curvature_aware_rank_amd as m   # sets argtypes / restypes
    return m.lib


def test_every_declared_symbol_is_exported(lib):
    names = declared_symbols()
    assert {"lrc_accumulate_cov", "lrc_whiten_decompose", "lrc_score_components", "lrc_allocate_ranks"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(8):
        assert lib.lrc_status_string(code).decode().startswith("LRC_")


def test_accumulate_cov_validation(lib):
    f = lib.lrc_accumulate_cov
    # (A, dt, n, d, lda, C, ldc, flags, info, ws, ws_bytes, stream)
    assert f(FAKE, 7, 10, 4, 4, FAKE, 4, 0, None, FAKE, 1 << 30, None) == EDTYPE          # dtype
    assert f(FAKE, 1, 10, 4, 4, FAKE, 4, 0x8, None, FAKE, 1 << 30, None) == EDTYPE        # flags
    assert f(None, 1, 10, 4, 4, FAKE, 4, 0, None, FAKE, 1 << 30, None) == EINVAL          # A null
    assert f(FAKE, 1, 10, 4, 4, None, 4, 0, None, FAKE, 1 << 30, None) == EINVAL          # C null
    assert f(FAKE, 1, 10, 4, 3, FAKE, 4, 0, FAKE, FAKE, 1 << 30, None) == EINVAL          # lda < d
    assert f(FAKE, 1, 10, 4, 4, FAKE, 3, 0, FAKE, FAKE, 1 << 30, None) == EINVAL          # ldc < d
    assert f(FAKE, 1, -1, 4, 4, FAKE, 4, 0, None, FAKE, 1 << 30, None) == EINVAL          # n < 0
    assert f(None, 1, 0, 4, 4, FAKE, 4, 0, None, None, 0, None) == 0                      # empty: no-op
    need = lib.lrc_accumulate_cov_workspace(1, 4096, 256, 0)
    assert need > 0
    assert f(FAKE, 1, 4096, 256, 256, FAKE, 256, 0, FAKE, FAKE, need - 1, None) == EWORKSPACE
    # QAW needs more scratch than plain accumulation
    assert lib.lrc_accumulate_cov_workspace(1, 4096, 256, 1) > need


def test_whiten_decompose_validation(lib):
    f = lib.lrc_whiten_decompose
    ok = dict(W=FAKE, d_out=8, d_in=6, ldw=6, batch=1, stride_w=48, X=FAKE, ldx=6, nx=10, G=None, ldg=0, ng=0,
              rank=3, damping=0.0, sigma=FAKE, left=FAKE, right=FAKE, info=FAKE)

    def call(ws_bytes=1 << 40, **over):
        a = dict(ok, **over)
        return f(a["W"], a["d_out"], a["d_in"], a["ldw"], a["batch"], a["stride_w"], a["X"], a["ldx"], a["nx"],
                 a["G"], a["ldg"], a["ng"], a["rank"], a["damping"], a["sigma"], a["left"], a["right"], a["info"],
                 FAKE, ws_bytes, None)

    assert call(W=None) == EINVAL
    assert call(rank=7) == EINVAL            # rank > min(d_out, d_in)
    assert call(rank=-1) == EINVAL
    assert call(ldw=5) == EINVAL
    assert call(ldx=5) == EINVAL
    assert call(nx=0) == EINVAL
    assert call(G=FAKE, ldg=8, ng=0) == EINVAL
    assert call(damping=-1.0) == EINVAL
    assert call(batch=2, stride_w=10) == EINVAL
    assert call(left=None) == EINVAL
    need = lib.lrc_whiten_decompose_workspace(8, 6, 1, 3, 1, 0)
    assert need > 0
    assert call(ws_bytes=need - 1) == EWORKSPACE


def test_whiten_decompose_strided_validation(lib):
    f = lib.lrc_whiten_decompose_strided
    ok = dict(W=FAKE, d_out=8, d_in=6, ldw=6, batch=3, stride_w=48, X=FAKE, ldx=6, sx=36, nx=10, G=FAKE, ldg=8,
              sg=64, ng=10, rank=3, damping=0.0, sigma=FAKE, left=FAKE, right=FAKE, info=FAKE)

    def call(ws_bytes=1 << 40, **over):
        a = dict(ok, **over)
        return f(a["W"], a["d_out"], a["d_in"], a["ldw"], a["batch"], a["stride_w"], a["X"], a["ldx"], a["sx"],
                 a["nx"], a["G"], a["ldg"], a["sg"], a["ng"], a["rank"], a["damping"], a["sigma"], a["left"],
                 a["right"], a["info"], FAKE, ws_bytes, None)

    assert call(sx=35) == EINVAL             # per-slice X sums overlap
    assert call(sg=63) == EINVAL             # per-slice G sums overlap
    assert call(sx=-36) == EINVAL
    assert call(ldx=5) == EINVAL
    assert call(G=None, ldg=0, ng=0, nx=0) == EINVAL
    ws = lib.lrc_whiten_decompose_strided_workspace
    per, shared = ws(8, 6, 3, 3, 3, 3), ws(8, 6, 3, 3, 1, 1)
    assert per > shared > 0                  # one Cholesky factor per slice
    assert shared == lib.lrc_whiten_decompose_workspace(8, 6, 3, 3, 1, 1)
    assert ws(8, 6, 3, 3, 2, 1) == 0 and ws(8, 6, 3, 3, -1, 0) == 0   # slices: 0, 1 or batch
    assert call(ws_bytes=per - 1) == EWORKSPACE
    assert call(sx=0, sg=0, ws_bytes=shared - 1) == EWORKSPACE


def test_score_components_validation(lib):
    f = lib.lrc_score_components
    # (A, B, dt, n, d_in, d_out, left, right, sigma, k, flags, accumulate, finalize, n_total, scores, info,
    #  ws, ws_bytes, stream)
    assert f(FAKE, FAKE, 1, 10, 4, 4, FAKE, FAKE, None, 4, 0x3, 0, 1, 10, FAKE, None, FAKE, 1 << 30, None) == EDTYPE
    assert f(FAKE, FAKE, 1, 10, 4, 4, FAKE, FAKE, None, 0, 0x1, 0, 1, 10, FAKE, None, FAKE, 1 << 30, None) == EINVAL
    assert f(None, None, 0, 0, 4, 4, FAKE, FAKE, None, 4, 0x2, 0, 1, 1, FAKE, FAKE, None, 0, None) == EINVAL  # no sigma
    assert f(FAKE, FAKE, 1, 10, 4, 4, FAKE, FAKE, None, 4, 0x1, 0, 1, 0, FAKE, FAKE, FAKE, 1 << 30, None) == EINVAL
    need = lib.lrc_score_components_workspace(1000, 4, 4, 4, 0x1)
    assert f(FAKE, FAKE, 1, 1000, 4, 4, FAKE, FAKE, None, 4, 0x1, 0, 1, 1000, FAKE, None, FAKE, need - 1,
             None) == EWORKSPACE


def test_allocate_ranks_validation(lib):
    f = lib.lrc_allocate_ranks
    assert f(FAKE, FAKE, FAKE, 0, 10, 5, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == EINVAL
    assert f(FAKE, FAKE, FAKE, 2, 10, -1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == EINVAL
    assert f(FAKE, None, FAKE, 2, 10, 5, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == EINVAL
    need = lib.lrc_allocate_ranks_workspace(2, 10)
    assert f(FAKE, FAKE, FAKE, 2, 10, 5, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == EWORKSPACE
    # order may be null (the cut is then selected without sorting); the mask may not
    assert f(FAKE, FAKE, FAKE, 2, 10, 5, None, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == EWORKSPACE
    assert f(FAKE, FAKE, FAKE, 2, 10, 5, None, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None) == EINVAL


def test_rank_scores_validation(lib):
    f = lib.lrc_rank_scores
    assert f(FAKE, FAKE, 2, 10, FAKE, 0.5, 0x3, FAKE, FAKE, None) == EDTYPE     # two modes
    assert f(FAKE, FAKE, 2, 10, FAKE, 0.5, 0x0, FAKE, FAKE, None) == EDTYPE     # no mode
    assert f(FAKE, FAKE, 0, 10, FAKE, 0.5, 0x1, FAKE, FAKE, None) == EINVAL     # n_mat 0
    assert f(FAKE, FAKE, 2, -1, FAKE, 0.5, 0x1, FAKE, FAKE, None) == EINVAL     # n_items < 0
    assert f(FAKE, None, 2, 10, FAKE, 0.5, 0x1, FAKE, FAKE, None) == EINVAL     # offsets null
    assert f(FAKE, FAKE, 2, 10, FAKE, 1.5, 0x2, FAKE, FAKE, None) == EINVAL     # alpha > 1
    assert f(FAKE, FAKE, 2, 10, FAKE, -0.1, 0x2, FAKE, FAKE, None) == EINVAL    # alpha < 0
    assert f(None, FAKE, 2, 10, FAKE, 0.5, 0x1, FAKE, FAKE, None) == EINVAL     # sigma null


def test_rotate_quantize_validation(lib):
    f = lib.lrc_rotate_quantize
    args = [FAKE, FAKE, 8, 4, 6, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 30, None]

    def call(**over):
        a = list(args)
        for i, v in over.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a3=6) == EINVAL          # r not a power of two
    assert call(a3=0) == EINVAL
    assert call(a3=16384) == EINVAL      # r above the LDS row
    assert call(a2=0) == EINVAL          # d_out
    assert call(a4=-1) == EINVAL         # d_in
    assert call(a5=None) == EINVAL       # signs
    assert call(a6=None) == EINVAL       # q_left
    need = lib.lrc_rotate_quantize_workspace(8, 4, 6)
    assert need > 0 and call(a13=need - 1) == EWORKSPACE
    g = lib.lrc_quantize_rows
    assert g(FAKE, 4, 8, 7, FAKE, FAKE, None) == EINVAL   # ldx < cols
    assert g(FAKE, 0, 8, 8, FAKE, FAKE, None) == EINVAL
    assert g(None, 4, 8, 8, FAKE, FAKE, None) == EINVAL


def test_lowrank_ffn_validation(lib):
    f = lib.lrc_lowrank_ffn
    ok = [FAKE, 1, 64, 96, FAKE, FAKE, FAKE, FAKE, 32, FAKE, FAKE, FAKE, FAKE, 32, FAKE, FAKE, FAKE, FAKE, 32, FAKE,
          FAKE, 1 << 30, None]

    def call(**over):
        a = list(ok)
        for i, v in over.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a0=None) == EINVAL          # x
    assert call(a2=60) == EINVAL            # d not a multiple of 16
    assert call(a8=20) == EINVAL            # rg not a multiple of 16
    assert call(a18=0) == EINVAL            # rd
    assert call(a1=0) == EINVAL             # n_tok
    assert call(a8=10240, a13=10240) == EINVAL   # a latent too large for LDS
    assert call(a4=ctypes.c_void_p(0x1008)) == EINVAL   # q_rg not 16-byte aligned
    need = lib.lrc_lowrank_ffn_workspace(1, 96, 32, 32, 32)
    assert need > 0 and call(a21=need - 1) == EWORKSPACE


def test_hybrid_ffn_validation(lib):
    f = lib.lrc_hybrid_ffn
    ok = [FAKE, 1, 64, 96, FAKE, FAKE, FAKE, FAKE, 32, FAKE, FAKE, FAKE, FAKE, 32, FAKE, FAKE, FAKE, FAKE, 32, 48,
          FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None]

    def call(**over):
        a = list(ok)
        for i, v in over.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a0=None) == EINVAL          # x
    assert call(a26=None) == EINVAL         # y
    assert call(a3=0, a19=0) == EINVAL      # no channels at all
    assert call(a19=40) == EINVAL           # n_dense not a multiple of 16
    assert call(a2=60) == EINVAL            # d not a multiple of 16
    assert call(a20=None) == EINVAL         # q_gd with dense channels
    assert call(a24=ctypes.c_void_p(0x1008)) == EINVAL   # q_dd not 16-byte aligned
    assert call(a8=20) == EINVAL            # rg not a multiple of 16 (low-rank part)
    assert call(a1=1 << 20, a19=1 << 12) == EINVAL       # n_tok * n_dense too large
    need = lib.lrc_hybrid_ffn_workspace(1, 96, 32, 32, 32, 48)
    assert need > lib.lrc_lowrank_ffn_workspace(1, 96, 32, 32, 32)
    assert call(a28=need - 1) == EWORKSPACE
    # dense only: the factor pointers may be null
    assert lib.lrc_hybrid_ffn_workspace(1, 0, 0, 0, 0, 48) > 0
    assert call(a3=0, a4=None, a5=None, a6=None, a7=None, a8=0, a28=0) == EWORKSPACE


def test_ffn_select_channels_validation(lib):
    f = lib.lrc_ffn_select_channels
    ok = [FAKE, FAKE, 40, 16, 16, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 16, 100, 0.0, 10, FAKE, FAKE, FAKE, FAKE,
          FAKE, 1 << 30, None]

    def call(**over):
        a = list(ok)
        for i, v in over.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a0=None) == EINVAL          # w_gate
    assert call(a10=None) == EINVAL         # Xsum
    assert call(a4=15) == EINVAL            # ldw < d
    assert call(a11=15) == EINVAL           # ldx < d
    assert call(a12=0) == EINVAL            # n_x
    assert call(a9=17) == EINVAL            # r > min(d_ff, d)
    assert call(a9=-1) == EINVAL
    assert call(a14=41) == EINVAL           # n_lowrank > d_ff
    assert call(a13=-1.0) == EINVAL         # damping
    assert call(a5=None) == EINVAL          # factors needed for r > 0
    assert call(a9=0, a5=None, a6=None, a7=None, a8=None, a20=0, a19=None) == EWORKSPACE   # r = 0: no factors
    need = lib.lrc_ffn_select_channels_workspace(40, 16)
    assert need > 0 and call(a20=need - 1) == EWORKSPACE


def test_profile_session_without_work(lib):
    # no kernel launched: the session records nothing and out-of-range queries fail
    assert lib.lrc_profile_start() == 0
    assert lib.lrc_profile_stop() == 0
    assert lib.lrc_profile_kernels() == 0
    assert lib.lrc_profile_kernel(0, None, None, None, None, None) == EINVAL
