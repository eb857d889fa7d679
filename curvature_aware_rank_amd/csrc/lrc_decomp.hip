// lrc_whiten_decompose: Cholesky -> whitening -> Gram + eigensolve -> back-map.
//
// LASER technical summary, Methodology 1 (Transformation): W~ = S_x W S_g with Cholesky
// factors, SVD of W~, truncation, factors mapped back to the original space.  In this
// library's out x in orientation that is W~ = L_g^T W L_x.  Swift-SVD technical summary
// 2A: the singular vectors come from one eigendecomposition of the aggregated covariance
// of the outputs (here the Gram of W~ on its smaller side); the other side follows from
// W~ itself, so only products with W (never a second decomposition) are needed:
//   Gram on the output side (k = d_out):  Left = L_g^-T U S^1/2,  Right = S^-1/2 (L_g U)^T W
//   Gram on the input side  (k = d_in) :  Right = S^1/2 V^T L_x^-1, Left = W (L_x V) S^-1/2
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "lrc_dense.h"

namespace lrc {
namespace {

// Eigensolver choice: a single Gram goes through tridiagonalisation + inverse iteration
// (O(k^3) once, a fixed number of launches); batches of Grams through block Jacobi, whose
// rounds process every item of the batch at once (its fixed sweep count costs more
// launches than one tridiagonalisation for a single Gram of any size).
// LRC_EIGENSOLVER=jacobi|tridiag overrides the choice (tridiag only applies to batch 1).
// Eigensolver routing: a single Gram, or a batch of large ones (reduced together, then
// solved slice after slice), takes the tridiagonal route; a batch of small
// Grams (per-head slices) takes the batched block-Jacobi solver, which handles every item
// of the batch in each of its launches.  LRC_EIGENSOLVER=jacobi or =tridiag forces one.
constexpr int64_t TRI_BATCH_MIN_K = 384;
bool use_tridiag(int64_t k, int64_t batch) {
  const char* e = getenv("LRC_EIGENSOLVER");
  if (e && strcmp(e, "jacobi") == 0) return false;
  if (e && strcmp(e, "tridiag") == 0) return true;
  return batch == 1 || k >= TRI_BATCH_MIN_K;
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
  if (i < n) p[i] = v;
}

// After a failed Cholesky (a pivot of X or G not positive) the whitened weight holds
// non-finite values.  Every item's info gets the failing pivot (p for X, d_in + p for G)
// and its Gram is replaced by diag(k, k-1, ..., 1): distinct, well separated eigenvalues,
// so the eigensolver's fixed work runs on benign data.  Nothing is read by the host; the
// outputs of such a call are undefined.
__global__ void chol_guard_kernel(const int* __restrict__ chol_info, int xstep, int gstep, int d_in,
                                  double* __restrict__ G, int64_t ldg, int64_t sG, int k, int32_t* __restrict__ info) {
  // slice b's pivots: chol_info[2 b] for X, [2 b + 1] for G (slot 0 / 1 when shared)
  const int b = blockIdx.y;
  const int cx = chol_info[2 * b * xstep], cg = chol_info[2 * b * gstep + 1];
  if (cx == 0 && cg == 0) return;
  double* g = G + b * sG;
  const int64_t kk = int64_t(k) * k;
  for (int64_t e = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; e < kk; e += int64_t(gridDim.x) * blockDim.x) {
    const int64_t i = e / k, c = e % k;
    g[i * ldg + c] = i == c ? double(k - i) : 0.0;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) info[b] = cx != 0 ? cx : d_in + cg;
}

// out[i][c] = in[i][c] * g(sigma[c]);  g = sqrt (mode 0) or 1/sqrt (mode 1, 0 where sigma == 0)
__global__ void scale_cols_kernel(const float* __restrict__ in, int64_t ldi, float* __restrict__ out, int64_t ldo,
                                  int64_t rows, int cols, const float* __restrict__ sigma, int mode) {
  const int64_t i = blockIdx.y;
  for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < cols; c += gridDim.x * blockDim.x) {
    const float s = sigma[c];
    float g;
    if (mode == 0) g = sqrtf(fmaxf(s, 0.f));
    else g = s > 0.f ? 1.0f / sqrtf(s) : 0.f;
    out[i * ldo + c] = in[i * ldi + c] * g;
  }
}

lrc_status scale_cols(hipStream_t st, const float* in, int64_t ldi, float* out, int64_t ldo, int64_t rows,
                      int64_t cols, const float* sigma, int mode) {
  if (rows <= 0 || cols <= 0) return LRC_OK;
  const dim3 g(unsigned(std::min<int64_t>(cdiv(cols, 256), 16)), unsigned(rows));
  scale_cols_kernel<<<g, 256, 0, st>>>(in, ldi, out, ldo, rows, int(cols), sigma, mode);
  LRC_LAUNCHED();
  return LRC_OK;
}

struct DWs {
  float *lx, *lg, *wt1, *wt2, *qt, *u, *p;
  int* chol_info;
  double* gram;
  void* jac;
};

// nx, ng: Cholesky factors to hold for X and G (0: no such covariance, 1: shared by the
// batch, batch: one per slice)
DWs carve_decomp(Carve& cv, int64_t d_out, int64_t d_in, int64_t batch, int64_t rank, int64_t nx, int64_t ng) {
  const int64_t k = std::min(d_out, d_in);
  const int64_t kp = jacobi_padded(k);
  const int64_t big = std::max(d_out, d_in);
  const bool hx = nx > 0, hg = ng > 0;
  DWs w;
  w.lx = hx ? cv.take<float>(size_t(nx * d_in * d_in)) : nullptr;
  w.lg = hg ? cv.take<float>(size_t(ng * d_out * d_out)) : nullptr;
  w.chol_info = cv.take<int>(size_t(2 * batch));
  w.wt1 = (hx || hg) ? cv.take<float>(size_t(batch * d_out * d_in)) : nullptr;
  w.wt2 = (hx && hg) ? cv.take<float>(size_t(batch * d_out * d_in)) : nullptr;
  w.gram = cv.take<double>(size_t(batch * kp * kp));
  w.qt = cv.take<float>(size_t(batch * std::max<int64_t>(rank, 1) * k));
  w.u = cv.take<float>(size_t(k * std::max<int64_t>(rank, 1)));
  w.p = cv.take<float>(size_t(big * std::max<int64_t>(rank, 1)));
  // one eigensolver runs per call
  w.jac = cv.take<char>(use_tridiag(k, batch) ? tridiag_workspace(k, std::max<int64_t>(rank, 1), batch)
                                              : jacobi_workspace(k, batch));
  return w;
}

}  // namespace
}  // namespace lrc

using namespace lrc;

namespace lrc {
namespace {

size_t decompose_workspace(int64_t d_out, int64_t d_in, int64_t batch, int64_t rank, int64_t nx, int64_t ng) {
  if (d_out <= 0 || d_in <= 0 || batch <= 0 || rank < 0) return 0;
  Carve cv(nullptr);
  carve_decomp(cv, d_out, d_in, batch, rank, nx, ng);
  return cv.bytes();
}

// slices of a covariance: 0 (absent), 1 (shared by the batch) or batch (one per slice)
int64_t cov_slices(const void* sum, int64_t stride, int64_t batch) {
  return sum == nullptr ? 0 : (stride == 0 ? 1 : batch);
}

lrc_status decompose(const float* W, int64_t d_out, int64_t d_in, int64_t ldw, int64_t batch, int64_t stride_w,
                     const float* Xsum, int64_t ldx, int64_t stride_x, int64_t n_x, const float* Gsum, int64_t ldg,
                     int64_t stride_g, int64_t n_g, int64_t rank, float damping, float* sigma, float* left,
                     float* right, int32_t* info, void* ws, size_t ws_bytes, hipStream_t st) {
  if (W == nullptr || sigma == nullptr || info == nullptr) return LRC_EINVAL;
  if (d_out <= 0 || d_in <= 0 || batch <= 0 || ldw < d_in) return LRC_EINVAL;
  if (d_out > (int64_t(1) << 20) || d_in > (int64_t(1) << 20) || batch > (int64_t(1) << 16)) return LRC_EINVAL;
  if (batch > 1 && stride_w < d_out * ldw) return LRC_EINVAL;
  const int64_t k = std::min(d_out, d_in);
  if (rank < 0 || rank > k) return LRC_EINVAL;
  if (rank > 0 && (left == nullptr || right == nullptr)) return LRC_EINVAL;
  if (Xsum != nullptr && (ldx < d_in || n_x <= 0)) return LRC_EINVAL;
  if (Gsum != nullptr && (ldg < d_out || n_g <= 0)) return LRC_EINVAL;
  // a covariance per slice lies at a stride that keeps the slices apart
  if (stride_x < 0 || (Xsum != nullptr && stride_x != 0 && stride_x < d_in * ldx)) return LRC_EINVAL;
  if (stride_g < 0 || (Gsum != nullptr && stride_g != 0 && stride_g < d_out * ldg)) return LRC_EINVAL;
  if (!(damping >= 0.f) || !(damping < 3.0e38f)) return LRC_EINVAL;
  const int64_t nx = cov_slices(Xsum, stride_x, batch), ng = cov_slices(Gsum, stride_g, batch);
  const bool hx = nx > 0, hg = ng > 0;
  const size_t need = decompose_workspace(d_out, d_in, batch, rank, nx, ng);
  if (ws == nullptr || ws_bytes < need) return LRC_EWORKSPACE;
  Carve cv(ws);
  DWs w = carve_decomp(cv, d_out, d_in, batch, rank, nx, ng);
  const int64_t kp = jacobi_padded(k);
  const int64_t mn = d_out * d_in;
  const int64_t sLx = nx > 1 ? d_in * d_in : 0, sLg = ng > 1 ? d_out * d_out : 0;
  fill_i32_kernel<<<unsigned(cdiv(batch, 256)), 256, 0, st>>>(info, batch, 0);
  LRC_LAUNCHED();
  fill_i32_kernel<<<unsigned(cdiv(2 * batch, 256)), 256, 0, st>>>(w.chol_info, 2 * batch, 0);
  LRC_LAUNCHED();
  // a2: Cholesky factors of the covariances (a failed pivot is recorded in chol_info and
  // acted on after the Gram, on the device)
  // (one covariance per slice: every launch of the factorisation covers the batch)
  if (hx) LRC_TRY(cholesky_f32_batched(st, Xsum, ldx, stride_x, d_in, n_x, damping, w.lx, w.chol_info, 2, nx));
  if (hg) LRC_TRY(cholesky_f32_batched(st, Gsum, ldg, stride_g, d_out, n_g, damping, w.lg, w.chol_info + 1, 2, ng));
  // a3: whitening  W~ = L_g^T W L_x
  const float* cur = W;
  int64_t ldc = ldw, scur = stride_w;
  if (hx) {
    LRC_TRY(gemm_f32(st, GEMM_K_FROM_COL, d_out, d_in, d_in, 1.f, cur, ldc, scur, w.lx, d_in, sLx, 0.f, w.wt1, d_in,
                     mn, batch));
    cur = w.wt1;
    ldc = d_in;
    scur = mn;
  }
  if (hg) {
    float* dst = hx ? w.wt2 : w.wt1;
    LRC_TRY(gemm_f32(st, GEMM_TA | GEMM_K_FROM_ROW, d_out, d_in, d_out, 1.f, w.lg, d_out, sLg, cur, ldc, scur, 0.f,
                     dst, d_in, mn, batch));
    cur = dst;
    ldc = d_in;
    scur = mn;
  }
  // a4: fp64 Gram of the smaller side and its eigendecomposition
  const bool left_side = d_out <= d_in;
  LRC_TRY(gram_f64(st, left_side, d_out, d_in, cur, ldc, scur, w.gram, kp, kp * kp, batch));
  if (hx || hg) {
    const dim3 g(unsigned(std::min<int64_t>(cdiv(k * k, 256), 64)), unsigned(batch));
    chol_guard_kernel<<<g, 256, 0, st>>>(w.chol_info, nx > 1 ? 1 : 0, ng > 1 ? 1 : 0, int(d_in), w.gram, kp, kp * kp,
                                         int(k), info);
    LRC_LAUNCHED();
  }
  const int64_t ncols = std::max<int64_t>(rank, 1);
  if (use_tridiag(k, batch))
    LRC_TRY(tridiag_eig(st, w.gram, kp * kp, k, kp, ncols, batch, sigma, k, w.qt, ncols * k, w.jac));
  else
    LRC_TRY(jacobi_eig(st, w.gram, k, batch, ncols, sigma, w.qt, info, w.jac));
  if (rank == 0) return LRC_OK;
  // a5: back-map to weight space
  for (int64_t b = 0; b < batch; ++b) {
    const float* wb = W + b * stride_w;
    const float* sb = sigma + b * k;
    const float* qb = w.qt + b * rank * k;
    float* lb = left + b * d_out * rank;
    float* rb = right + b * rank * d_in;
    const float* lgb = hg ? w.lg + b * sLg : nullptr;
    const float* lxb = hx ? w.lx + b * sLx : nullptr;
    LRC_TRY(transpose_f32(st, qb, k, w.u, rank, rank, k));  // u: k x r (singular vectors as columns)
    if (left_side) {
      // Left = L_g^-T U S^1/2
      LRC_TRY(scale_cols(st, w.u, rank, lb, rank, k, rank, sb, 0));
      if (hg) LRC_TRY(trsm_lower_t(st, lgb, d_out, lb, rank, rank));
      // Right = (L_g U S^-1/2)^T W
      const float* pu = w.u;
      if (hg) {
        LRC_TRY(gemm_f32(st, GEMM_K_TO_ROW, d_out, rank, d_out, 1.f, lgb, d_out, 0, w.u, rank, 0, 0.f, w.p, rank, 0, 1));
        pu = w.p;
      }
      LRC_TRY(scale_cols(st, pu, rank, w.p, rank, d_out, rank, sb, 1));
      LRC_TRY(gemm_f32(st, GEMM_TA, rank, d_in, d_out, 1.f, w.p, rank, 0, wb, ldw, 0, 0.f, rb, d_in, 0, 1));
    } else {
      // Right = (L_x^-T V S^1/2)^T
      LRC_TRY(scale_cols(st, w.u, rank, w.p, rank, k, rank, sb, 0));
      if (hx) LRC_TRY(trsm_lower_t(st, lxb, d_in, w.p, rank, rank));
      LRC_TRY(transpose_f32(st, w.p, rank, rb, d_in, d_in, rank));
      // Left = W (L_x V S^-1/2)
      const float* pv = w.u;
      if (hx) {
        LRC_TRY(gemm_f32(st, GEMM_K_TO_ROW, d_in, rank, d_in, 1.f, lxb, d_in, 0, w.u, rank, 0, 0.f, w.p, rank, 0, 1));
        pv = w.p;
      }
      LRC_TRY(scale_cols(st, pv, rank, w.p, rank, d_in, rank, sb, 1));
      LRC_TRY(gemm_f32(st, 0, d_out, rank, d_in, 1.f, wb, ldw, 0, w.p, rank, 0, 0.f, lb, rank, 0, 1));
    }
  }
  return LRC_OK;
}

}  // namespace
}  // namespace lrc

extern "C" size_t lrc_whiten_decompose_workspace(int64_t d_out, int64_t d_in, int64_t batch, int64_t rank, int has_x,
                                                 int has_g) {
  return decompose_workspace(d_out, d_in, batch, rank, has_x != 0 ? 1 : 0, has_g != 0 ? 1 : 0);
}

extern "C" size_t lrc_whiten_decompose_strided_workspace(int64_t d_out, int64_t d_in, int64_t batch, int64_t rank,
                                                         int64_t x_slices, int64_t g_slices) {
  if (x_slices < 0 || g_slices < 0 || (x_slices > 1 && x_slices != batch) || (g_slices > 1 && g_slices != batch))
    return 0;
  return decompose_workspace(d_out, d_in, batch, rank, x_slices, g_slices);
}

extern "C" lrc_status lrc_whiten_decompose(const float* W, int64_t d_out, int64_t d_in, int64_t ldw, int64_t batch,
                                           int64_t stride_w, const float* Xsum, int64_t ldx, int64_t n_x,
                                           const float* Gsum, int64_t ldg, int64_t n_g, int64_t rank, float damping,
                                           float* sigma, float* left, float* right, int32_t* info, void* ws,
                                           size_t ws_bytes, void* stream) {
  return decompose(W, d_out, d_in, ldw, batch, stride_w, Xsum, ldx, 0, n_x, Gsum, ldg, 0, n_g, rank, damping, sigma,
                   left, right, info, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

extern "C" lrc_status lrc_whiten_decompose_strided(const float* W, int64_t d_out, int64_t d_in, int64_t ldw,
                                                   int64_t batch, int64_t stride_w, const float* Xsum, int64_t ldx,
                                                   int64_t stride_x, int64_t n_x, const float* Gsum, int64_t ldg,
                                                   int64_t stride_g, int64_t n_g, int64_t rank, float damping,
                                                   float* sigma, float* left, float* right, int32_t* info, void* ws,
                                                   size_t ws_bytes, void* stream) {
  return decompose(W, d_out, d_in, ldw, batch, stride_w, Xsum, ldx, stride_x, n_x, Gsum, ldg, stride_g, n_g, rank,
                   damping, sigma, left, right, info, ws, ws_bytes, static_cast<hipStream_t>(stream));
}
