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

// Eigensolver choice: a single Gram of size >= 512 goes through tridiagonalisation +
// inverse iteration (O(k^3) once); batches of small Grams through block Jacobi, whose
// rounds process every item of the batch at once.  LRC_EIGENSOLVER=jacobi|tridiag
// overrides the choice (tridiag only applies to batch 1).
bool use_tridiag(int64_t k, int64_t batch) {
  if (batch != 1) return false;
  const char* e = getenv("LRC_EIGENSOLVER");
  if (e && strcmp(e, "jacobi") == 0) return false;
  if (e && strcmp(e, "tridiag") == 0) return true;
  return k >= 512;
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
  if (i < n) p[i] = v;
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

DWs carve_decomp(Carve& cv, int64_t d_out, int64_t d_in, int64_t batch, int64_t rank, bool hx, bool hg) {
  const int64_t k = std::min(d_out, d_in);
  const int64_t kp = jacobi_padded(k);
  const int64_t big = std::max(d_out, d_in);
  DWs w;
  w.lx = hx ? cv.take<float>(size_t(d_in * d_in)) : nullptr;
  w.lg = hg ? cv.take<float>(size_t(d_out * d_out)) : nullptr;
  w.chol_info = cv.take<int>(2);
  w.wt1 = (hx || hg) ? cv.take<float>(size_t(batch * d_out * d_in)) : nullptr;
  w.wt2 = (hx && hg) ? cv.take<float>(size_t(batch * d_out * d_in)) : nullptr;
  w.gram = cv.take<double>(size_t(batch * kp * kp));
  w.qt = cv.take<float>(size_t(batch * std::max<int64_t>(rank, 1) * k));
  w.u = cv.take<float>(size_t(k * std::max<int64_t>(rank, 1)));
  w.p = cv.take<float>(size_t(big * std::max<int64_t>(rank, 1)));
  // the two eigensolvers run one after the other at most (a clustered spectrum falls back
  // from the tridiagonal route to Jacobi), so they share one region
  size_t jb = jacobi_workspace(k, batch);
  if (use_tridiag(k, batch)) jb = std::max(jb, tridiag_workspace(k, std::max<int64_t>(rank, 1)));
  w.jac = cv.take<char>(jb);
  return w;
}

}  // namespace
}  // namespace lrc

using namespace lrc;

extern "C" size_t lrc_whiten_decompose_workspace(int64_t d_out, int64_t d_in, int64_t batch, int64_t rank, int has_x,
                                                 int has_g) {
  if (d_out <= 0 || d_in <= 0 || batch <= 0 || rank < 0) return 0;
  Carve cv(nullptr);
  carve_decomp(cv, d_out, d_in, batch, rank, has_x != 0, has_g != 0);
  return cv.bytes();
}

extern "C" lrc_status lrc_whiten_decompose(const float* W, int64_t d_out, int64_t d_in, int64_t ldw, int64_t batch,
                                           int64_t stride_w, const float* Xsum, int64_t ldx, int64_t n_x,
                                           const float* Gsum, int64_t ldg, int64_t n_g, int64_t rank, float damping,
                                           float* sigma, float* left, float* right, int32_t* info, void* ws,
                                           size_t ws_bytes, void* stream) {
  if (W == nullptr || sigma == nullptr || info == nullptr) return LRC_EINVAL;
  if (d_out <= 0 || d_in <= 0 || batch <= 0 || ldw < d_in) return LRC_EINVAL;
  if (d_out > (int64_t(1) << 20) || d_in > (int64_t(1) << 20) || batch > (int64_t(1) << 16)) return LRC_EINVAL;
  if (batch > 1 && stride_w < d_out * ldw) return LRC_EINVAL;
  const int64_t k = std::min(d_out, d_in);
  if (rank < 0 || rank > k) return LRC_EINVAL;
  if (rank > 0 && (left == nullptr || right == nullptr)) return LRC_EINVAL;
  if (Xsum != nullptr && (ldx < d_in || n_x <= 0)) return LRC_EINVAL;
  if (Gsum != nullptr && (ldg < d_out || n_g <= 0)) return LRC_EINVAL;
  if (!(damping >= 0.f) || !(damping < 3.0e38f)) return LRC_EINVAL;
  const bool hx = Xsum != nullptr, hg = Gsum != nullptr;
  const size_t need = lrc_whiten_decompose_workspace(d_out, d_in, batch, rank, hx, hg);
  if (ws == nullptr || ws_bytes < need) return LRC_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Carve cv(ws);
  DWs w = carve_decomp(cv, d_out, d_in, batch, rank, hx, hg);
  const int64_t kp = jacobi_padded(k);
  const int64_t mn = d_out * d_in;

  fill_i32_kernel<<<unsigned(cdiv(batch, 256)), 256, 0, st>>>(info, batch, 0);
  LRC_LAUNCHED();
  fill_i32_kernel<<<1, 64, 0, st>>>(w.chol_info, 2, 0);
  LRC_LAUNCHED();

  // a2: Cholesky factors of the covariances
  if (hx) LRC_TRY(cholesky_f32(st, Xsum, ldx, d_in, n_x, damping, w.lx, w.chol_info));
  if (hg) LRC_TRY(cholesky_f32(st, Gsum, ldg, d_out, n_g, damping, w.lg, w.chol_info + 1));
  if (hx || hg) {
    int ci[2] = {0, 0};
    LRC_HIP(hipMemcpyAsync(ci, w.chol_info, sizeof(ci), hipMemcpyDeviceToHost, st));
    LRC_HIP(hipStreamSynchronize(st));
    if (ci[0] != 0 || ci[1] != 0) {
      const int32_t v = ci[0] != 0 ? ci[0] : int32_t(d_in + ci[1]);
      fill_i32_kernel<<<unsigned(cdiv(batch, 256)), 256, 0, st>>>(info, batch, v);
      LRC_LAUNCHED();
      return LRC_ENOTPD;
    }
  }

  // a3: whitening  W~ = L_g^T W L_x
  const float* cur = W;
  int64_t ldc = ldw, scur = stride_w;
  if (hx) {
    LRC_TRY(gemm_f32(st, GEMM_K_FROM_COL, d_out, d_in, d_in, 1.f, cur, ldc, scur, w.lx, d_in, 0, 0.f, w.wt1, d_in, mn,
                     batch));
    cur = w.wt1;
    ldc = d_in;
    scur = mn;
  }
  if (hg) {
    float* dst = hx ? w.wt2 : w.wt1;
    LRC_TRY(gemm_f32(st, GEMM_TA | GEMM_K_FROM_ROW, d_out, d_in, d_out, 1.f, w.lg, d_out, 0, cur, ldc, scur, 0.f, dst,
                     d_in, mn, batch));
    cur = dst;
    ldc = d_in;
    scur = mn;
  }

  // a4: fp64 Gram of the smaller side and its eigendecomposition
  const bool left_side = d_out <= d_in;
  LRC_TRY(gram_f64(st, left_side, d_out, d_in, cur, ldc, scur, w.gram, kp, kp * kp, batch));
  const int64_t ncols = std::max<int64_t>(rank, 1);
  bool jacobi = true;
  if (use_tridiag(k, batch)) {
    bool clustered = false;
    LRC_TRY(tridiag_eig(st, w.gram, k, kp, ncols, sigma, w.qt, w.jac, &clustered));
    jacobi = clustered;
    // the tridiagonalisation consumed the Gram: form it again for the Jacobi solver
    if (clustered) LRC_TRY(gram_f64(st, left_side, d_out, d_in, cur, ldc, scur, w.gram, kp, kp * kp, batch));
  }
  if (jacobi) {
    const lrc_status es = jacobi_eig(st, w.gram, k, batch, ncols, sigma, w.qt, info, w.jac);
    if (es != LRC_OK) return es;
  }
  if (rank == 0) return LRC_OK;

  // a5: back-map to weight space
  for (int64_t b = 0; b < batch; ++b) {
    const float* wb = W + b * stride_w;
    const float* sb = sigma + b * k;
    const float* qb = w.qt + b * rank * k;
    float* lb = left + b * d_out * rank;
    float* rb = right + b * rank * d_in;
    LRC_TRY(transpose_f32(st, qb, k, w.u, rank, rank, k));  // u: k x r (singular vectors as columns)
    if (left_side) {
      // Left = L_g^-T U S^1/2
      LRC_TRY(scale_cols(st, w.u, rank, lb, rank, k, rank, sb, 0));
      if (hg) LRC_TRY(trsm_lower_t(st, w.lg, d_out, lb, rank, rank));
      // Right = (L_g U S^-1/2)^T W
      const float* pu = w.u;
      if (hg) {
        LRC_TRY(gemm_f32(st, GEMM_K_TO_ROW, d_out, rank, d_out, 1.f, w.lg, d_out, 0, w.u, rank, 0, 0.f, w.p, rank, 0, 1));
        pu = w.p;
      }
      LRC_TRY(scale_cols(st, pu, rank, w.p, rank, d_out, rank, sb, 1));
      LRC_TRY(gemm_f32(st, GEMM_TA, rank, d_in, d_out, 1.f, w.p, rank, 0, wb, ldw, 0, 0.f, rb, d_in, 0, 1));
    } else {
      // Right = (L_x^-T V S^1/2)^T
      LRC_TRY(scale_cols(st, w.u, rank, w.p, rank, k, rank, sb, 0));
      if (hx) LRC_TRY(trsm_lower_t(st, w.lx, d_in, w.p, rank, rank));
      LRC_TRY(transpose_f32(st, w.p, rank, rb, d_in, d_in, rank));
      // Left = W (L_x V S^-1/2)
      const float* pv = w.u;
      if (hx) {
        LRC_TRY(gemm_f32(st, GEMM_K_TO_ROW, d_in, rank, d_in, 1.f, w.lx, d_in, 0, w.u, rank, 0, 0.f, w.p, rank, 0, 1));
        pv = w.p;
      }
      LRC_TRY(scale_cols(st, pv, rank, w.p, rank, d_in, rank, sb, 1));
      LRC_TRY(gemm_f32(st, 0, d_out, rank, d_in, 1.f, wb, ldw, 0, w.p, rank, 0, 0.f, lb, rank, 0, 1));
    }
  }
  return LRC_OK;
}
