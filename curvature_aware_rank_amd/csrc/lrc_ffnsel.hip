// FFN hybrid channel selection: which hidden channels of an FFN take the low-rank branch.
//
// LASER technical summary, 3 (Hybrid SVD-Quantization for FFNs), items Channel selection
// and Hybrid architecture: a temporary SVD of the gate and up projections identifies the
// hidden channels that the low-rank form reconstructs well ("SVD-friendly"); those are
// compressed, the others stay dense.  Readings: the temporary SVD is the whitened
// decomposition the caller already ran (same covariance X, G = I, rank r); a channel's
// reconstruction error is the expected squared error of its two pre-activations under the
// calibration distribution,
//   err[h] = sum over P in {gate, up} of dW_P[h] X dW_P[h]^T,  dW_P = W_P - Left_P Right_P,
// computed as the squared row norm of dW_P L_x (X = L_x L_x^T); the n_lowrank channels with
// the smallest error (ties by index) are selected.
//
// Steps on the device: Cholesky of X (the shared blocked kernel), D = W - Left Right and
// E = D L_x on the fp32 GEMM (triangular operand), squared row norms of E accumulated in
// fp64 in a fixed order, then every channel's rank among the (err, index) pairs by
// counting, which gives the order and the selection without a sort.
#include "lrc_internal.h"
#include "lrc_dense.h"

namespace lrc {
namespace {

constexpr int ST = 256;          // threads per workgroup
constexpr int KCH = 2048;        // keys per LDS chunk of the rank count

__global__ void fsel_fill_i32_kernel(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// err[h] (+)= sum_c E[h][c]^2 in fp64: one workgroup per row, lanes take columns
// c = tid + ST u in order, then a fixed butterfly over the wave and the four waves
__global__ __launch_bounds__(ST) void fsel_row_sq_kernel(const float* __restrict__ E, int64_t lde, int cols,
                                                         int accumulate, double* __restrict__ err) {
  __shared__ double red[ST / 64];
  const int64_t h = blockIdx.x;
  const int tid = threadIdx.x;
  const float* row = E + h * lde;
  double s = 0.0;
  for (int c = tid; c < cols; c += ST) {
    const double v = double(row[c]);
    s = fma(v, v, s);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) {
    const double t = (red[0] + red[1]) + (red[2] + red[3]);
    err[h] = accumulate ? err[h] + t : t;
  }
}

// rank of channel h among the (err, index) pairs in ascending order: the number of
// channels g with err[g] < err[h], or err[g] == err[h] and g < h.  The keys are the
// errors' bit patterns as unsigned integers (for the non-negative values here, and +inf,
// the same order as the values; a NaN sorts after them), so the order is total and every
// rank is distinct.  order[rank] = h; lowrank[h] = rank < n_lowrank.  After a failed
// Cholesky of X (chol_info != 0) the errors are meaningless: info gets the pivot and
// nothing is written.
__global__ __launch_bounds__(ST) void fsel_rank_kernel(const double* __restrict__ err, int n, int n_lowrank,
                                                       const int* __restrict__ chol_info, int32_t* __restrict__ info,
                                                       int32_t* __restrict__ order, uint8_t* __restrict__ lowrank) {
  __shared__ uint64_t keys[KCH];
  const int ci = *chol_info;
  if (ci != 0) {
    if (blockIdx.x == 0 && threadIdx.x == 0) *info = ci;
    return;
  }
  const int h = blockIdx.x * ST + threadIdx.x;
  const uint64_t mine = h < n ? uint64_t(__double_as_longlong(err[h])) : 0;
  int rank = 0;
  for (int g0 = 0; g0 < n; g0 += KCH) {
    const int cnt = min(KCH, n - g0);
    __syncthreads();
    for (int t = threadIdx.x; t < cnt; t += ST) keys[t] = uint64_t(__double_as_longlong(err[g0 + t]));
    __syncthreads();
    if (h < n) {
      for (int t = 0; t < cnt; ++t) {
        const uint64_t k = keys[t];
        const int g = g0 + t;
        rank += (k < mine || (k == mine && g < h)) ? 1 : 0;
      }
    }
  }
  if (h < n) {
    order[rank] = h;
    lowrank[h] = rank < n_lowrank ? 1 : 0;
  }
}

struct FselWs {
  float* lx;
  float* D;
  float* E;
  int* info;
};

FselWs carve_fsel(Carve& cv, int64_t d_ff, int64_t d) {
  FselWs w;
  w.lx = cv.take<float>(size_t(d * d));
  w.D = cv.take<float>(size_t(d_ff * d));
  w.E = cv.take<float>(size_t(d_ff * d));
  w.info = cv.take<int>(1);
  return w;
}

}  // namespace
}  // namespace lrc

using namespace lrc;

extern "C" size_t lrc_ffn_select_channels_workspace(int64_t d_ff, int64_t d) {
  if (d_ff <= 0 || d <= 0) return 0;
  Carve cv(nullptr);
  carve_fsel(cv, d_ff, d);
  return cv.bytes();
}

extern "C" lrc_status lrc_ffn_select_channels(const float* w_gate, const float* w_up, int64_t d_ff, int64_t d,
                                              int64_t ldw, const float* left_gate, const float* right_gate,
                                              const float* left_up, const float* right_up, int64_t r,
                                              const float* Xsum, int64_t ldx, int64_t n_x, float damping,
                                              int64_t n_lowrank, double* err, int32_t* order, uint8_t* lowrank,
                                              int32_t* info, void* ws, size_t ws_bytes, void* stream) {
  if (w_gate == nullptr || w_up == nullptr || Xsum == nullptr || err == nullptr || order == nullptr ||
      lowrank == nullptr || info == nullptr)
    return LRC_EINVAL;
  if (d_ff <= 0 || d <= 0 || ldw < d || ldx < d || n_x <= 0 || r < 0 || r > std::min(d_ff, d) || n_lowrank < 0 ||
      n_lowrank > d_ff || !(damping >= 0.f) || d_ff > (int64_t(1) << 31) - 1 || d > (int64_t(1) << 31) - 1)
    return LRC_EINVAL;
  if (r > 0 && (left_gate == nullptr || right_gate == nullptr || left_up == nullptr || right_up == nullptr))
    return LRC_EINVAL;
  const size_t need = lrc_ffn_select_channels_workspace(d_ff, d);
  if (ws == nullptr || ws_bytes < need) return LRC_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Carve cv(ws);
  FselWs w = carve_fsel(cv, d_ff, d);

  fsel_fill_i32_kernel<<<1, 64, 0, st>>>(w.info, 1, 0);
  LRC_LAUNCHED();
  fsel_fill_i32_kernel<<<1, 64, 0, st>>>(info, 1, 0);
  LRC_LAUNCHED();
  // a failed pivot is acted on by the rank kernel, on the device
  LRC_TRY(cholesky_f32(st, Xsum, ldx, d, n_x, damping, w.lx, w.info));
  const float* Ws[2] = {w_gate, w_up};
  const float* Ls[2] = {left_gate, left_up};
  const float* Rs[2] = {right_gate, right_up};
  for (int p = 0; p < 2; ++p) {
    // D = W - Left Right
    LRC_HIP(hipMemcpy2DAsync(w.D, size_t(d) * sizeof(float), Ws[p], size_t(ldw) * sizeof(float),
                             size_t(d) * sizeof(float), size_t(d_ff), hipMemcpyDeviceToDevice, st));
    if (r > 0)
      LRC_TRY(gemm_f32(st, 0, d_ff, d, r, -1.f, Ls[p], r, 0, Rs[p], d, 0, 1.f, w.D, d, 0, 1));
    // E = D L_x (L_x lower triangular: k runs from the tile's first column)
    LRC_TRY(gemm_f32(st, GEMM_K_FROM_COL, d_ff, d, d, 1.f, w.D, d, 0, w.lx, d, 0, 0.f, w.E, d, 0, 1));
    ProfScope scope("fsel_row_sq_kernel", st, 2.0 * double(d_ff) * double(d), 4.0 * double(d_ff) * double(d));
    fsel_row_sq_kernel<<<unsigned(d_ff), ST, 0, st>>>(w.E, d, int(d), p, err);
    LRC_LAUNCHED();
  }
  fsel_rank_kernel<<<unsigned(cdiv(d_ff, ST)), ST, 0, st>>>(err, int(d_ff), int(n_lowrank), w.info, info, order,
                                                           lowrank);
  LRC_LAUNCHED();
  return LRC_OK;
}
