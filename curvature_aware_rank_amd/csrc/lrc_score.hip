// Component scores (LASER technical summary, Methodology 2: empirical-Fisher importance
// score; K-FAC: the loss of dropping one component alone).
//
//   FISHER: s_i = 1/(2N) sum_t (b_t . left_i)^2 (a_t . right_i)^2
//
// A workgroup owns 64 tokens x 64 components: it forms both projections P = A Right^T and
// Q = B Left for its tile in registers (LDS-staged operands), squares and multiplies
// them, and sums its 64 tokens in a fixed order; a second pass adds the token-tile
// partial sums in order (fp64), so the result is bit-reproducible.
#include "lrc_internal.h"

namespace lrc {
namespace {

constexpr int ST = 64;  // tokens and components per tile
constexpr int SK = 16;  // reduction step

template <typename T>
__device__ __forceinline__ float ld_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld_f32<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_f32<uint16_t>(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }

template <typename T>
__global__ __launch_bounds__(256) void fisher_partial_kernel(const T* __restrict__ A, const T* __restrict__ B, int64_t n,
                                                             int d_in, int d_out, const float* __restrict__ left,
                                                             const float* __restrict__ right, int k,
                                                             float* __restrict__ partial) {
  __shared__ float xs[SK][ST + 1];
  __shared__ float fs[SK][ST + 1];
  __shared__ float red[16][ST + 1];
  const int c0 = blockIdx.x * ST;
  const int64_t t0 = int64_t(blockIdx.y) * ST;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float p[4][4] = {}, q[4][4] = {};
  // P = A Right^T over d_in
  for (int k0 = 0; k0 < d_in; k0 += SK) {
    for (int e = threadIdx.x; e < SK * ST; e += 256) {
      const int r = e / SK, kk = e % SK;
      const int64_t t = t0 + r;
      const int gk = k0 + kk, comp = c0 + r;
      xs[kk][r] = (t < n && gk < d_in) ? ld_f32(A, t * d_in + gk) : 0.f;
      fs[kk][r] = (comp < k && gk < d_in) ? right[int64_t(comp) * d_in + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < SK; ++kk) {
      float xv[4], fv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { xv[i] = xs[kk][ty * 4 + i]; fv[i] = fs[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) p[i][j] = fmaf(xv[i], fv[j], p[i][j]);
    }
    __syncthreads();
  }
  // Q = B Left over d_out
  for (int k0 = 0; k0 < d_out; k0 += SK) {
    for (int e = threadIdx.x; e < SK * ST; e += 256) {
      {
        const int r = e / SK, kk = e % SK;
        const int64_t t = t0 + r;
        const int gk = k0 + kk;
        xs[kk][r] = (t < n && gk < d_out) ? ld_f32(B, t * d_out + gk) : 0.f;
      }
      {
        const int kk = e / ST, c = e % ST;
        const int gk = k0 + kk, comp = c0 + c;
        fs[kk][c] = (comp < k && gk < d_out) ? left[int64_t(gk) * k + comp] : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < SK; ++kk) {
      float xv[4], fv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { xv[i] = xs[kk][ty * 4 + i]; fv[i] = fs[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) q[i][j] = fmaf(xv[i], fv[j], q[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pp = p[i][j] * p[i][j], qq = q[i][j] * q[i][j];
      s = fmaf(pp, qq, s);
    }
    red[ty][tx * 4 + j] = s;
  }
  __syncthreads();
  if (threadIdx.x < ST) {
    float s = 0.f;
    for (int r = 0; r < 16; ++r) s += red[r][threadIdx.x];
    const int comp = c0 + threadIdx.x;
    if (comp < k) partial[int64_t(blockIdx.y) * k + comp] = s;
  }
}

__global__ void fisher_final_kernel(const float* __restrict__ partial, int ntb, int k, int accumulate, int finalize,
                                    double inv2n, float* __restrict__ scores) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= k) return;
  double s = accumulate ? double(scores[i]) : 0.0;
  for (int b = 0; b < ntb; ++b) s += double(partial[int64_t(b) * k + i]);
  if (finalize) s *= inv2n;
  scores[i] = float(s);
}

__global__ void kfac_kernel(const float* __restrict__ sigma, int k, float* __restrict__ scores) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < k) scores[i] = 0.5f * sigma[i] * sigma[i];
}

}  // namespace
}  // namespace lrc

using namespace lrc;

extern "C" size_t lrc_score_components_workspace(int64_t n_tokens, int64_t d_in, int64_t d_out, int64_t k,
                                                 uint32_t flags) {
  (void)d_in;
  (void)d_out;
  if (n_tokens < 0 || k <= 0) return 0;
  if (!(flags & LRC_SCORE_FISHER)) return 0;
  Carve cv(nullptr);
  cv.take<float>(size_t(cdiv(n_tokens, ST) * k));
  return cv.bytes();
}

extern "C" lrc_status lrc_score_components(const void* A, const void* B, lrc_dtype dt, int64_t n_tokens, int64_t d_in,
                                           int64_t d_out, const float* left, const float* right, const float* sigma,
                                           int64_t k, uint32_t flags, int accumulate, int finalize, int64_t n_total,
                                           float* scores, void* ws, size_t ws_bytes, void* stream) {
  if (flags != LRC_SCORE_FISHER && flags != LRC_SCORE_KFAC) return LRC_EDTYPE;
  if (scores == nullptr || k <= 0 || k > (int64_t(1) << 30)) return LRC_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (flags == LRC_SCORE_KFAC) {
    if (sigma == nullptr) return LRC_EINVAL;
    kfac_kernel<<<unsigned(cdiv(k, 256)), 256, 0, st>>>(sigma, int(k), scores);
    LRC_LAUNCHED();
    return LRC_OK;
  }
  if (dt != LRC_F32 && dt != LRC_BF16) return LRC_EDTYPE;
  if (n_tokens < 0 || d_in <= 0 || d_out <= 0 || d_in > (int64_t(1) << 30) || d_out > (int64_t(1) << 30))
    return LRC_EINVAL;
  if (left == nullptr || right == nullptr) return LRC_EINVAL;
  if (n_tokens > 0 && (A == nullptr || B == nullptr)) return LRC_EINVAL;
  if (finalize && n_total <= 0) return LRC_EINVAL;
  if (n_tokens > (int64_t(65535) * ST)) return LRC_EINVAL;  // one chunk per call at most 4M tokens
  const size_t need = lrc_score_components_workspace(n_tokens, d_in, d_out, k, flags);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return LRC_EWORKSPACE;
  float* partial = static_cast<float*>(ws);
  const int ntb = int(cdiv(n_tokens, ST));
  if (ntb > 0) {
    const dim3 grid(unsigned(cdiv(k, ST)), unsigned(ntb));
    // algorithmic work: the two projections (2 N k (d_in + d_out)) and 3 flops per
    // (token, component) for the squares and the product; A and B read once, the factors
    // once, one fp32 partial per (64-token block, component) written
    const double esz = dt == LRC_BF16 ? 2.0 : 4.0;
    ProfScope scope("fisher_partial_kernel", st,
                    2.0 * double(n_tokens) * double(k) * double(d_in + d_out) + 3.0 * double(n_tokens) * double(k),
                    esz * double(n_tokens) * double(d_in + d_out) + 4.0 * double(k) * double(d_in + d_out) +
                        4.0 * double(ntb) * double(k));
    if (dt == LRC_BF16)
      fisher_partial_kernel<uint16_t><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(A),
                                                            static_cast<const uint16_t*>(B), n_tokens, int(d_in),
                                                            int(d_out), left, right, int(k), partial);
    else
      fisher_partial_kernel<float><<<grid, 256, 0, st>>>(static_cast<const float*>(A), static_cast<const float*>(B),
                                                         n_tokens, int(d_in), int(d_out), left, right, int(k), partial);
    LRC_LAUNCHED();
  }
  const double inv2n = finalize ? 1.0 / (2.0 * double(n_total)) : 1.0;
  fisher_final_kernel<<<unsigned(cdiv(k, 256)), 256, 0, st>>>(partial, ntb, int(k), accumulate, finalize, inv2n,
                                                               scores);
  LRC_LAUNCHED();
  return LRC_OK;
}
