// Factor codec: an orthogonal rotation between the low-rank factors, then round-to-nearest
// int8 of both branches.
//
// LASER technical summary, 3 (Hybrid SVD-Quantization for FFNs), item Quantization: an
// orthogonal rotation is inserted between the SVD factors to smooth outliers, and both the
// low-rank and the dense branch are quantised round-to-nearest.  Readings: the rotation is
// R = H_r diag(signs) / sqrt(r) (Sylvester Hadamard, r a power of two, caller's +-1 signs),
// left' = left R, right' = R^T right (so left' right' = left right); the quantiser is
// symmetric int8 per row (one output channel): scale = fl32(max|row| / 127),
// q = clamp(round_half_even(fl32(x / scale)), -127, 127), an all-zero row gives zeros.
//
// A row of left (or a column of right, via a transpose) is rotated by one workgroup with a
// fast Walsh-Hadamard transform in fp64 in LDS; the result is rounded once to fp32.
#include "lrc_internal.h"
#include "lrc_dense.h"

namespace lrc {
namespace {

constexpr int CT = 256;          // threads per workgroup
constexpr int ROT_MAX = 8192;    // largest rank the LDS row holds

// block-wide max of non-negative floats (exact in any order)
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

// quantise this thread's values v[] (columns c = tid + CT u) of one row with the row scale
__device__ __forceinline__ float row_scale(float amax) { return __fdiv_rn(amax, 127.0f); }
__device__ __forceinline__ int8_t quant(float x, float s) {
  return s > 0.f ? int8_t(fminf(fmaxf(rintf(__fdiv_rn(x, s)), -127.f), 127.f)) : int8_t(0);
}

// Y = X H diag(signs) / sqrt(r) row by row (X rows x r, leading dim ldx); writes Y (fp32,
// leading dim r) if Y != nullptr and, if q != nullptr, the row's int8 codes and scale.
// (X and Y may be the same buffer: a row is read whole into LDS before it is written)
__global__ __launch_bounds__(CT) void rot_rows_kernel(const float* X, int64_t ldx, int r,
                                                      const float* __restrict__ signs, float* Y,
                                                      int8_t* __restrict__ q, float* __restrict__ scale) {
  extern __shared__ double buf[];   // r doubles (dynamic size)
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const float* x = X + row * ldx;
  for (int k = tid; k < r; k += CT) buf[k] = double(x[k]);
  // in-place Walsh-Hadamard transform (natural order): butterflies of stride h
  for (int h = 1; h < r; h <<= 1) {
    __syncthreads();
    for (int bi = tid; bi < r / 2; bi += CT) {
      const int i = (bi / h) * 2 * h + (bi % h), j = i + h;
      const double a = buf[i], c = buf[j];
      buf[i] = a + c;
      buf[j] = a - c;
    }
  }
  __syncthreads();
  const double inv = 1.0 / sqrt(double(r));
  float amax = 0.f;
  for (int k = tid; k < r; k += CT) {
    const float y = float(buf[k] * double(signs[k]) * inv);
    buf[k] = double(y);
    amax = fmaxf(amax, fabsf(y));
    if (Y != nullptr) Y[row * r + k] = y;
  }
  if (q == nullptr) return;
  const float s = row_scale(block_max(amax, red));
  for (int k = tid; k < r; k += CT) q[row * r + k] = quant(float(buf[k]), s);
  if (tid == 0) scale[row] = s;
}

// int8 codes and scale of every row of X (rows x cols, leading dim ldx)
__global__ __launch_bounds__(CT) void quant_rows_kernel(const float* __restrict__ X, int64_t ldx, int64_t cols,
                                                        int8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const float* x = X + row * ldx;
  float amax = 0.f;
  for (int64_t k = threadIdx.x; k < cols; k += CT) amax = fmaxf(amax, fabsf(x[k]));
  const float s = row_scale(block_max(amax, red));
  for (int64_t k = threadIdx.x; k < cols; k += CT) q[row * cols + k] = quant(x[k], s);
  if (threadIdx.x == 0) scale[row] = s;
}

bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

}  // namespace
}  // namespace lrc

using namespace lrc;

extern "C" size_t lrc_rotate_quantize_workspace(int64_t d_out, int64_t r, int64_t d_in) {
  (void)d_out;
  if (r <= 0 || d_in <= 0) return 0;
  Carve cv(nullptr);
  cv.take<float>(size_t(d_in * r));
  cv.take<float>(size_t(r * d_in));
  return cv.bytes();
}

extern "C" lrc_status lrc_rotate_quantize(const float* left, const float* right, int64_t d_out, int64_t r,
                                          int64_t d_in, const float* signs, int8_t* q_left, float* s_left,
                                          int8_t* q_right, float* s_right, float* left_rot, float* right_rot,
                                          void* ws, size_t ws_bytes, void* stream) {
  if (left == nullptr || right == nullptr || signs == nullptr || q_left == nullptr || s_left == nullptr ||
      q_right == nullptr || s_right == nullptr)
    return LRC_EINVAL;
  if (d_out <= 0 || d_in <= 0 || !pow2(r) || r > ROT_MAX || d_out > (int64_t(1) << 31) - 1 ||
      d_in > (int64_t(1) << 31) - 1)
    return LRC_EINVAL;
  const size_t need = lrc_rotate_quantize_workspace(d_out, r, d_in);
  if (ws == nullptr || ws_bytes < need) return LRC_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Carve cv(ws);
  float* rt = cv.take<float>(size_t(d_in * r));        // right^T, rotated in place
  float* rr = right_rot != nullptr ? right_rot : cv.take<float>(size_t(r * d_in));
  ProfScope scope("rot_rows_kernel", st, 0.0, 4.0 * double(d_out + d_in) * double(r) * 2.0);
  const size_t lds = size_t(r) * sizeof(double);
  if (lds > 48 * 1024)
    LRC_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&rot_rows_kernel),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)));
  rot_rows_kernel<<<unsigned(d_out), CT, lds, st>>>(left, r, int(r), signs, left_rot, q_left, s_left);
  LRC_LAUNCHED();
  LRC_TRY(transpose_f32(st, right, d_in, rt, r, r, d_in));
  rot_rows_kernel<<<unsigned(d_in), CT, lds, st>>>(rt, r, int(r), signs, rt, nullptr, nullptr);
  LRC_LAUNCHED();
  LRC_TRY(transpose_f32(st, rt, r, rr, d_in, d_in, r));
  quant_rows_kernel<<<unsigned(r), CT, 0, st>>>(rr, d_in, d_in, q_right, s_right);
  LRC_LAUNCHED();
  return LRC_OK;
}

extern "C" lrc_status lrc_quantize_rows(const float* X, int64_t rows, int64_t cols, int64_t ldx, int8_t* q,
                                        float* scale, void* stream) {
  if (X == nullptr || q == nullptr || scale == nullptr || rows <= 0 || cols <= 0 || ldx < cols ||
      rows > (int64_t(1) << 31) - 1)
    return LRC_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  quant_rows_kernel<<<unsigned(rows), CT, 0, st>>>(X, ldx, cols, q, scale);
  LRC_LAUNCHED();
  return LRC_OK;
}
