// Internal helpers shared by the liblrc translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "lrc.h"

namespace lrc {

// ---------------------------------------------------------------------------------
// error plumbing
// ---------------------------------------------------------------------------------
void set_last_hip_error(hipError_t e);

#define LRC_HIP(expr)                                   \
  do {                                                  \
    hipError_t lrc_e_ = (expr);                         \
    if (lrc_e_ != hipSuccess) {                         \
      ::lrc::set_last_hip_error(lrc_e_);                \
      return LRC_EHIP;                                  \
    }                                                   \
  } while (0)

#define LRC_LAUNCHED() LRC_HIP(hipGetLastError())

#define LRC_TRY(expr)                                   \
  do {                                                  \
    lrc_status lrc_s_ = (expr);                         \
    if (lrc_s_ != LRC_OK) return lrc_s_;                \
  } while (0)

// ---------------------------------------------------------------------------------
// workspace carving: the same code computes sizes (base == nullptr) and pointers
// ---------------------------------------------------------------------------------
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t n) {
    size_t a = (off + 255) & ~size_t(255);
    off = a + n * sizeof(T);
    return base ? reinterpret_cast<T*>(base + a) : nullptr;
  }
  size_t bytes() const { return (off + 255) & ~size_t(255); }
};

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int device_cu_count();  // compute units of the current device (cached per device)

// measurement support (see lrc_profile_start): a scope around one kernel launch
bool prof_enabled();
void prof_add_work(const char* name, double flops, double bytes);
struct ProfScope {
  const char* name;
  hipStream_t st;
  double flops, bytes;
  hipEvent_t e0 = nullptr;
  ProfScope(const char* n, hipStream_t s, double f, double b);
  ~ProfScope();
};

// One kernel launched through hipExtLaunchKernelGGL with start/stop: the two events then
// carry the kernel's own begin and end (no marker packets of their own in the stream, so
// a short kernel reads as long as in a kernel trace).  Both are null when the session is
// off, which makes the launch an ordinary one.
struct ProfKernel {
  const char* name;
  double flops, bytes;
  hipEvent_t start = nullptr, stop = nullptr;
  ProfKernel(const char* n, double f, double b);
  ~ProfKernel();
};

// ---------------------------------------------------------------------------------
// device-side types and conversions
// ---------------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// ---------------------------------------------------------------------------------
// internal launchers (defined in the .hip files)
// ---------------------------------------------------------------------------------
// fp32 GEMM: C = alpha * op(A) * op(B) + beta * C  (row-major, batched by strides)
enum GemmFlags : unsigned {
  GEMM_TA = 1u,          // op(A) = A^T   (A stored k x m)
  GEMM_TB = 2u,          // op(B) = B^T   (B stored n x k)
  GEMM_LOWER = 4u,       // only tiles/elements with row >= col are produced
  GEMM_K_FROM_COL = 8u,  // op(B) is lower triangular: k starts at the tile's first column
  GEMM_K_FROM_ROW = 16u, // op(A) is upper triangular: k starts at the tile's first row
  GEMM_K_TO_ROW = 32u,   // op(A) is lower triangular: k ends after the tile's last row
  GEMM_MIRROR = 64u,     // with GEMM_LOWER: also write the transpose into the upper part
};
lrc_status gemm_f32(hipStream_t st, unsigned flags, int64_t m, int64_t n, int64_t k, float alpha,
                    const float* A, int64_t lda, int64_t sA, const float* B, int64_t ldb,
                    int64_t sB, float beta, float* C, int64_t ldc, int64_t sC, int64_t batch);

// Gram of the smaller side in fp64 from fp32 input: G = M M^T (rows) or M^T M (cols)
lrc_status gram_f64(hipStream_t st, bool rows, int64_t m, int64_t n, const float* M, int64_t ldm,
                    int64_t sM, double* G, int64_t ldg, int64_t sG, int64_t batch);

}  // namespace lrc
