// Dense building blocks of the decomposition: fp32 GEMM on MFMA, fp64 Gram of the
// whitened weight, blocked Cholesky (LASER Methodology 1, Transformation: S_x and S_g
// are Cholesky factors of X and G) and blocked triangular solves for the back-map.
#include "lrc_internal.h"
#include "lrc_dense.h"

namespace lrc {
namespace {

// ---------------------------------------------------------------------------------
// fp32 GEMM: 64 x 64 output tile per workgroup, 4 waves in 2 x 2, each wave a 32 x 32
// block as 2 x 2 v_mfma_f32_16x16x4f32 blocks.  Operands are staged k-major in LDS in
// chunks of GK (a lane reads its fragment element with one 4-byte read); the next
// chunk's global loads (clamped addresses, masked when stored) are in flight while the
// current chunk's MFMAs run.
// Fragment layout (16x16x4): A[row = l%16][k = l/16], B[k = l/16][col = l%16],
// D element r of lane l = D[4*(l/16) + r][l%16].
// ---------------------------------------------------------------------------------
constexpr int GT = 64;
constexpr int GK = 32;
constexpr int GPE = (GT * GK) / 256;   // staged elements per thread per operand
constexpr int WT = GT / 32;            // 16 x 16 blocks per wave side

// VEC: m, n, k, lda, ldb multiples of 4 and A, B 16-byte aligned.  The staged element
// order makes elements e .. e + 3 (e a multiple of 4) contiguous in memory for every
// layout, so each thread stages its operands as 16-byte groups, each wholly inside or
// wholly outside the matrix (groups are clamped as a whole and masked at the LDS store).
template <bool VEC>
__global__ __launch_bounds__(256) void gemm_f32_kernel(unsigned flags, int m, int n, int k, float alpha,
                                                       const float* __restrict__ A, int64_t lda, int64_t sA,
                                                       const float* __restrict__ B, int64_t ldb, int64_t sB,
                                                       float beta, float* __restrict__ C, int64_t ldc, int64_t sC) {
  __shared__ float As[GK][GT + 4];
  __shared__ float Bs[GK][GT + 4];
  A += blockIdx.z * sA;
  B += blockIdx.z * sB;
  C += blockIdx.z * sC;
  // Tiles of a triangular operand carry unequal work; they are dispatched longest first,
  // so that the launch does not end on a few long tiles started late: with k from the
  // tile's first column, column by column (rows within a column); with k up to its last
  // row, bottom row first.  Otherwise row by row, columns within a row.
  int tr_ = blockIdx.y, tc_ = blockIdx.x;
  if ((flags & GEMM_K_FROM_COL) && !(flags & GEMM_K_FROM_ROW)) {
    const int lin = blockIdx.y * gridDim.x + blockIdx.x;
    tc_ = lin / gridDim.y;
    tr_ = lin % gridDim.y;
  } else if (flags & GEMM_K_TO_ROW) {
    tr_ = gridDim.y - 1 - blockIdx.y;
  }
  const int row0 = tr_ * GT, col0 = tc_ * GT;
  if (row0 >= m || col0 >= n) return;
  if ((flags & GEMM_LOWER) && col0 > row0 + GT - 1) return;
  int kb = 0, ke = k;
  if (flags & GEMM_K_FROM_COL) kb = max(kb, col0);
  if (flags & GEMM_K_FROM_ROW) kb = max(kb, row0);
  if (flags & GEMM_K_TO_ROW) ke = min(ke, row0 + GT);
  kb = (kb / GK) * GK;
  const bool ta = flags & GEMM_TA, tb = flags & GEMM_TB;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  f32x4 acc[WT][WT];
#pragma unroll
  for (int i = 0; i < WT; ++i)
#pragma unroll
    for (int j = 0; j < WT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // staged element e = tid + 256 it: (row r, kk) of A and (kk, column c) of B, with the
  // index order that makes consecutive threads read consecutive addresses
  auto a_rk = [&](int e, int& r, int& kk) {
    if (ta) { kk = e / GT; r = e % GT; } else { r = e / GK; kk = e % GK; }
  };
  auto b_kc = [&](int e, int& kk, int& c) {
    if (tb) { c = e / GK; kk = e % GK; } else { kk = e / GT; c = e % GT; }
  };
  float ga[GPE], gb[GPE];
  auto load = [&](int k0) {
    if (VEC) {
#pragma unroll
      for (int g = 0; g < GPE / 4; ++g) {
        const int e = 4 * (tid + g * 256);
        int r, kk, c, kk2;
        a_rk(e, r, kk);
        b_kc(e, kk2, c);
        // the group runs along kk (A) / c (B) when not transposed, along r / kk2 otherwise
        const int gr = ta ? min(row0 + r, m - 4) : min(row0 + r, m - 1);
        const int gk = ta ? min(k0 + kk, k - 1) : min(k0 + kk, k - 4);
        const int gc = tb ? min(col0 + c, n - 1) : min(col0 + c, n - 4);
        const int gk2 = tb ? min(k0 + kk2, k - 4) : min(k0 + kk2, k - 1);
        const float4 va = *reinterpret_cast<const float4*>(ta ? A + int64_t(gk) * lda + gr : A + int64_t(gr) * lda + gk);
        const float4 vb = *reinterpret_cast<const float4*>(tb ? B + int64_t(gc) * ldb + gk2 : B + int64_t(gk2) * ldb + gc);
        ga[4 * g] = va.x;
        ga[4 * g + 1] = va.y;
        ga[4 * g + 2] = va.z;
        ga[4 * g + 3] = va.w;
        gb[4 * g] = vb.x;
        gb[4 * g + 1] = vb.y;
        gb[4 * g + 2] = vb.z;
        gb[4 * g + 3] = vb.w;
      }
    } else {
#pragma unroll
      for (int it = 0; it < GPE; ++it) {
        const int e = tid + it * 256;
        int r, kk, c, kk2;
        a_rk(e, r, kk);
        b_kc(e, kk2, c);
        const int gr = min(row0 + r, m - 1), gk = min(k0 + kk, k - 1);
        const int gc = min(col0 + c, n - 1), gk2 = min(k0 + kk2, k - 1);
        ga[it] = ta ? A[int64_t(gk) * lda + gr] : A[int64_t(gr) * lda + gk];
        gb[it] = tb ? B[int64_t(gc) * ldb + gk2] : B[int64_t(gk2) * ldb + gc];
      }
    }
  };
  auto store = [&](int k0) {
#pragma unroll
    for (int it = 0; it < GPE; ++it) {
      // VEC: group g = it / 4 holds elements 4 (tid + 256 g) + it % 4
      const int e = VEC ? 4 * (tid + (it / 4) * 256) + (it % 4) : tid + it * 256;
      int r, kk, c, kk2;
      a_rk(e, r, kk);
      b_kc(e, kk2, c);
      As[kk][r] = (row0 + r < m && k0 + kk < ke) ? ga[it] : 0.f;
      Bs[kk2][c] = (col0 + c < n && k0 + kk2 < ke) ? gb[it] : 0.f;
    }
  };
  if (kb < ke) load(kb);
  for (int k0 = kb; k0 < ke; k0 += GK) {
    __syncthreads();
    store(k0);
    __syncthreads();
    if (k0 + GK < ke) load(k0 + GK);
#pragma unroll
    for (int kq = 0; kq < GK; kq += 4) {
      float a[WT], b[WT];
#pragma unroll
      for (int i = 0; i < WT; ++i) a[i] = As[kq + (lane >> 4)][wr * 32 + i * 16 + (lane & 15)];
#pragma unroll
      for (int j = 0; j < WT; ++j) b[j] = Bs[kq + (lane >> 4)][wc * 32 + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < WT; ++i)
#pragma unroll
        for (int j = 0; j < WT; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  const bool lower = flags & GEMM_LOWER, mirror = flags & GEMM_MIRROR;
#pragma unroll
  for (int i = 0; i < WT; ++i)
#pragma unroll
    for (int j = 0; j < WT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + wr * 32 + i * 16 + 4 * (lane >> 4) + r;
        const int col = col0 + wc * 32 + j * 16 + (lane & 15);
        if (row >= m || col >= n) continue;
        if (lower && row < col) continue;
        float v = alpha * acc[i][j][r];
        if (beta != 0.f) v += beta * C[int64_t(row) * ldc + col];
        C[int64_t(row) * ldc + col] = v;
        if (mirror && row != col) C[int64_t(col) * ldc + row] = v;
      }
}

// ---------------------------------------------------------------------------------
// fp64 Gram from an fp32 matrix (products exact in fp64): G = M M^T or M^T M, lower
// triangle only.  64 x 64 tiles, 256 threads with 4 x 4 outputs each.
// ---------------------------------------------------------------------------------
// Gram in fp64 on MFMA (v_mfma_f64_16x16x4): one 64 x 64 lower tile per workgroup, four
// waves of 32 x 32 (2 x 2 MFMA blocks).  fp32 inputs are widened exactly; products of two
// fp32 values are exact in fp64, sums are fp64.  The reduction runs in chunks of GRK
// staged through LDS as doubles; the next chunk's loads are in flight during the MFMAs.
constexpr int GRK = 32;
constexpr int GRP = 64 + 4;   // LDS pitch (floats) of a k row

template <bool VEC>
__global__ __launch_bounds__(256) void gram_f64_kernel(bool rows, int p, int q, const float* __restrict__ M,
                                                       int64_t ldm, int64_t sM, double* __restrict__ G,
                                                       int64_t ldg, int64_t sG) {
  // operands stay fp32 in LDS and are widened (exactly) as the MFMA fragments are read
  __shared__ float xs[GRK][GRP];
  __shared__ float ys[GRK][GRP];
  M += blockIdx.z * sM;
  G += blockIdx.z * sG;
  int lin = blockIdx.x, ti = 0;
  while (lin > ti) { lin -= ti + 1; ++ti; }
  const int tj = lin;
  const int dim = rows ? p : q;     // Gram dimension
  const int red = rows ? q : p;     // reduction length
  if (ti * 64 >= dim) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  // staging: 8 elements per thread per operand, as two groups of 4 consecutive elements in
  // memory.  rows: element (c, kk) at M[c * ldm + k]; thread takes c = tid / 4,
  // kk = (tid % 4) * 8 + 4 g + u.  cols: element at M[k * ldm + c]; thread takes
  // kk = tid / 16 + 16 g, c = (tid % 16) * 4 + u.  VEC (dim, red, ldm multiples of 4, 16-byte
  // base): each group is one 16-byte load, wholly in or out of range.
  auto elem = [&](int g, int u, int& c, int& kk) {
    if (rows) { c = tid >> 2; kk = (tid & 3) * 8 + 4 * g + u; } else { kk = (tid >> 4) + 16 * g; c = (tid & 15) * 4 + u; }
  };
  float gx[2][4], gy[2][4];
  auto load = [&](int k0) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      if (VEC) {
        int c, kk;
        elem(g, 0, c, kk);
        if (rows) {
          const int gk = min(k0 + kk, red - 4);
          const int ci = min(ti * 64 + c, dim - 1), cj = min(tj * 64 + c, dim - 1);
          const float4 vx = *reinterpret_cast<const float4*>(M + int64_t(ci) * ldm + gk);
          const float4 vy = *reinterpret_cast<const float4*>(M + int64_t(cj) * ldm + gk);
          gx[g][0] = vx.x; gx[g][1] = vx.y; gx[g][2] = vx.z; gx[g][3] = vx.w;
          gy[g][0] = vy.x; gy[g][1] = vy.y; gy[g][2] = vy.z; gy[g][3] = vy.w;
        } else {
          const int gk = min(k0 + kk, red - 1);
          const int ci = min(ti * 64 + c, dim - 4), cj = min(tj * 64 + c, dim - 4);
          const float4 vx = *reinterpret_cast<const float4*>(M + int64_t(gk) * ldm + ci);
          const float4 vy = *reinterpret_cast<const float4*>(M + int64_t(gk) * ldm + cj);
          gx[g][0] = vx.x; gx[g][1] = vx.y; gx[g][2] = vx.z; gx[g][3] = vx.w;
          gy[g][0] = vy.x; gy[g][1] = vy.y; gy[g][2] = vy.z; gy[g][3] = vy.w;
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          int c, kk;
          elem(g, u, c, kk);
          const int gk = min(k0 + kk, red - 1);
          const int ci = min(ti * 64 + c, dim - 1), cj = min(tj * 64 + c, dim - 1);
          gx[g][u] = rows ? M[int64_t(ci) * ldm + gk] : M[int64_t(gk) * ldm + ci];
          gy[g][u] = rows ? M[int64_t(cj) * ldm + gk] : M[int64_t(gk) * ldm + cj];
        }
      }
    }
  };
  auto store = [&](int k0) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        int c, kk;
        elem(g, u, c, kk);
        const bool okk = k0 + kk < red;
        xs[kk][c] = (okk && ti * 64 + c < dim) ? gx[g][u] : 0.f;
        ys[kk][c] = (okk && tj * 64 + c < dim) ? gy[g][u] : 0.f;
      }
  };
  f64x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
  const int l16 = lane & 15, lq = lane >> 4;
  load(0);
  for (int k0 = 0; k0 < red; k0 += GRK) {
    __syncthreads();
    store(k0);
    __syncthreads();
    if (k0 + GRK < red) load(k0 + GRK);
#pragma unroll
    for (int kk = 0; kk < GRK; kk += 4) {
      double a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = double(xs[kk + lq][wr * 32 + i * 16 + l16]);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = double(ys[kk + lq][wc * 32 + j * 16 + l16]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  // output of an fp64 16 x 16 block: lane l, element e -> row l / 16 + 4 e, column l % 16
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = ti * 64 + wr * 32 + i * 16 + lq + 4 * e, c = tj * 64 + wc * 32 + j * 16 + l16;
        if (r < dim && c < dim && r >= c) G[int64_t(r) * ldg + c] = acc[i][j][e];
      }
}

// ---------------------------------------------------------------------------------
// Cholesky pieces (lower, in place on an fp32 n x n buffer whose strict upper part is 0)
// ---------------------------------------------------------------------------------
// L = lower(S) / cnt + damping * I ; strict upper part zeroed.  S is read lower only.
__global__ void sym_scale_kernel(const float* __restrict__ S, int64_t lds_, int64_t n, double inv_cnt, float damping,
                                 float* __restrict__ L, int64_t ldl, int64_t sS, int64_t sL) {
  S += blockIdx.z * sS;   // slice blockIdx.z of a batch
  L += blockIdx.z * sL;
  const int64_t i = blockIdx.y;
  for (int64_t j = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; j < n; j += int64_t(gridDim.x) * blockDim.x) {
    float v = 0.f;
    if (j <= i) {
      v = float(double(S[i * lds_ + j]) * inv_cnt);
      if (j == i) v += damping;
    }
    L[i * ldl + j] = v;
  }
}

constexpr int NB = 64;  // Cholesky / triangular-solve block size

// unblocked factorisation of the diagonal block at k0 (one workgroup)
// Unblocked Cholesky of one diagonal block (b <= 64), a single wave: lane i keeps row i
// in registers; per column j the pivot comes from lane j, the scaled column goes through
// LDS to every lane (one store per lane, then broadcast reads that the wave's in-order
// LDS queue serves after the store), and each lane updates its own row.
__global__ __launch_bounds__(64) void potf2_kernel(float* __restrict__ L, int64_t ldl, int64_t n, int64_t k0,
                                                   int* __restrict__ info, int64_t sL, int sinfo) {
  L += blockIdx.y * sL;   // slice blockIdx.y of a batch
  info += blockIdx.y * sinfo;
  __shared__ __align__(16) float colv[NB];
  const int lane = threadIdx.x;
  const int b = int(min<int64_t>(NB, n - k0));
  if (*info != 0) return;
  const int rr = min(lane, b - 1);
  float a[NB];
  // a full block at a 16-byte aligned position moves in 16-byte pieces
  const bool vec = b == NB && ldl % 4 == 0 && k0 % 4 == 0 && (reinterpret_cast<uintptr_t>(L) & 15) == 0;
  if (vec) {
#pragma unroll
    for (int c = 0; c < NB; c += 4) {
      const float4 v = *reinterpret_cast<const float4*>(L + (k0 + lane) * ldl + k0 + c);
      a[c] = v.x;
      a[c + 1] = v.y;
      a[c + 2] = v.z;
      a[c + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int c = 0; c < NB; ++c) a[c] = L[(k0 + rr) * ldl + k0 + min(c, b - 1)];
  }
#pragma unroll
  for (int c = 0; c < NB; ++c) a[c] = (c <= lane && lane < b && c < b) ? a[c] : 0.f;
  int fail = 0;   // uniform: the pivot is read from lane j into a scalar register
  // fully unrolled (static register indices); finished or failed columns are skipped.
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    if (j < b && fail == 0) {
      const float piv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[j]), j));
      if (!(piv > 0.f) || !isfinite(piv)) {
        fail = j + 1;
      } else {
        // correctly rounded square root and reciprocal: the smallest singular values of
        // an ill-conditioned whitening are sensitive to the last bits of these pivots
        const float djj = sqrtf(piv);
        const float inv = 1.0f / djj;
        a[j] = lane == j ? djj : (lane > j ? a[j] * inv : a[j]);
        const float lij = a[j];
        colv[lane] = lij;
        // every lane updates its whole row: entries above the diagonal (c > lane) are never
        // read as pivots or multipliers (those come from lanes c > j, column j) and stay
        // finite; the store writes zeros there.  The column is read back four entries per
        // LDS read, all reads issued before the first update (the reads of one wave follow
        // its write in order).
        float4 cv[NB / 4];
#pragma unroll
        for (int g = (j + 1) / 4; g < NB / 4; ++g) cv[g] = *reinterpret_cast<const float4*>(&colv[4 * g]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int g = (j + 1) / 4; g < NB / 4; ++g) {
          if (4 * g > j) a[4 * g] = fmaf(-lij, cv[g].x, a[4 * g]);
          if (4 * g + 1 > j) a[4 * g + 1] = fmaf(-lij, cv[g].y, a[4 * g + 1]);
          if (4 * g + 2 > j) a[4 * g + 2] = fmaf(-lij, cv[g].z, a[4 * g + 2]);
          a[4 * g + 3] = fmaf(-lij, cv[g].w, a[4 * g + 3]);
        }
      }
    }
  }
  if (fail) {
    if (lane == 0) *info = int(k0 + fail);
    return;
  }
  if (vec) {
#pragma unroll
    for (int c = 0; c < NB; c += 4)
      *reinterpret_cast<float4*>(L + (k0 + lane) * ldl + k0 + c) =
          float4{c <= lane ? a[c] : 0.f, c + 1 <= lane ? a[c + 1] : 0.f, c + 2 <= lane ? a[c + 2] : 0.f,
                 c + 3 <= lane ? a[c + 3] : 0.f};
  } else if (lane < b) {
#pragma unroll
    for (int c = 0; c < NB; ++c)
      if (c < b) L[(k0 + lane) * ldl + k0 + c] = c <= lane ? a[c] : 0.f;
  }
}

// Rows below a factored diagonal block: X <- X D^-T (one lane per row, 64 rows per wave).
// Rows are loaded as 16-byte groups when the pitch and base allow; the solve reads each
// row of D from LDS four entries at a time (broadcast reads, the FMAs in column order).
__global__ __launch_bounds__(64) void trsm_panel_kernel(float* __restrict__ L, int64_t ldl, int64_t n, int64_t k0,
                                                        const int* __restrict__ info, int64_t sL, int sinfo) {
  L += blockIdx.y * sL;   // slice blockIdx.y of a batch
  info += blockIdx.y * sinfo;
  __shared__ __align__(16) float D[NB][NB + 4];
  __shared__ float rdiag[NB];
  if (*info != 0) return;
  const int lane = threadIdx.x;
  const int64_t r = k0 + NB + int64_t(blockIdx.x) * 64 + lane;
  const int64_t rc = r < n ? r : n - 1;
  float x[NB], dcol[NB];
  // all loads first: row `lane` of the diagonal block (column of D^T) and this lane's row
  const float* drow = L + (k0 + lane) * ldl + k0;
  const float* xrow = L + rc * ldl + k0;
  if (ldl % 4 == 0 && (reinterpret_cast<uintptr_t>(L) & 15) == 0) {
#pragma unroll
    for (int c = 0; c < NB; c += 4) {
      const float4 dv = *reinterpret_cast<const float4*>(drow + c);
      const float4 xv = *reinterpret_cast<const float4*>(xrow + c);
      dcol[c] = dv.x;
      dcol[c + 1] = dv.y;
      dcol[c + 2] = dv.z;
      dcol[c + 3] = dv.w;
      x[c] = xv.x;
      x[c + 1] = xv.y;
      x[c + 2] = xv.z;
      x[c + 3] = xv.w;
    }
  } else {
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      dcol[c] = drow[c];
      x[c] = xrow[c];
    }
  }
  float dl = 1.f;
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    D[lane][c] = dcol[c];
    dl = c == lane ? dcol[c] : dl;   // static register index, lane-selected
  }
  rdiag[lane] = 1.0f / dl;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    float v = x[j];
#pragma unroll
    for (int c4 = 0; c4 < j; c4 += 4) {
      const float4 d = *reinterpret_cast<const float4*>(&D[j][c4]);
      v = fmaf(-x[c4], d.x, v);
      if (c4 + 1 < j) v = fmaf(-x[c4 + 1], d.y, v);
      if (c4 + 2 < j) v = fmaf(-x[c4 + 2], d.z, v);
      if (c4 + 3 < j) v = fmaf(-x[c4 + 3], d.w, v);
    }
    x[j] = v * rdiag[j];
  }
  if (r < n) {
#pragma unroll
    for (int c = 0; c < NB; ++c) L[r * ldl + k0 + c] = x[c];
  }
}

// Y <- D^-T Y for one diagonal block D (b x b, lower, at (k0, k0) of L) and the b rows
// k0.. of Y (ncol columns, leading dim ldb): one lane per column, the block in LDS.
// Column-oriented: x_c = y_c / D[c][c], then every y_i with i < c drops D[c][i] x_c, so
// a step is one division plus independent updates, and row c of D is read four entries
// per LDS read.
__global__ __launch_bounds__(64) void trsm_upper_diag_kernel(const float* __restrict__ L, int64_t ldl, int64_t k0, int b,
                                                             float* __restrict__ Bm, int64_t ldb, int64_t ncol) {
  __shared__ __align__(16) float D[NB][NB + 4];
  if (b == NB && ldl % 4 == 0 && k0 % 4 == 0 && (reinterpret_cast<uintptr_t>(L) & 15) == 0) {
    // a full block in 16-byte pieces, all loads issued before the first LDS store
    float4 v[NB * NB / 4 / 64];
#pragma unroll
    for (int q = 0; q < NB * NB / 4 / 64; ++q) {
      const int e = threadIdx.x + 64 * q, i = e / (NB / 4), j = 4 * (e % (NB / 4));
      v[q] = *reinterpret_cast<const float4*>(L + (k0 + i) * ldl + k0 + j);
    }
#pragma unroll
    for (int q = 0; q < NB * NB / 4 / 64; ++q) {
      const int e = threadIdx.x + 64 * q, i = e / (NB / 4), j = 4 * (e % (NB / 4));
      *reinterpret_cast<float4*>(&D[i][j]) = v[q];
    }
  } else {
#pragma unroll 16
    for (int e = threadIdx.x; e < NB * NB; e += 64) {
      const int i = e / NB, j = e % NB;
      D[i][j] = (i < b && j < b) ? L[(k0 + i) * ldl + k0 + j] : (i == j ? 1.f : 0.f);
    }
  }
  __syncthreads();
  const int64_t col = int64_t(blockIdx.x) * 64 + threadIdx.x;
  if (col >= ncol) return;
  float y[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) y[i] = (i < b) ? Bm[(k0 + i) * ldb + col] : 0.f;
#pragma unroll
  for (int c = NB - 1; c >= 0; --c) {
    y[c] = y[c] / D[c][c];
    const float xc = y[c];
#pragma unroll
    for (int g = 0; g < c / 4 + 1; ++g) {
      if (4 * g >= c) break;
      const float4 dv = *reinterpret_cast<const float4*>(&D[c][4 * g]);
      y[4 * g] = fmaf(-dv.x, xc, y[4 * g]);
      if (4 * g + 1 < c) y[4 * g + 1] = fmaf(-dv.y, xc, y[4 * g + 1]);
      if (4 * g + 2 < c) y[4 * g + 2] = fmaf(-dv.z, xc, y[4 * g + 2]);
      if (4 * g + 3 < c) y[4 * g + 3] = fmaf(-dv.w, xc, y[4 * g + 3]);
    }
  }
#pragma unroll
  for (int i = 0; i < NB; ++i)
    if (i < b) Bm[(k0 + i) * ldb + col] = y[i];
}

__global__ void transpose_f32_kernel(const float* __restrict__ S, int64_t lds_, float* __restrict__ D, int64_t ldd,
                                     int rows, int cols) {
  __shared__ float t[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  for (int i = threadIdx.y; i < 32; i += 8) {
    const int r = r0 + i, c = c0 + threadIdx.x;
    if (r < rows && c < cols) t[i][threadIdx.x] = S[int64_t(r) * lds_ + c];
  }
  __syncthreads();
  for (int i = threadIdx.y; i < 32; i += 8) {
    const int c = c0 + i, r = r0 + threadIdx.x;
    if (r < rows && c < cols) D[int64_t(c) * ldd + r] = t[threadIdx.x][i];
  }
}

}  // namespace

lrc_status gemm_f32(hipStream_t st, unsigned flags, int64_t m, int64_t n, int64_t k, float alpha, const float* A,
                    int64_t lda, int64_t sA, const float* B, int64_t ldb, int64_t sB, float beta, float* C,
                    int64_t ldc, int64_t sC, int64_t batch) {
  if (m <= 0 || n <= 0 || batch <= 0) return LRC_OK;
  const dim3 grid(unsigned(cdiv(n, GT)), unsigned(cdiv(m, GT)), unsigned(batch));
  // algorithmic flops: 2 m n k, halved for a triangular operand and for a triangular output
  double fl = 2.0 * double(m) * double(n) * double(k) * double(batch);
  if (flags & (GEMM_K_FROM_COL | GEMM_K_FROM_ROW | GEMM_K_TO_ROW)) fl *= 0.5;
  if (flags & GEMM_LOWER) fl *= 0.5;
  ProfScope scope("gemm_f32_kernel", st, fl, 4.0 * double(batch) * (double(m) * k + double(k) * n + 2.0 * double(m) * n));
  const bool vec = m % 4 == 0 && n % 4 == 0 && k % 4 == 0 && lda % 4 == 0 && ldb % 4 == 0 && sA % 4 == 0 &&
                   sB % 4 == 0 && reinterpret_cast<uintptr_t>(A) % 16 == 0 && reinterpret_cast<uintptr_t>(B) % 16 == 0;
  if (vec)
    gemm_f32_kernel<true><<<grid, 256, 0, st>>>(flags, int(m), int(n), int(k), alpha, A, lda, sA, B, ldb, sB, beta, C,
                                                ldc, sC);
  else
    gemm_f32_kernel<false><<<grid, 256, 0, st>>>(flags, int(m), int(n), int(k), alpha, A, lda, sA, B, ldb, sB, beta,
                                                 C, ldc, sC);
  LRC_LAUNCHED();
  return LRC_OK;
}

lrc_status gram_f64(hipStream_t st, bool rows, int64_t p, int64_t q, const float* M, int64_t ldm, int64_t sM,
                    double* G, int64_t ldg, int64_t sG, int64_t batch) {
  const int64_t dim = rows ? p : q;
  const int64_t t = cdiv(dim, 64);
  const dim3 grid(unsigned(t * (t + 1) / 2), 1, unsigned(batch));
  const double other = rows ? double(q) : double(p);
  ProfScope scope("gram_f64_kernel", st, double(batch) * double(dim) * double(dim + 1) * other,
                  double(batch) * (4.0 * double(p) * double(q) + 4.0 * double(dim) * double(dim + 1)));
  const bool vec = dim % 4 == 0 && (rows ? q : p) % 4 == 0 && ldm % 4 == 0 && sM % 4 == 0 &&
                   reinterpret_cast<uintptr_t>(M) % 16 == 0;
  if (vec)
    gram_f64_kernel<true><<<grid, 256, 0, st>>>(rows, int(p), int(q), M, ldm, sM, G, ldg, sG);
  else
    gram_f64_kernel<false><<<grid, 256, 0, st>>>(rows, int(p), int(q), M, ldm, sM, G, ldg, sG);
  LRC_LAUNCHED();
  return LRC_OK;
}

lrc_status cholesky_f32_batched(hipStream_t st, const float* S, int64_t lds_, int64_t sS, int64_t n, int64_t cnt,
                                float damping, float* L, int* info, int sinfo, int64_t batch) {
  if (batch <= 0 || n <= 0) return LRC_OK;
  const int64_t sL = n * n;
  const unsigned nb_ = unsigned(batch);
  const dim3 g(unsigned(std::min<int64_t>(cdiv(n, 256), 64)), unsigned(n), nb_);
  sym_scale_kernel<<<g, 256, 0, st>>>(S, lds_, n, 1.0 / double(cnt), damping, L, n, sS, sL);
  LRC_LAUNCHED();
  for (int64_t k0 = 0; k0 < n; k0 += NB) {
    {
      // work: the block's NB^3 / 3 multiply-adds; bytes: the block read and written
      const double nb = double(std::min<int64_t>(NB, n - k0));
      ProfScope scope("potf2_kernel", st, nb * nb * nb / 3.0 * batch, 8.0 * nb * nb * batch);
      potf2_kernel<<<dim3(1, nb_), 64, 0, st>>>(L, n, n, k0, info, sL, sinfo);
      LRC_LAUNCHED();
    }
    const int64_t below = n - k0 - NB;
    if (below <= 0) break;
    {
      ProfScope scope("trsm_panel_kernel", st, double(below) * NB * NB * batch,
                      (8.0 * double(below) * NB + 4.0 * NB * NB) * batch);
      trsm_panel_kernel<<<dim3(unsigned(cdiv(below, 64)), nb_), 64, 0, st>>>(L, n, n, k0, info, sL, sinfo);
      LRC_LAUNCHED();
    }
    float* p = L + (k0 + NB) * n + k0;
    float* c = L + (k0 + NB) * n + (k0 + NB);
    LRC_TRY(gemm_f32(st, GEMM_TB | GEMM_LOWER, below, below, NB, -1.f, p, n, sL, p, n, sL, 1.f, c, n, sL, batch));
  }
  return LRC_OK;
}

lrc_status cholesky_f32(hipStream_t st, const float* S, int64_t lds_, int64_t n, int64_t cnt, float damping, float* L,
                        int* info) {
  return cholesky_f32_batched(st, S, lds_, 0, n, cnt, damping, L, info, 0, 1);
}

lrc_status trsm_lower_t(hipStream_t st, const float* L, int64_t n, float* Bm, int64_t ldb, int64_t ncol) {
  // right-looking, last block first: solve the diagonal block, then take its rows'
  // contribution out of every row above at once (one GEMM over all of them, 64 deep)
  const int64_t nblk = cdiv(n, NB);
  for (int64_t ib = nblk - 1; ib >= 0; --ib) {
    const int64_t k0 = ib * NB;
    const int b = int(std::min<int64_t>(NB, n - k0));
    {
      ProfScope scope("trsm_upper_diag_kernel", st, double(b) * double(b) * double(ncol),
                      8.0 * double(b) * double(ncol) + 4.0 * double(b) * double(b));
      trsm_upper_diag_kernel<<<unsigned(cdiv(ncol, 64)), 64, 0, st>>>(L, n, k0, b, Bm, ldb, ncol);
      LRC_LAUNCHED();
    }
    if (k0 > 0) {
      // B[0:k0] -= L[k0:k0+b, 0:k0]^T * X[k0:k0+b]
      LRC_TRY(gemm_f32(st, GEMM_TA, k0, ncol, b, -1.f, L + k0 * n, n, 0, Bm + k0 * ldb, ldb, 0, 1.f, Bm, ldb, 0, 1));
    }
  }
  return LRC_OK;
}

lrc_status transpose_f32(hipStream_t st, const float* S, int64_t lds_, float* D, int64_t ldd, int64_t rows,
                         int64_t cols) {
  const dim3 grid(unsigned(cdiv(cols, 32)), unsigned(cdiv(rows, 32)));
  transpose_f32_kernel<<<grid, dim3(32, 8), 0, st>>>(S, lds_, D, ldd, int(rows), int(cols));
  LRC_LAUNCHED();
  return LRC_OK;
}

}  // namespace lrc
