// Component scores (LASER technical summary, Methodology 2: empirical-Fisher importance
// score; K-FAC: the loss of dropping one component alone).
//
//   FISHER: s_i = 1/(2N) sum_t (b_t . left_i)^2 (a_t . right_i)^2
//
// Both projections P = A Right^T (N x k) and Q = B Left (N x k) are formed tile by tile
// and never stored: a workgroup squares and multiplies its P and Q tiles and sums its
// tokens in a fixed order; a second pass adds the token-tile partial sums in order
// (fp64), so the result is bit-reproducible.
//
// bf16 activations (widths a multiple of 8) run on MFMA: each fp32 factor f is split into
// bf16 parts f = hi + lo + r with hi = bf16(f), lo = bf16(f - hi), |r| <= 2^-16 |f|, and
// a . f is taken as (a . hi) + (a . lo) with bf16 x bf16 products (exact) accumulated in
// fp32.  A workgroup owns 256 tokens x 128 components; each of its eight waves holds the
// P and Q accumulators of 64 tokens x 64 components; the activation and factor tiles
// (hi and lo) of each 64-wide reduction chunk are shared through LDS.  fp32 activations
// use a VALU kernel of 64 x 64 tiles.
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

// ---------------------------------------------------------------------------------
// MFMA path (bf16 activations)
// ---------------------------------------------------------------------------------
constexpr int FT = 256;      // tokens per workgroup (4 token groups of 64)
constexpr int FC = 128;      // components per workgroup
constexpr int FK = 64;       // reduction chunk
constexpr int FP = FK + 8;   // LDS row pitch of a factor tile (bf16): 144 B, conflict-free 16-B reads

// hi/lo bf16 split of fp32 values, element-wise (row-major kept)
__global__ void split_kernel(const float* __restrict__ F, int64_t total, uint16_t* __restrict__ hi,
                             uint16_t* __restrict__ lo) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += int64_t(gridDim.x) * blockDim.x) {
    const float f = F[i];
    const uint16_t h = f32_to_bf16_bits(f);
    hi[i] = h;
    lo[i] = f32_to_bf16_bits(f - bf16_bits_to_f32(h));
  }
}

// hi/lo bf16 split with a transpose: F is rows x cols, hi and lo are cols x rows
__global__ __launch_bounds__(256) void split_transpose_kernel(const float* __restrict__ F, int rows, int cols,
                                                              uint16_t* __restrict__ hi, uint16_t* __restrict__ lo) {
  __shared__ float t[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    t[i][tx] = (r < rows && c < cols) ? F[int64_t(r) * cols + c] : 0.f;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows) {
      const float f = t[tx][i];
      const uint16_t h = f32_to_bf16_bits(f);
      hi[int64_t(c) * rows + r] = h;
      lo[int64_t(c) * rows + r] = f32_to_bf16_bits(f - bf16_bits_to_f32(h));
    }
  }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// source of the zero pieces that pad the Fisher kernel's staged tiles
__device__ __attribute__((aligned(16))) uint32_t fisher_zero16[4] = {0u, 0u, 0u, 0u};  // never written

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

constexpr int FW = 8;                    // waves per workgroup: 4 token groups of 64 x 2 component halves
constexpr int FNF = FC / 32 / (FW / 4);  // 32-component blocks per wave
constexpr int FS_T = 4;       // token tiles per XCD super-tile
constexpr int FS_C = 8;       // component tiles per XCD super-tile

// acc[f][nf] (32 tokens x 32 components each) += X[tokens, 0:d] . F[components, 0:d]^T
// for this wave's 64 tokens (tile rows 64 tg ..) and its components (32 FNF ch .. of the
// workgroup's 128), with F given as bf16 hi and lo parts (components x d, row-major).
// Both the workgroup's activation tile (256 tokens) and its factor tile (128 components,
// hi and lo) go through LDS, two stages of one 64-wide reduction chunk each: the global
// loads are whole 128-byte row pieces (8 lanes per row), so every cache line a load
// instruction touches is used in full; rows are padded to FP so that the fragment reads
// (one row per lane) are conflict-free.  The loads of the next two chunks are in flight in
// registers while the current one is computed.
__device__ __forceinline__ void fisher_phase(const uint16_t* __restrict__ X, int d, int64_t n, int64_t t0, int tg,
                                             int ch, const uint16_t* __restrict__ Fh,
                                             const uint16_t* __restrict__ Fl, int k, int c0, uint16_t* fs,
                                             uint16_t* xs, f32x16 (&acc)[2][FNF]) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int lr = lane & 31, lh = lane >> 5;
  const int nch = (d + FK - 1) / FK;
  // staging: thread takes 16-B groups g = tid + 64 FW q: row g / 8, column group g % 8
  constexpr int FQ = FC * 8 / (64 * FW);   // factor groups per thread per part
  constexpr int XQ = FT * 8 / (64 * FW);   // activation groups per thread
  const int grow = tid >> 3, gcol = (tid & 7) * 8;
  // pieces outside the matrices (columns past d, factor rows past k, tokens past n) are
  // read from a 16-byte zero constant: the choice is made on the address, so a store to
  // LDS takes the loaded registers as they are and waits only for its own loads
  const uint16_t* zero = reinterpret_cast<const uint16_t*>(fisher_zero16);
  auto load_f = [&](u32x4 (&g)[2][FQ], u32x4 (&ga)[XQ], int kc) {
    const bool colok = kc + gcol < d;
    const int col = min(kc + gcol, d - 8);
#pragma unroll
    for (int q = 0; q < FQ; ++q) {
      const int row = c0 + grow + 8 * FW * q;
      const bool ok = colok && row < k;
      const int64_t off = int64_t(min(row, k - 1)) * d + col;
      g[0][q] = *reinterpret_cast<const u32x4*>(ok ? Fh + off : zero);
      g[1][q] = *reinterpret_cast<const u32x4*>(ok ? Fl + off : zero);
    }
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
      const int64_t row = t0 + grow + 8 * FW * q;
      const bool ok = colok && row < n;
      ga[q] = *reinterpret_cast<const u32x4*>(ok ? X + min<int64_t>(row, n - 1) * d + col : zero);
    }
  };
  auto store_f = [&](const u32x4 (&g)[2][FQ], const u32x4 (&ga)[XQ], int buf) {
#pragma unroll
    for (int q = 0; q < FQ; ++q)
#pragma unroll
      for (int hl = 0; hl < 2; ++hl)
        *reinterpret_cast<u32x4*>(fs + (buf * 2 + hl) * (FC * FP) + (grow + 8 * FW * q) * FP + gcol) = g[hl][q];
#pragma unroll
    for (int q = 0; q < XQ; ++q)
      *reinterpret_cast<u32x4*>(xs + buf * (FT * FP) + (grow + 8 * FW * q) * FP + gcol) = ga[q];
  };
  // the four (or eight) hi products of a step, then its lo products: an MFMA never waits
  // for the result of the one issued just before it
  auto compute = [&](int buf) {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      u32x4 fr[2][FNF], ar[2];
#pragma unroll
      for (int f = 0; f < 2; ++f)
        ar[f] = *reinterpret_cast<const u32x4*>(xs + buf * (FT * FP) + (tg * 64 + f * 32 + lr) * FP + s4 * 16 +
                                                lh * 8);
#pragma unroll
      for (int nf = 0; nf < FNF; ++nf) {
        const int off = (ch * 32 * FNF + nf * 32 + lr) * FP + s4 * 16 + lh * 8;
        fr[0][nf] = *reinterpret_cast<const u32x4*>(fs + (buf * 2 + 0) * (FC * FP) + off);
        fr[1][nf] = *reinterpret_cast<const u32x4*>(fs + (buf * 2 + 1) * (FC * FP) + off);
      }
#pragma unroll
      for (int hl = 0; hl < 2; ++hl)
#pragma unroll
        for (int nf = 0; nf < FNF; ++nf)
#pragma unroll
          for (int f = 0; f < 2; ++f)
            acc[f][nf] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ar[f]), as_bf16x8(fr[hl][nf]),
                                                                 acc[f][nf], 0, 0, 0);
    }
  };
  // two register sets: the loads of chunk c + 3 are issued after chunk c is computed and
  // stored to LDS after chunk c + 2 is computed, so two compute phases cover their latency.
  // The loop body has no branch: the chunk count is rounded up to even (a chunk past the
  // end loads zeros, whose products add exactly 0), and loads run past the last chunk
  // (reading the zero constant).  So on every path the loads a store waits for are
  // followed by exactly one newer set, which the wait before the store leaves in flight.
  const int nch2 = (nch + 1) & ~1;
  u32x4 g0[2][FQ], ga0[XQ], g1[2][FQ], ga1[XQ];
  load_f(g0, ga0, 0);
  load_f(g1, ga1, FK);
  store_f(g0, ga0, 0);
  load_f(g0, ga0, 2 * FK);
  __syncthreads();
  for (int c = 0; c < nch2; c += 2) {
    compute(0);
    store_f(g1, ga1, 1);
    load_f(g1, ga1, (c + 3) * FK);
    __syncthreads();
    compute(1);
    store_f(g0, ga0, 0);
    load_f(g0, ga0, (c + 4) * FK);
    __syncthreads();
  }
}

// Workgroup numbering (consecutive workgroup ids go to consecutive XCDs): the 32
// workgroups an XCD runs side by side form one super-tile of 4 token tiles x 8 component
// tiles, so at every reduction step the L2 of that XCD holds 4 activation slices and 8
// factor slices, each fetched once and read by 8 or 4 workgroups (a column of 32 component
// tiles per XCD would fetch every factor byte for one workgroup only).  Eight waves: wave
// w takes tokens 64 (w / 2) .. of the tile and components 64 (w % 2) .. of the
// workgroup's 128, so two waves share each SIMD (128 accumulator registers each) and cover
// each other's latencies; every activation fragment read from LDS feeds four MFMAs (two
// component blocks, hi and lo), every factor fragment two.
__global__ __launch_bounds__(64 * FW, 1) void fisher_mfma_kernel(const uint16_t* __restrict__ A,
                                                                 const uint16_t* __restrict__ B, int64_t n,
                                                                 int d_in, int d_out, const uint16_t* __restrict__ Rh,
                                                                 const uint16_t* __restrict__ Rl,
                                                                 const uint16_t* __restrict__ Lh,
                                                                 const uint16_t* __restrict__ Ll, int k, int n_ct,
                                                                 int n_tt, float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint16_t fs[2 * 2 * FC * FP];
  __shared__ __attribute__((aligned(16))) uint16_t xs[2 * FT * FP];
  __shared__ float red[FT / 64][FC];
  const int xcd = blockIdx.x & 7;
  const int i = blockIdx.x >> 3;
  const int w = i % (FS_T * FS_C);
  const int sup = (i / (FS_T * FS_C)) * 8 + xcd;     // super-tile
  const int n_sc = (n_ct + FS_C - 1) / FS_C;
  const int tt = (sup / n_sc) * FS_T + w / FS_C;
  const int ct = (sup % n_sc) * FS_C + w % FS_C;
  if (tt >= n_tt || ct >= n_ct) return;
  const int c0 = ct * FC;
  const int64_t t0 = int64_t(tt) * FT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tg = wave / (FW / 4), ch = wave % (FW / 4);
  const int64_t tw = t0 + tg * 64;
  f32x16 accp[2][FNF], accq[2][FNF];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int nf = 0; nf < FNF; ++nf)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        accp[f][nf][e] = 0.f;
        accq[f][nf][e] = 0.f;
      }
  fisher_phase(A, d_in, n, t0, tg, ch, Rh, Rl, k, c0, fs, xs, accp);
  fisher_phase(B, d_out, n, t0, tg, ch, Lh, Ll, k, c0, fs, xs, accq);
  // output layout of a 32 x 32 block: lane l, element e -> token row 8 (e / 4) + 4 (l / 32) + e % 4,
  // component column l % 32
  const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int nf = 0; nf < FNF; ++nf) {
    float sum = 0.f;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t t = tw + f * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
        const float pv = accp[f][nf][e], qv = accq[f][nf][e];
        // rows past the last token were staged as zeros; the mask keeps them out in any case
        sum = fmaf(t < n ? pv * pv : 0.f, qv * qv, sum);
      }
    sum += __shfl_xor(sum, 32);
    if (lh == 0) red[tg][ch * 32 * FNF + nf * 32 + lr] = sum;
  }
  __syncthreads();
  if (tid < FC && c0 + tid < k)
    partial[int64_t(tt) * k + c0 + tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

__global__ void fisher_final_kernel(const float* __restrict__ partial, int ntb, int k, int accumulate, int finalize,
                                    double inv2n, float* __restrict__ scores, int32_t* __restrict__ info) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= k) return;
  double s = accumulate ? double(scores[i]) : 0.0;
  for (int b = 0; b < ntb; ++b) s += double(partial[int64_t(b) * k + i]);
  if (finalize) s *= inv2n;
  const float f = float(s);
  scores[i] = f;
  if (info && !isfinite(f)) *info = LRC_ENONFINITE;
}

__global__ void kfac_kernel(const float* __restrict__ sigma, int k, float* __restrict__ scores,
                            int32_t* __restrict__ info) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= k) return;
  const float f = 0.5f * sigma[i] * sigma[i];
  scores[i] = f;
  if (info && !isfinite(f)) *info = LRC_ENONFINITE;
}

}  // namespace
}  // namespace lrc

using namespace lrc;

namespace {
// workspace of the MFMA path: token-tile partials, then the hi/lo parts of Right
// (k x d_in) and of Left^T (k x d_out)
struct FisherWs {
  float* partial;
  uint16_t *rh, *rl, *lh, *ll;
};
FisherWs carve_fisher_mfma(Carve& cv, int64_t n_tokens, int64_t d_in, int64_t d_out, int64_t k) {
  FisherWs w;
  w.partial = cv.take<float>(size_t(std::max<int64_t>(1, cdiv(n_tokens, FT)) * k));
  w.rh = cv.take<uint16_t>(size_t(k * d_in));
  w.rl = cv.take<uint16_t>(size_t(k * d_in));
  w.lh = cv.take<uint16_t>(size_t(k * d_out));
  w.ll = cv.take<uint16_t>(size_t(k * d_out));
  return w;
}
// the MFMA kernel reads activation rows in 16-byte pieces
bool fisher_use_mfma(lrc_dtype dt, const void* A, const void* B, int64_t d_in, int64_t d_out) {
  return dt == LRC_BF16 && d_in % 8 == 0 && d_out % 8 == 0 && reinterpret_cast<uintptr_t>(A) % 16 == 0 &&
         reinterpret_cast<uintptr_t>(B) % 16 == 0;
}
}  // namespace

extern "C" size_t lrc_score_components_workspace(int64_t n_tokens, int64_t d_in, int64_t d_out, int64_t k,
                                                 uint32_t flags) {
  if (n_tokens < 0 || k <= 0 || d_in <= 0 || d_out <= 0) return 0;
  if (!(flags & LRC_SCORE_FISHER)) return 0;
  // enough for either kernel (the activation type is not known here)
  Carve valu(nullptr);
  valu.take<float>(size_t(cdiv(n_tokens, ST) * k));
  Carve mfma(nullptr);
  carve_fisher_mfma(mfma, n_tokens, d_in, d_out, k);
  return std::max(valu.bytes(), mfma.bytes());
}

extern "C" lrc_status lrc_score_components(const void* A, const void* B, lrc_dtype dt, int64_t n_tokens, int64_t d_in,
                                           int64_t d_out, const float* left, const float* right, const float* sigma,
                                           int64_t k, uint32_t flags, int accumulate, int finalize, int64_t n_total,
                                           float* scores, int32_t* info, void* ws, size_t ws_bytes, void* stream) {
  if (flags != LRC_SCORE_FISHER && flags != LRC_SCORE_KFAC) return LRC_EDTYPE;
  if (scores == nullptr || k <= 0 || k > (int64_t(1) << 30)) return LRC_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (flags == LRC_SCORE_KFAC) {
    if (sigma == nullptr) return LRC_EINVAL;
    kfac_kernel<<<unsigned(cdiv(k, 256)), 256, 0, st>>>(sigma, int(k), scores, info);
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
  const double inv2n = finalize ? 1.0 / (2.0 * double(n_total)) : 1.0;
  if (fisher_use_mfma(dt, A, B, d_in, d_out)) {
    Carve cv(ws);
    const FisherWs w = carve_fisher_mfma(cv, n_tokens, d_in, d_out, k);
    const int n_tt = int(cdiv(n_tokens, FT));
    if (n_tt > 0) {
      {
        const int64_t tot = k * d_in;
        split_kernel<<<unsigned(std::min<int64_t>(cdiv(tot, 256), 8192)), 256, 0, st>>>(right, tot, w.rh, w.rl);
        LRC_LAUNCHED();
        const dim3 g(unsigned(cdiv(k, 64)), unsigned(cdiv(d_out, 64)));
        split_transpose_kernel<<<g, 256, 0, st>>>(left, int(d_out), int(k), w.lh, w.ll);
        LRC_LAUNCHED();
      }
      const int n_ct = int(cdiv(k, FC));
      // super-tiles of FS_T token tiles x FS_C component tiles, dealt to the 8 XCDs
      const int64_t n_sup = cdiv(n_tt, FS_T) * cdiv(n_ct, FS_C);
      const int64_t nblk = cdiv(n_sup, 8) * 8 * FS_T * FS_C;
      if (nblk > (int64_t(1) << 31) - 1) return LRC_EINVAL;
      // algorithmic work as for the VALU kernel below; the bytes count the bf16 hi/lo
      // factor copies this kernel reads
      ProfScope scope("fisher_mfma_kernel", st,
                      2.0 * double(n_tokens) * double(k) * double(d_in + d_out) + 3.0 * double(n_tokens) * double(k),
                      2.0 * double(n_tokens) * double(d_in + d_out) + 4.0 * double(k) * double(d_in + d_out) +
                          4.0 * double(n_tt) * double(k));
      fisher_mfma_kernel<<<unsigned(nblk), 64 * FW, 0, st>>>(static_cast<const uint16_t*>(A),
                                                         static_cast<const uint16_t*>(B), n_tokens, int(d_in),
                                                         int(d_out), w.rh, w.rl, w.lh, w.ll, int(k), n_ct, n_tt,
                                                         w.partial);
      LRC_LAUNCHED();
    }
    fisher_final_kernel<<<unsigned(cdiv(k, 256)), 256, 0, st>>>(w.partial, n_tt, int(k), accumulate, finalize, inv2n,
                                                                 scores, info);
    LRC_LAUNCHED();
    return LRC_OK;
  }
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
  fisher_final_kernel<<<unsigned(cdiv(k, 256)), 256, 0, st>>>(partial, ntb, int(k), accumulate, finalize, inv2n,
                                                               scores, info);
  LRC_LAUNCHED();
  return LRC_OK;
}
