// Covariance streaming: C[lower] += A^T A  (bf16 MFMA SYRK, fp32 SYRK, int8 QAW pre-pass).
//
// LASER technical summary, Methodology 1 (K-FAC surrogate: activation / gradient
// covariances estimated on a calibration set; QAW: estimated from quantised
// activations) and Swift-SVD technical summary 2A (incremental, one-pass aggregation of
// a covariance over batches of tokens).
//
// bf16 path (the hot one).  The reduction axis is the token axis, which is the strided
// axis of the token-major input, while an MFMA operand wants 8 consecutive reduction
// elements per lane.  Each thread therefore loads an 8 tokens x 8 channels block with
// eight 16-byte loads, transposes it in registers (v_perm-style half-word shuffles) and
// stores it channel-major into LDS, from where a lane reads a whole MFMA fragment with
// one 16-byte LDS read.  Tiles are 256 x 256 of the lower triangle, 8 waves each own a
// 128 x 64 block computed with v_mfma_f32_32x32x16_bf16 (fp32 accumulation of exact
// bf16 products).  Tokens are split S ways so that the launch fills the chip; partial
// tiles are summed in split order by whichever workgroup of a tile finishes last (an
// arrival counter, no waiting), so results are bit-reproducible.  Workgroups of one
// split are mapped so that each XCD works on one compact group of tiles over the same
// token range: the operand panels they share stay in that XCD's L2.
#include "lrc_internal.h"

namespace lrc {
namespace {

constexpr int TB = 256;              // tile edge in channels
constexpr int KS = 64;               // tokens per LDS stage
constexpr int PITCH = KS + 8;        // bf16 per channel row in LDS: 144 B
constexpr int NTH = 512;             // threads per workgroup
constexpr int OPER = TB * PITCH;     // bf16 per operand per stage
constexpr int NXCD = 8;              // XCDs on MI355X
constexpr int QAW_CHUNK = 32768;     // tokens per QAW pre-pass chunk

struct TileRC { int ti, tj; };

// lower-triangle tile (ti >= tj) of linear index `lin`, tiles grouped in 4 x 4 super-tiles
__device__ __forceinline__ TileRC tile_of(int lin, int n1) {
  constexpr int G = 4;
  const int ns = (n1 + G - 1) / G;
  int acc = 0;
  for (int si = 0; si < ns; ++si) {
    for (int sj = 0; sj <= si; ++sj) {
      const int r0 = si * G, r1 = min(n1, r0 + G), c0 = sj * G, c1 = min(n1, c0 + G);
      const int cnt = (si != sj) ? (r1 - r0) * (c1 - c0) : (r1 - r0) * (r1 - r0 + 1) / 2;
      if (lin < acc + cnt) {
        int local = lin - acc;
        if (si != sj) {
          const int w = c1 - c0;
          return {r0 + local / w, c0 + local % w};
        }
        int r = 0;
        while (local > r) { local -= r + 1; ++r; }
        return {r0 + r, r0 + local};
      }
      acc += cnt;
    }
  }
  return {-1, -1};
}

template <bool VEC>
__device__ __forceinline__ void load_block(const uint16_t* __restrict__ X, int64_t ldx, int64_t t0,
                                           int64_t t_end, int c, int d, uint4 (&r)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t t = t0 + j;
    if (VEC) {
      if (t < t_end && c < d)
        r[j] = *reinterpret_cast<const uint4*>(X + t * ldx + c);
      else
        r[j] = make_uint4(0u, 0u, 0u, 0u);
    } else {
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = (t < t_end && c + e < d) ? X[t * ldx + c + e] : 0u;
      r[j] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                        h[6] | (h[7] << 16));
    }
  }
}

// r[j] holds channels 0..7 of token j (two per word); o[c] receives tokens 0..7 of channel c
__device__ __forceinline__ void transpose8(const uint4 (&r)[8], uint4 (&o)[8]) {
  uint32_t in[32];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    in[4 * j + 0] = r[j].x; in[4 * j + 1] = r[j].y; in[4 * j + 2] = r[j].z; in[4 * j + 3] = r[j].w;
  }
  uint32_t out[32];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a = in[(2 * p) * 4 + (c >> 1)];
      const uint32_t b = in[(2 * p + 1) * 4 + (c >> 1)];
      out[4 * c + p] = (c & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) o[c] = make_uint4(out[4 * c], out[4 * c + 1], out[4 * c + 2], out[4 * c + 3]);
}

// C[lower] += X^T Y over tokens [0, n) (X, Y: n x d bf16 bits, leading dim ldx).
// grid.x = NXCD * tiles_per_xcd * splits.
template <bool VEC>
__global__ __launch_bounds__(NTH, 1) void syrk_bf16_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Y, int64_t ldx, int64_t n, int d,
    int n1, int n_tiles, int tiles_per_xcd, int splits, int steps_per_split, float* __restrict__ C,
    int64_t ldc, float* __restrict__ partial, unsigned* __restrict__ counters) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 2 * OPER];
  __shared__ int s_last;

  const int b = blockIdx.x;
  const int xcd = b % NXCD;
  const int local = b / NXCD;
  const int split = local / tiles_per_xcd;
  const int tile = xcd * tiles_per_xcd + local % tiles_per_xcd;
  if (tile >= n_tiles || split >= splits) return;
  const TileRC tc = tile_of(tile, n1);
  const int ti = tc.ti, tj = tc.tj;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 2, wc = wave & 3;

  // loader role: operand, channel group, token group
  const int op = tid >> 8;
  const int u = tid & 255;
  const int cg = u >> 3, tg = u & 7;
  const uint16_t* src = op ? Y : X;
  const int chan = (op ? tj : ti) * TB + cg * 8;

  const int64_t tok_begin = int64_t(split) * steps_per_split * KS;
  const int64_t tok_end = min<int64_t>(n, tok_begin + int64_t(steps_per_split) * KS);
  const int nsteps = tok_end > tok_begin ? int((tok_end - tok_begin + KS - 1) / KS) : 0;

  // wave-level skip of 32x32 blocks strictly above the diagonal of a diagonal tile
  bool live[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      live[i][j] = (ti != tj) || (wr * 128 + i * 32 + 31 >= wc * 64 + j * 32);

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  uint4 pre[8];
  auto stage_store = [&](int buf) {
    uint4 o[8];
    transpose8(pre, o);
    uint16_t* dst = lds + (buf * 2 + op) * OPER + (cg * 8) * PITCH + tg * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) *reinterpret_cast<uint4*>(dst + c * PITCH) = o[c];
  };

  if (nsteps > 0) {
    load_block<VEC>(src, ldx, tok_begin + tg * 8, tok_end, chan, d, pre);
    stage_store(0);
  }
  __syncthreads();

  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) load_block<VEC>(src, ldx, tok_begin + int64_t(s + 1) * KS + tg * 8, tok_end, chan, d, pre);

    const uint16_t* xa = lds + (buf * 2 + 0) * OPER;
    const uint16_t* yb = lds + (buf * 2 + 1) * OPER;
#pragma unroll
    for (int kk = 0; kk < KS / 16; ++kk) {
      const int koff = kk * 16 + (lane >> 5) * 8;
      bf16x8 fa[4], fb[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(xa + (wr * 128 + i * 32 + (lane & 31)) * PITCH + koff);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(yb + (wc * 64 + j * 32 + (lane & 31)) * PITCH + koff);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (live[i][j]) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (s + 1 < nsteps) stage_store(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  Output layout of a 32x32 block: lane l, element e ->
  //      row 8*(e/4) + 4*(l/32) + e%4, column l%32.
  const int r_base = wr * 128, c_base = wc * 64;
  if (splits == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (!live[i][j]) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int lr = r_base + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          const int lc = c_base + j * 32 + (lane & 31);
          const int row = ti * TB + lr, col = tj * TB + lc;
          if (row < d && col < d && (ti != tj || row >= col)) C[int64_t(row) * ldc + col] += acc[i][j][e];
        }
      }
    return;
  }

  float* part = partial + (int64_t(split) * n_tiles + tile) * (TB * TB);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int lr = r_base + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int lc = c_base + j * 32 + (lane & 31);
        part[lr * TB + lc] = acc[i][j][e];
      }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = atomicAdd(&counters[tile], 1u);
    s_last = (prev == unsigned(splits - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  // last arriving split: sum all splits in split order, add into C
  for (int idx = tid; idx < TB * TB / 4; idx += NTH) {
    const int lr = (idx * 4) / TB, lc = (idx * 4) % TB;
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int s2 = 0; s2 < splits; ++s2) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(partial + (int64_t(s2) * n_tiles + tile) * (TB * TB) + lr * TB + lc);
      sum += v;
    }
    const int row = ti * TB + lr;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int col = tj * TB + lc + e;
      if (row < d && col < d && (ti != tj || row >= col)) C[int64_t(row) * ldc + col] += sum[e];
    }
  }
  if (tid == 0) counters[tile] = 0u;
}

__global__ void zero_u32_kernel(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// ---- QAW pre-pass: per token scale, integer code q, and s^2 q split into bf16 hi + lo
template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p) { return bf16_bits_to_f32(*p); }

template <typename T>
__global__ __launch_bounds__(256) void qaw_prepass_kernel(const T* __restrict__ A, int64_t lda, int d,
                                                          uint16_t* __restrict__ Q, uint16_t* __restrict__ H,
                                                          uint16_t* __restrict__ L, int64_t ldq) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const T* row = A + t * lda;
  float m = 0.f;
  for (int j = threadIdx.x; j < d; j += 256) m = fmaxf(m, fabsf(load_as_f32(row + j)));
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = __fdiv_rn(m, 127.0f);
  const float s2 = s * s;
  for (int j = threadIdx.x; j < d; j += 256) {
    const float a = load_as_f32(row + j);
    float q = 0.f;
    if (s > 0.f) q = fminf(fmaxf(rintf(__fdiv_rn(a, s)), -127.f), 127.f);
    const float w = s2 * q;
    const uint16_t hi = f32_to_bf16_bits(w);
    const uint16_t lo = f32_to_bf16_bits(w - bf16_bits_to_f32(hi));
    Q[t * ldq + j] = f32_to_bf16_bits(q);  // |q| <= 127: exact in bf16
    H[t * ldq + j] = hi;
    L[t * ldq + j] = lo;
  }
}

// ---- fp32 input: plain LDS-tiled SYRK, 64 x 64 lower tiles, no split (deterministic)
__global__ __launch_bounds__(256) void syrk_f32_kernel(const float* __restrict__ A, int64_t lda, int64_t n,
                                                       int d, float* __restrict__ C, int64_t ldc) {
  __shared__ float xs[16][65];
  __shared__ float ys[16][65];
  int lin = blockIdx.x, ti = 0;
  while (lin > ti) { lin -= ti + 1; ++ti; }
  const int tj = lin;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int64_t t0 = 0; t0 < n; t0 += 16) {
    for (int e = threadIdx.x; e < 16 * 64; e += 256) {
      const int r = e >> 6, c = e & 63;
      const int64_t t = t0 + r;
      const int cx = ti * 64 + c, cy = tj * 64 + c;
      xs[r][c] = (t < n && cx < d) ? A[t * lda + cx] : 0.f;
      ys[r][c] = (t < n && cy < d) ? A[t * lda + cy] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float xv[4], yv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { xv[i] = xs[r][ty * 4 + i]; yv[i] = ys[r][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xv[i], yv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = ti * 64 + ty * 4 + i, col = tj * 64 + tx * 4 + j;
      if (row < d && col < d && row >= col) C[int64_t(row) * ldc + col] += acc[i][j];
    }
}

struct SyrkPlan {
  int n1, n_tiles, tiles_per_xcd, splits, steps_per_split;
};

SyrkPlan plan_syrk(int64_t n, int64_t d, int max_splits = 64) {
  SyrkPlan p;
  p.n1 = int(cdiv(d, TB));
  p.n_tiles = p.n1 * (p.n1 + 1) / 2;
  p.tiles_per_xcd = int(cdiv(p.n_tiles, NXCD));
  const int64_t nsteps = cdiv(n, KS);
  // The plan depends on the shape only (a 256-CU MI355X is assumed), so that workspace
  // sizes are known without a device and equal inputs give equal bits on any device.
  const int cus = 256;
  // cost model: workgroup rounds x (steps per workgroup + partial write/reduce overhead)
  int best = 1;
  double best_cost = 1e300;
  const int smax = int(std::min<int64_t>(std::max(1, max_splits), std::max<int64_t>(1, nsteps)));
  for (int s = 1; s <= smax; ++s) {
    const int64_t wgs = int64_t(NXCD) * p.tiles_per_xcd * s;
    const double rounds = double(cdiv(wgs, cus));
    const double cost = rounds * (double(cdiv(nsteps, s)) + (s > 1 ? 4.0 : 0.0));
    if (cost < best_cost - 1e-9) { best_cost = cost; best = s; }
  }
  p.splits = best;
  p.steps_per_split = int(cdiv(nsteps, best));
  p.splits = int(cdiv(nsteps, p.steps_per_split));  // drop empty splits
  if (p.splits < 1) p.splits = 1;
  return p;
}

size_t syrk_partial_floats(const SyrkPlan& p) {
  return p.splits > 1 ? size_t(p.splits) * p.n_tiles * TB * TB : 0;
}

// bf16 SYRK launch over a token block, partial/counter space from the carve
lrc_status launch_syrk_bf16(hipStream_t st, const uint16_t* X, const uint16_t* Y, int64_t ldx, int64_t n,
                            int64_t d, float* C, int64_t ldc, float* partial, unsigned* counters, int split_cap) {
  if (n <= 0) return LRC_OK;
  const SyrkPlan p = plan_syrk(n, d, split_cap);  // never more splits than the partial buffer holds
  const bool vec = (d % 8 == 0) && (ldx % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(Y) & 15) == 0);
  const dim3 grid(unsigned(NXCD * p.tiles_per_xcd * p.splits));
  // algorithmic work: n d (d + 1) / 2 products and adds for the lower triangle incl. the
  // diagonal; bytes: the token block once (twice when the two operands differ) plus one
  // read and one write of the fp32 lower triangle
  const double tri = double(d) * double(d + 1) / 2;
  ProfScope scope("syrk_bf16_kernel", st, 2.0 * double(n) * tri,
                  double(n) * double(d) * 2.0 * (X == Y ? 1 : 2) + 8.0 * tri);
  if (vec)
    syrk_bf16_kernel<true><<<grid, NTH, 0, st>>>(X, Y, ldx, n, int(d), p.n1, p.n_tiles, p.tiles_per_xcd,
                                                 p.splits, p.steps_per_split, C, ldc, partial, counters);
  else
    syrk_bf16_kernel<false><<<grid, NTH, 0, st>>>(X, Y, ldx, n, int(d), p.n1, p.n_tiles, p.tiles_per_xcd,
                                                  p.splits, p.steps_per_split, C, ldc, partial, counters);
  LRC_LAUNCHED();
  return LRC_OK;
}

size_t cov_workspace(lrc_dtype dt, int64_t n, int64_t d, uint32_t flags, void* base, float** partial,
                     unsigned** counters, uint16_t** q, uint16_t** h, uint16_t** l, int64_t* chunk, int* split_cap) {
  Carve cv(base);
  const bool quant = flags & LRC_COV_QUANT_INT8_TOKEN;
  int64_t nb = n;
  if (quant) nb = std::min<int64_t>(n, QAW_CHUNK);
  size_t pf = 0;
  int nt = 0, cap = 1;
  if (dt == LRC_BF16 || quant) {
    // launches see token blocks of nb tokens and, for QAW, one final block of n % nb
    SyrkPlan p = plan_syrk(std::max<int64_t>(nb, 1), d);
    cap = p.splits;
    if (quant && n % nb) cap = std::max(cap, plan_syrk(n % nb, d).splits);
    p.splits = cap;
    pf = syrk_partial_floats(p);
    nt = p.n_tiles;
  }
  float* pp = cv.take<float>(pf);
  unsigned* cc = cv.take<unsigned>(size_t(std::max(nt, 1)));
  uint16_t *qq = nullptr, *hh = nullptr, *ll = nullptr;
  if (quant) {
    qq = cv.take<uint16_t>(size_t(nb) * d);
    hh = cv.take<uint16_t>(size_t(nb) * d);
    ll = cv.take<uint16_t>(size_t(nb) * d);
  }
  if (partial) *partial = pp;
  if (counters) *counters = cc;
  if (q) *q = qq;
  if (h) *h = hh;
  if (l) *l = ll;
  if (chunk) *chunk = nb;
  if (split_cap) *split_cap = cap;
  return cv.bytes();
}

}  // namespace
}  // namespace lrc

using namespace lrc;

extern "C" size_t lrc_accumulate_cov_workspace(lrc_dtype dt, int64_t n_tokens, int64_t d, uint32_t flags) {
  if (n_tokens < 0 || d <= 0) return 0;
  return cov_workspace(dt, n_tokens, d, flags, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
}

extern "C" lrc_status lrc_accumulate_cov(const void* A, lrc_dtype dt, int64_t n_tokens, int64_t d, int64_t lda,
                                         float* C, int64_t ldc, uint32_t flags, void* ws, size_t ws_bytes,
                                         void* stream) {
  if (dt != LRC_F32 && dt != LRC_BF16) return LRC_EDTYPE;
  if (flags & ~uint32_t(LRC_COV_QUANT_INT8_TOKEN)) return LRC_EDTYPE;
  if (n_tokens < 0 || d <= 0 || d > (int64_t(1) << 30) || lda < d || ldc < d) return LRC_EINVAL;
  if (C == nullptr) return LRC_EINVAL;
  if (n_tokens == 0) return LRC_OK;
  if (A == nullptr) return LRC_EINVAL;
  const size_t need = lrc_accumulate_cov_workspace(dt, n_tokens, d, flags);
  if (ws_bytes < need || (need > 0 && ws == nullptr)) return LRC_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);

  float* partial = nullptr;
  unsigned* counters = nullptr;
  uint16_t *q = nullptr, *h = nullptr, *l = nullptr;
  int64_t chunk = 0;
  int cap = 1;
  cov_workspace(dt, n_tokens, d, flags, ws, &partial, &counters, &q, &h, &l, &chunk, &cap);
  const bool quant = flags & LRC_COV_QUANT_INT8_TOKEN;
  const int n1 = int(cdiv(d, TB));
  const int nt = n1 * (n1 + 1) / 2;

  if (!quant && dt == LRC_F32) {
    const int tiles = int(cdiv(d, 64) * (cdiv(d, 64) + 1) / 2);
    const double tri = double(d) * double(d + 1) / 2;
    ProfScope scope("syrk_f32_kernel", st, 2.0 * double(n_tokens) * tri, double(n_tokens) * double(d) * 4.0 + 8.0 * tri);
    syrk_f32_kernel<<<tiles, 256, 0, st>>>(static_cast<const float*>(A), lda, n_tokens, int(d), C, ldc);
    LRC_LAUNCHED();
    return LRC_OK;
  }
  zero_u32_kernel<<<unsigned(cdiv(nt, 256)), 256, 0, st>>>(counters, nt);
  LRC_LAUNCHED();
  if (!quant) {
    const uint16_t* a = static_cast<const uint16_t*>(A);
    return launch_syrk_bf16(st, a, a, lda, n_tokens, d, C, ldc, partial, counters, cap);
  }
  for (int64_t t0 = 0; t0 < n_tokens; t0 += chunk) {
    const int64_t nb = std::min(chunk, n_tokens - t0);
    {
    ProfScope scope("qaw_prepass_kernel", st, 0.0, double(nb) * double(d) * ((dt == LRC_BF16 ? 2 : 4) + 6));
    if (dt == LRC_BF16)
      qaw_prepass_kernel<uint16_t><<<unsigned(nb), 256, 0, st>>>(static_cast<const uint16_t*>(A) + t0 * lda, lda,
                                                                 int(d), q, h, l, d);
    else
      qaw_prepass_kernel<float><<<unsigned(nb), 256, 0, st>>>(static_cast<const float*>(A) + t0 * lda, lda,
                                                              int(d), q, h, l, d);
    LRC_LAUNCHED();
    }
    LRC_TRY(launch_syrk_bf16(st, q, h, d, nb, d, C, ldc, partial, counters, cap));
    LRC_TRY(launch_syrk_bf16(st, q, l, d, nb, d, C, ldc, partial, counters, cap));
  }
  return LRC_OK;
}
