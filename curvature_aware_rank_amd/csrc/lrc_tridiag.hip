// Symmetric eigensolver for one large Gram of the whitened weight (Swift-SVD technical
// summary 2A: the decomposition is one eigendecomposition of the aggregated output
// covariance), fp64 throughout:
//
//   1. Householder tridiagonalisation Q^T C Q = T, blocked in 32-column panels with the
//      rank-2 updates of a panel deferred (each column is brought up to date when it is
//      reached; the trailing matrix gets one rank-64 update per panel).  Per column:
//        - symv kernel: y = C_trailing v over 64 x 64 lower tiles (every tile adds its
//          row sums and, off the diagonal, its column sums to per-tile partials), plus the
//          panel products V^T v and W^T v and v^T C v;
//        - w kernel: reduces the partials, w = tau (y - W V^T v - V W^T v) + alpha v
//          with alpha = -tau/2 (w^T v), stores v and w, and brings the next column up to
//          date with the panel so far (its squared norm goes to per-block partials).
//      The reflector of column i (v[i+1] = 1) is stored in column i below the diagonal.
//   2. All eigenvalues of T by Sturm-count multisection (16 points per step, 12 steps).
//   3. Eigenvectors of the wanted (largest) eigenvalues by inverse iteration on T with
//      partial pivoting, two solves (the eigenvalues are accurate to ~eps ||T||): the
//      factorisation and both solves of every vector in parallel; after each solve, per
//      cluster of eigenvalues closer than 1e-9 ||T|| (a lone one is a cluster of one),
//      each iterate is orthogonalised against the cluster's earlier vectors and
//      normalised (one wave per cluster of up to 32 members, modified Gram-Schmidt; a
//      workgroup per longer cluster, block Gram-Schmidt applied twice).  Nothing is read
//      back to the host: the whole solve is enqueued at once.
//   4. Back-transformation Z <- Q Z in blocks of 128 reflectors, I - V T V^T (T from the
//      forward columnwise recurrence on V^T V).
// A batch of Grams goes through every stage together: each launch covers all slices (a
// grid dimension indexes the slice), so the per-step launch and latency costs are paid
// once for the batch.
// Every reduction has a fixed order, so equal inputs give equal bits.
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

#include <hip/hip_ext.h>

#include "lrc_dense.h"

namespace lrc {
namespace {

constexpr int NB = 32;          // tridiagonalisation panel width
constexpr int TS = 64;          // tile and row-block size of the symv / w kernels
constexpr int BW = 128;         // reflectors per back-transformation block
constexpr int BT_CHUNK = 128;   // rows per partial of V^T Z
constexpr int G_CHUNK = 256;    // rows per partial of V^T V
constexpr int WR = 32;          // rows per workgroup of the w kernel (16 or 32; 16 measured no faster)
constexpr int WPB = TS / WR;    // w workgroups per 64-row block
constexpr int NPB = 4 * WPB;    // squared-norm partials per 64-row block (one per w wave)
constexpr int BIS_PTS = 16;     // Sturm points per eigenvalue per multisection step
constexpr int BIS_ITERS = 12;   // 17^12 > 2^49: width below 2^-48 of the bounds, under a count's own n eps accuracy
constexpr int BIS_STAGE = 2048; // d, e^2 staged through LDS in chunks of this many
constexpr int CL_MAX = 32;      // larger clusters are orthogonalised by a whole workgroup
// eigenvalues closer than CL_TOL ||T|| share a cluster.  Bisection leaves an eigenvalue
// within about n eps ||T|| (< 1e-12 ||T|| here), so two inverse iterations reduce a
// neighbour at distance >= CL_TOL ||T|| to (1e-12 / CL_TOL)^2 = 1e-6 of the start vector
// or less: such vectors need no orthogonalisation against each other.  A wider tolerance
// would merge the densely spaced smallest eigenvalues of a whitened Gram (spacing about
// 1e-7 ||T||) into clusters of thousands, whose orthogonalisation is quadratic in size.
constexpr double CL_TOL = 1e-9;
constexpr double EPS = 2.220446049250313e-16;

// first row / column of the 64-row blocks of the trailing matrix that starts at s0: the
// 16-column boundary at or below s0, so that every tile row starts on a 128-byte line
__host__ __device__ __forceinline__ int blk_origin(int s0) { return s0 & ~15; }

__device__ __forceinline__ void tile_of(int t, int& b, int& c) {
  // t = b (b + 1) / 2 + c, 0 <= c <= b
  int bb = int((sqrt(8.0 * double(t) + 1.0) - 1.0) * 0.5);
  while ((bb + 1) * (bb + 2) / 2 <= t) ++bb;
  while (bb * (bb + 1) / 2 > t) --bb;
  b = bb;
  c = t - bb * (bb + 1) / 2;
}

__device__ __forceinline__ void house_from_sum(double xn2, double x0, double& tau, double& beta, double& scale) {
  if (xn2 == 0.0) {
    tau = 0.0;
    beta = x0;
    scale = 0.0;
    return;
  }
  const double nrm = sqrt(x0 * x0 + xn2);
  beta = x0 >= 0.0 ? -nrm : nrm;
  tau = (beta - x0) / beta;
  scale = 1.0 / (x0 - beta);
}

// Cross-lane moves of a double with DPP (register-to-register, no LDS round trip)
template <int CTRL>
__device__ __forceinline__ double dpp_mov(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}
constexpr int DPP_QUAD_XOR1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int DPP_QUAD_XOR2 = 0x4E;   // quad_perm [2, 3, 0, 1]
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_MIRROR = 0x140;

// sum over the 4 lanes of a quad (every lane of the quad gets the same bits)
__device__ __forceinline__ double quad_sum(double v) {
  v += dpp_mov<DPP_QUAD_XOR1>(v);
  v += dpp_mov<DPP_QUAD_XOR2>(v);
  return v;
}

// sum over the 64 lanes of a wave in a fixed order (quads, 8-lane halves, 16-lane rows,
// then the four rows); every lane gets the same bits
__device__ __forceinline__ double wave_sum(double v) {
  v = quad_sum(v);
  v += dpp_mov<DPP_HALF_MIRROR>(v);
  v += dpp_mov<DPP_MIRROR>(v);
  auto lane_val = [&](int l) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                            __builtin_amdgcn_readlane(__double2loint(v), l));
  };
  return (lane_val(0) + lane_val(16)) + (lane_val(32) + lane_val(48));
}

// block-wide sum of one value per thread (256 threads), fixed tree; result to all
__device__ __forceinline__ double block_sum256(double v, double* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

// ---- 1a. first column of a panel: d[i], x0, squared-norm partials (no deferred updates;
// NPB partials per 64-row block, as the w kernel writes them: the block's sum, then zeros)
// and the column as a contiguous vector xv[r] (rows i .. n - 1) for the symv kernel
__global__ __launch_bounds__(256) void tri_colstart_kernel(const double* __restrict__ A, int64_t lda, int n, int i,
                                                           double* __restrict__ npart, double* __restrict__ x0,
                                                           double* __restrict__ d, double* __restrict__ xv, int64_t sA,
                                                           int64_t wsi) {
  __shared__ double red[256];
  {   // slice blockIdx.y of a batch: its matrix and its block of loop arrays
    const int64_t it = blockIdx.y;
    A += it * sA;
    npart += it * wsi;
    x0 += it * wsi;
    d += it * wsi;
    xv += it * wsi;
  }
  const int tid = threadIdx.x;
  const int r = i + blockIdx.x * TS + tid;
  double sq = 0.0;
  if (tid < TS && r < n) {
    const double val = A[int64_t(r) * lda + i];
    xv[r] = val;
    if (r == i) d[i] = val;
    if (r == i + 1) *x0 = val;
    if (r >= i + 2) sq = val * val;
  }
  const double s = block_sum256(sq, red);
  if (tid < NPB) npart[NPB * blockIdx.x + tid] = tid == 0 ? s : 0.0;
}

// ---- 1b. symv over the trailing matrix (rows/cols i+1 .. n-1) with the raw column
// x = C[i+1:, i] (the reflector is v = scale x + (1 - scale x0) e_{i+1}; the w kernel
// applies that), one 64 x 64 lower tile per workgroup.  Outputs: P[x][y][*], the
// contribution to y-block x from the tile pairing x and y; S[t] = tile part of x^T C x;
// on diagonal tiles the panel products V^T x, W^T x over the block's rows.  x is read from
// the contiguous copy xv of column i (rows i + 1 ..) that the previous kernel wrote.
// Each thread holds a 4 x 4 patch of the tile in registers (rows 4 rb .., columns 4 cb ..,
// rb = tid / 16, cb = tid % 16), loaded as 16-byte pairs (EVEN: the tile's first column is
// even; otherwise three pairs per row, of which the middle four values are used).  Row
// sums reduce over the 16 lanes of a DPP row by a transposing butterfly; column partials
// go through a 16 x 64 LDS table and are added in row-band order.
constexpr int DPP_ROW_ROR8 = 0x128;   // row_ror:8, lane i <-> i + 8 within 16 lanes

__global__ __launch_bounds__(256) void tri_symv_kernel(const double* __restrict__ A, int64_t lda, int n, int i, int i0,
                                                       int jj, const double* __restrict__ Wp,
                                                       const double* __restrict__ xv, double* __restrict__ P,
                                                       double* __restrict__ S, double* __restrict__ SV,
                                                       double* __restrict__ SW, int64_t sA, int64_t wsi) {
  {   // slice blockIdx.y of a batch
    const int64_t it = blockIdx.y;
    A += it * sA;
    Wp += it * wsi;
    xv += it * wsi;
    P += it * wsi;
    S += it * wsi;
    SV += it * wsi;
    SW += it * wsi;
  }
  __shared__ double rsum[TS];
  __shared__ double cpart[16][TS + 1];
  __shared__ double red[8][2][NB];
  const int tid = threadIdx.x;
  const int s0 = i + 1;
  const int so = blk_origin(s0);   // blocks start at a 16-column boundary
  const int nbt = (n - so + TS - 1) / TS;
  const int ntile = nbt * (nbt + 1) / 2;
  if (int(blockIdx.x) >= ntile) {
    // panel workgroup for row block pb: V^T x and W^T x over the block's 64 rows, 32
    // columns x 8 groups of 8 rows, summed over the groups in order
    const int pb = blockIdx.x - ntile;
    const int R0 = so + pb * TS;
    const int pc = tid & 31, pg = tid >> 5;
    const int pcc = min(pc, jj - 1);
    double va[8], wa[8], xa[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int r = min(R0 + pg * 8 + q, n - 1);
      va[q] = A[int64_t(r) * lda + i0 + pcc];
      wa[q] = Wp[int64_t(r) * NB + pcc];
      xa[q] = xv[r];
    }
    double sv = 0.0, sw = 0.0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int r = R0 + pg * 8 + q;
      const bool ok = pc < jj && r >= s0 && r < n;
      sv += ok ? va[q] * xa[q] : 0.0;
      sw += ok ? wa[q] * xa[q] : 0.0;
    }
    red[pg][0][pc] = sv;
    red[pg][1][pc] = sw;
    __syncthreads();
    if (tid < jj) {
      double a0 = 0.0, a1 = 0.0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        a0 += red[q][0][tid];
        a1 += red[q][1][tid];
      }
      SV[pb * NB + tid] = a0;
      SW[pb * NB + tid] = a1;
    }
    return;
  }
  int b, c;
  tile_of(blockIdx.x, b, c);
  const int R0 = so + b * TS, C0 = so + c * TS;
  const bool diag = b == c;
  const int rb = tid >> 4, cb = tid & 15;
  const int c4 = C0 + 4 * cb;
  // every load is unconditional from a clamped address and masked at use: the tile's
  // columns start at a 16-column boundary, so every 4-column patch row is two 16-byte
  // pairs at even columns, at most at pe, the last even column; for odd n the pair
  // (n - 1, n) reads one element of the row padding (the pitch is even and exceeds n).
  // Entries left of s0 (and above it) are read and masked.
  const int pe = (n - 1) & ~1;
  double tv[4][4];
  {
    const int p0 = min(c4, pe), p1 = min(c4 + 2, pe);
    double2 u[4][2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = min(R0 + 4 * rb + k, n - 1);
      u[k][0] = *reinterpret_cast<const double2*>(A + int64_t(r) * lda + p0);
      u[k][1] = *reinterpret_cast<const double2*>(A + int64_t(r) * lda + p1);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      tv[k][0] = u[k][0].x;
      tv[k][1] = u[k][0].y;
      tv[k][2] = u[k][1].x;
      tv[k][3] = u[k][1].y;
    }
  }
  // x on the patch's columns (vcl) and rows (vbl), masked with the tile below
  double vcl[4], vbl[4];
  const int rr4 = R0 + 4 * rb;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    vcl[e] = xv[min(c4 + e, n - 1)];
    vbl[e] = xv[min(rr4 + e, n - 1)];
  }
  double xe = 0.0;   // x on row R0 + tid (x^T C x epilogue)
  if (tid < TS) xe = xv[min(R0 + tid, n - 1)];
  // row sums over the tile's lower part incl. the diagonal; column sums strictly below it
  double rp[4] = {0.0, 0.0, 0.0, 0.0}, cp[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int row = 4 * rb + k;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int col = 4 * cb + e;
      const bool in = R0 + row >= s0 && R0 + row < n && C0 + col >= s0 && C0 + col < n;
      const bool okr = in && (!diag || col <= row);
      const bool okc = in && (!diag || col < row);
      rp[k] += okr ? tv[k][e] * vcl[e] : 0.0;
      cp[e] += okc ? tv[k][e] * vbl[k] : 0.0;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) cpart[rb][4 * cb + e] = cp[e];
  {
    // four row values over 16 lanes: exchange halves with the lane 8 away, then with the
    // mirrored lane of the 8-lane half, then sum the quad; row 4 rb + 2 b3 + b2 results
    const bool h = cb & 8;
    const double s0v = h ? rp[0] : rp[2], s1v = h ? rp[1] : rp[3];
    const double k0v = h ? rp[2] : rp[0], k1v = h ? rp[3] : rp[1];
    const double a0 = k0v + dpp_mov<DPP_ROW_ROR8>(s0v);
    const double a1 = k1v + dpp_mov<DPP_ROW_ROR8>(s1v);
    const bool h2 = cb & 4;
    const double sv = h2 ? a0 : a1, kv = h2 ? a1 : a0;
    const double r = quad_sum(kv + dpp_mov<DPP_HALF_MIRROR>(sv));
    if ((cb & 3) == 0) rsum[4 * rb + 2 * ((cb >> 3) & 1) + ((cb >> 2) & 1)] = r;
  }
  __syncthreads();
  if (tid < TS) {
    double c_ = 0.0;
#pragma unroll
    for (int q = 0; q < 16; ++q) c_ += cpart[q][tid];
    const double r_ = rsum[tid];
    const double xb = R0 + tid >= s0 && R0 + tid < n ? xe : 0.0;
    if (diag) {
      P[(int64_t(b) * nbt + b) * TS + tid] = r_ + c_;
    } else {
      P[(int64_t(b) * nbt + c) * TS + tid] = r_;
      P[(int64_t(c) * nbt + b) * TS + tid] = c_;
    }
    // x_b^T (tile contribution), fixed butterfly over the first wave
    const double sacc = wave_sum(diag ? xb * (r_ + c_) : 2.0 * (xb * r_));
    if (tid == 0) S[blockIdx.x] = sacc;
  }
}

// ---- 1c. for WR rows of the trailing rows (TS / WR workgroups per 64-row block): the
// Householder scalars of column i, v = scale x + c e_{s0} (c = 1 - scale x0),
// C v = scale (C x) + c C e_{s0},
// w = tau (C v - W V^T v - V W^T v) + alpha v with alpha = -tau^2/2 (v^T C v - 2 (V^T v).(W^T v));
// store v (column i) and w (column jj of W); then bring column s0 up to date with the
// panel's reflectors 0..jj (if it is in the panel) and write its squared-norm partials
// (one per wave: WR / 4 rows each, NPB per 64-row block).
// Every global load is issued in one phase, from clamped addresses and masked after: the
// rows' symv partials, the panel partials and the rows' panel entries as 16-byte pairs
// along contiguous rows, columns i and s0 once per row (one pair when i is even).  Half a
// block per workgroup halves the per-workgroup bytes that are not shared by all of them
// (the load phase is bound by what one CU can fetch) and the per-row work per thread;
// a quarter block measured no faster (the bytes every workgroup needs then dominate).
// sum over the 8 lanes of an aligned octet (every lane of the octet gets the same bits)
__device__ __forceinline__ double oct_sum(double v) {
  v = quad_sum(v);
  return v + dpp_mov<DPP_HALF_MIRROR>(v);
}
// sum over the TPR (8 or 16) lanes of an aligned group
template <int TPR>
__device__ __forceinline__ double group_sum(double v) {
  v = oct_sum(v);
  if constexpr (TPR == 16) v += dpp_mov<DPP_MIRROR>(v);
  return v;
}

template <bool EVEN>
__global__ __launch_bounds__(256) void tri_w_kernel(double* __restrict__ A, int64_t lda, int n, int i, int i0, int jj,
                                                    int do_next, double* __restrict__ Wp,
                                                    const double* __restrict__ npart, const double* __restrict__ x0p,
                                                    const double* __restrict__ P, const double* __restrict__ S,
                                                    const double* __restrict__ SV, const double* __restrict__ SW,
                                                    double* __restrict__ npart_next, double* __restrict__ x0_next,
                                                    double* __restrict__ d, double* __restrict__ e,
                                                    double* __restrict__ tau_out, double* __restrict__ xv_next,
                                                    int64_t sA, int64_t wsi) {
  {   // slice blockIdx.y of a batch
    const int64_t it = blockIdx.y;
    A += it * sA;
    Wp += it * wsi;
    npart += it * wsi;
    x0p += it * wsi;
    P += it * wsi;
    S += it * wsi;
    SV += it * wsi;
    SW += it * wsi;
    npart_next += it * wsi;
    x0_next += it * wsi;
    d += it * wsi;
    e += it * wsi;
    tau_out += it * wsi;
    xv_next += it * wsi;
  }
  constexpr int RPAIRS = WR / 2;       // row pairs of the symv partials
  constexpr int NCG = 256 / RPAIRS;    // column-block groups (16 or 32)
  constexpr int NPU = TS / NCG;        // column blocks per group below 64 blocks
  constexpr int TPR = 256 / WR;        // threads per row in the row stage (8 or 16)
  constexpr int NRU = WR / 16;         // panel row groups of 16
  static_assert(WR == 16 || WR == 32, "16 or 32 rows per workgroup");
  __shared__ double Vs[WR][NB + 1], Ws[WR][NB + 1];
  __shared__ double yp[NCG][WR];
  __shared__ double svq[16][NB], swq[16][NB];
  __shared__ double vn[NB], wn[NB];
  __shared__ double svw[4][NB], sww[4][NB];   // per-wave copies of V^T v, W^T v
  __shared__ double colI[WR], colS[WR];
  __shared__ double red[3][4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int s0 = i + 1;
  const int so = blk_origin(s0);   // the symv's block origin
  const int nbt = (n - so + TS - 1) / TS;
  const int ntile = nbt * (nbt + 1) / 2;
  const int npp = NPB * ((n - blk_origin(i) + TS - 1) / TS);   // partials written for column i
  const int b = blockIdx.x / WPB, h = blockIdx.x % WPB;
  const int lr0 = h * WR;        // first row of this workgroup within its 64-row block
  const int R0 = so + b * TS + lr0;
  const int xp = tid % RPAIRS, cg = tid / RPAIRS;   // symv partials: row pair 2 xp, column blocks cg + NCG u
  const int cq = tid & 15, qg = tid >> 4;   // panel: column pair 2 cq, row (block) group qg + 16 u
  // panel column pair start, never past column i0 + jj = i
  const int pcs = max(min(2 * cq, (jj - 1) & ~1), 0);

  // ---- load phase
  double2 pp[NPU], svl[4], swl[4], pv[NRU], pw[NRU];
#pragma unroll
  for (int u = 0; u < NPU; ++u)
    pp[u] = *reinterpret_cast<const double2*>(P + (int64_t(b) * nbt + min(cg + NCG * u, nbt - 1)) * TS + lr0 + 2 * xp);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int q = min(qg + 16 * u, nbt - 1);
    svl[u] = *reinterpret_cast<const double2*>(SV + q * NB + pcs);
    swl[u] = *reinterpret_cast<const double2*>(SW + q * NB + pcs);
  }
#pragma unroll
  for (int u = 0; u < NRU; ++u) {
    const int r = min(R0 + qg + 16 * u, n - 1);
    pv[u] = *reinterpret_cast<const double2*>(A + int64_t(r) * lda + i0 + pcs);
    pw[u] = *reinterpret_cast<const double2*>(Wp + int64_t(r) * NB + pcs);
  }
  double2 vnl = make_double2(0.0, 0.0), wnl = make_double2(0.0, 0.0);
  if (tid < 16) {
    vnl = *reinterpret_cast<const double2*>(A + int64_t(s0) * lda + i0 + pcs);
    wnl = *reinterpret_cast<const double2*>(Wp + int64_t(s0) * NB + pcs);
  }
  double ci = 0.0, cs0 = 0.0;
  if (tid < WR) {
    const int r = min(R0 + tid, n - 1);
    if (EVEN) {
      const double2 t2 = *reinterpret_cast<const double2*>(A + int64_t(r) * lda + i);
      ci = t2.x;
      cs0 = t2.y;
    } else {
      ci = A[int64_t(r) * lda + i];
      cs0 = A[int64_t(r) * lda + s0];
    }
  }
  double ts[9];
#pragma unroll
  for (int u = 0; u < 9; ++u) ts[u] = S[min(tid + 256 * u, ntile - 1)];
  const double tnp0 = npart[min(tid, npp - 1)];
  const double tnp1 = npart[min(tid + 256, npp - 1)];
  const double tp0 = P[int64_t(min(tid, nbt - 1)) * TS + (s0 - so)];   // row s0: block 0, local s0 - so
  const double x0v = *x0p;
  const double a00 = A[int64_t(s0) * lda + s0];

  // ---- partial sums to LDS (fixed order: sequential within a lane), block sums by wave
  {
    double ya = 0.0, yb = 0.0;
#pragma unroll
    for (int u = 0; u < NPU; ++u) {
      const bool ok = cg + NCG * u < nbt;
      ya += ok ? pp[u].x : 0.0;
      yb += ok ? pp[u].y : 0.0;
    }
    for (int c = cg + 64; c < nbt; c += NCG) {   // more than 64 row blocks
      const double2 t2 = *reinterpret_cast<const double2*>(P + (int64_t(b) * nbt + c) * TS + lr0 + 2 * xp);
      ya += t2.x;
      yb += t2.y;
    }
    yp[cg][2 * xp] = ya;
    yp[cg][2 * xp + 1] = yb;
  }
  {
    double a0 = 0.0, a1 = 0.0, b0 = 0.0, b1 = 0.0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool ok = qg + 16 * u < nbt;
      a0 += ok ? svl[u].x : 0.0;
      a1 += ok ? svl[u].y : 0.0;
      b0 += ok ? swl[u].x : 0.0;
      b1 += ok ? swl[u].y : 0.0;
    }
    for (int q = qg + 64; q < nbt; q += 16) {
      const double2 t1 = *reinterpret_cast<const double2*>(SV + q * NB + pcs);
      const double2 t2 = *reinterpret_cast<const double2*>(SW + q * NB + pcs);
      a0 += t1.x;
      a1 += t1.y;
      b0 += t2.x;
      b1 += t2.y;
    }
    svq[qg][2 * cq] = a0;
    svq[qg][2 * cq + 1] = a1;
    swq[qg][2 * cq] = b0;
    swq[qg][2 * cq + 1] = b1;
  }
#pragma unroll
  for (int u = 0; u < NRU; ++u) {
    const int rr = qg + 16 * u;
    const bool okr = R0 + rr >= s0 && R0 + rr < n;
    Vs[rr][2 * cq] = okr && 2 * cq < jj ? pv[u].x : 0.0;
    Vs[rr][2 * cq + 1] = okr && 2 * cq + 1 < jj ? pv[u].y : 0.0;
    Ws[rr][2 * cq] = okr && 2 * cq < jj ? pw[u].x : 0.0;
    Ws[rr][2 * cq + 1] = okr && 2 * cq + 1 < jj ? pw[u].y : 0.0;
  }
  if (tid < 16) {
    vn[2 * tid] = 2 * tid < jj ? vnl.x : 0.0;
    vn[2 * tid + 1] = 2 * tid + 1 < jj ? vnl.y : 0.0;
    wn[2 * tid] = 2 * tid < jj ? wnl.x : 0.0;
    wn[2 * tid + 1] = 2 * tid + 1 < jj ? wnl.y : 0.0;
  }
  if (tid < WR) {
    const bool ok = R0 + tid >= s0 && R0 + tid < n;
    colI[tid] = ok ? ci : 0.0;
    colS[tid] = ok ? cs0 : 0.0;
  }
  {
    double v0 = (tid < npp ? tnp0 : 0.0) + (tid + 256 < npp ? tnp1 : 0.0);
    for (int t = tid + 512; t < npp; t += 256) v0 += npart[t];
    double v1 = 0.0;
#pragma unroll
    for (int u = 0; u < 9; ++u) v1 += tid + 256 * u < ntile ? ts[u] : 0.0;
    for (int t = tid + 256 * 9; t < ntile; t += 256) v1 += S[t];
    double y0 = tid < nbt ? tp0 : 0.0;
    for (int c = tid + 256; c < nbt; c += 256) y0 += P[int64_t(c) * TS + (s0 - so)];
    v0 = wave_sum(v0);
    v1 = wave_sum(v1);
    y0 = wave_sum(y0);
    if (lane == 0) {
      red[0][wv] = v0;
      red[1][wv] = v1;
      red[2][wv] = y0;
    }
  }
  __syncthreads();
  const double xn2 = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
  double tau, beta, scale;
  house_from_sum(xn2, x0v, tau, beta, scale);
  const double cfac = 1.0 - scale * x0v;
  if (blockIdx.x == 0 && tid == 0) {
    e[i] = beta;
    tau_out[i] = tau;
  }
  // every wave derives the scalars itself (no second block barrier): lanes c < jj form
  // V^T v and W^T v, the wave's own LDS copy serves its rows below; then (V^T v).(W^T v)
  // and row s0's correction by butterflies
  double svc = 0.0, swc = 0.0;
  if (lane < jj) {
    double b0 = 0.0, b1 = 0.0;
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      b0 += svq[g][lane];
      b1 += swq[g][lane];
    }
    svc = scale * b0 + cfac * vn[lane];
    swc = scale * b1 + cfac * wn[lane];
  }
  if (lane < NB) {
    svw[wv][lane] = svc;
    sww[wv][lane] = swc;
  }
  const double dsw = wave_sum(svc * swc);
  const double corr0 = wave_sum(lane < jj ? wn[lane] * svc + vn[lane] * swc : 0.0);
  const double v1 = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  const double y0raw = (red[2][0] + red[2][1]) + (red[2][2] + red[2][3]);
  const double y0 = scale * y0raw + cfac * a00;
  const double vav = scale * scale * v1 + 2.0 * scale * cfac * y0raw + cfac * cfac * a00;
  const double alpha = -0.5 * tau * tau * (vav - 2.0 * dsw);
  const double w0 = tau * (y0 - corr0) + alpha;   // w of row s0 (v = 1 there)
  // the wave's LDS copy is read by other lanes of the same wave only
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // rows x = tid / TPR (a wave's rows only): the row's TPR lanes split the panel columns
  // (c = part + TPR k) and the row-sum groups (2 part, 2 part + 1)
  const int x = tid / TPR, part = tid % TPR;
  const int r = R0 + x;
  double corr = 0.0, c2 = 0.0;
#pragma unroll
  for (int k = 0; k < NB / TPR; ++k) {   // columns c >= jj hold zeros in every operand
    const int c = part + TPR * k;
    const double vr = Vs[x][c], wr = Ws[x][c];
    corr += wr * svw[wv][c] + vr * sww[wv][c];
    c2 += vr * wn[c] + wr * vn[c];
  }
  double yr = yp[2 * part][x] + yp[2 * part + 1][x];
  corr = group_sum<TPR>(corr);
  c2 = group_sum<TPR>(c2);
  yr = group_sum<TPR>(yr);
  double v = 0.0, w = 0.0;
  const double cs0x = colS[x];
  if (r >= s0 && r < n) {
    const double y = scale * yr + cfac * cs0x - corr;
    v = r == s0 ? 1.0 : colI[x] * scale;
    w = r == s0 ? w0 : tau * y + alpha * v;   // row s0: the value every block uses
    if (part == 0) {
      Wp[int64_t(r) * NB + jj] = w;
      A[int64_t(r) * lda + i] = v;
    }
  }
  if (!do_next) return;
  // column s0: rows s0.., C[r][s0] -= sum_c V[r][c] W[s0][c] + W[r][c] V[s0][c], c = 0..jj.
  // The diagonal entry goes to d[s0] only: every workgroup of this launch reads the
  // panel-start C[s0][s0] (a00 above), so it must not be overwritten here (a workgroup
  // that starts after this one has finished would read the updated value); nothing reads
  // it later (the next columns' trailing matrices start below and right of it).
  double sq = 0.0;
  if (r >= s0 && r < n && part == 0) {
    const double val = cs0x - (c2 + (v * w0 + w));
    if (r > s0) A[int64_t(r) * lda + s0] = val;
    xv_next[r] = val;
    if (r == s0) d[s0] = val;
    if (r == s0 + 1) *x0_next = val;
    if (r >= s0 + 2) sq = val * val;
  }
  sq = wave_sum(sq);
  if (lane == 0) npart_next[NPB * b + 4 * h + wv] = sq;
}

// ---- 1d. trailing rank-2 panel update, lower tiles of rows/cols j1 .. n-1:
// C -= V W^T + W V^T  (V rows in C's panel columns i0 .. i0+pb-1), as one product of
// K = 2 NB on fp64 MFMA: [V_r | W_r] [W_c | V_c]^T.  One 64 x 64 tile per workgroup, four
// waves of 32 x 32; the tile's old values are loaded at the start, with the operands.
constexpr int SYP = 64 + 2;   // LDS pitch (doubles) of an operand k row

__global__ __launch_bounds__(256) void tri_syr2k_kernel(double* __restrict__ A, int64_t lda, int n, int i0, int pb,
                                                        int j1, const double* __restrict__ Wp,
                                                        double* __restrict__ npart, double* __restrict__ x0,
                                                        double* __restrict__ d, double* __restrict__ xv, int64_t sA,
                                                        int64_t wsi) {
  {   // slice blockIdx.y of a batch
    const int64_t it = blockIdx.y;
    A += it * sA;
    Wp += it * wsi;
    npart += it * wsi;
    x0 += it * wsi;
    d += it * wsi;
    xv += it * wsi;
  }
  // the K = 64 product in two halves through one LDS pair (V_r W_c^T, then W_r V_c^T), so
  // that four workgroups fit on a CU
  __shared__ double opa[NB][SYP], opb[NB][SYP];
  __shared__ double sqp[8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int l16 = lane & 15, lq = lane >> 4;
  int b, c;
  tile_of(blockIdx.x, b, c);
  const int R0 = j1 + b * TS, C0 = j1 + c * TS;
  // old tile values this thread updates (fp64 16 x 16 output: lane l, element e -> row
  // l / 16 + 4 e, column l % 16)
  double old[2][2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = min(R0 + wr * 32 + i * 16 + lq + 4 * e, n - 1);
        const int cc = min(C0 + wc * 32 + j * 16 + l16, n - 1);
        old[i][j][e] = A[int64_t(r) * lda + cc];
      }
  // operands: thread takes row x = tid / 4 and panel columns (tid % 4) * 8 .. + 7 as four
  // 16-byte pairs (the panel starts at an even column; pairs past pb are masked below)
  const int x = tid >> 2, t0 = (tid & 3) * 8;
  double2 vr[4], wr8[4], vc[4], wc8[4];
  {
    const int r = min(R0 + x, n - 1), cc = min(C0 + x, n - 1);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int tc = min(t0 + 2 * u, (pb - 1) & ~1);
      vr[u] = *reinterpret_cast<const double2*>(A + int64_t(r) * lda + i0 + tc);
      wr8[u] = *reinterpret_cast<const double2*>(Wp + int64_t(r) * NB + tc);
      vc[u] = *reinterpret_cast<const double2*>(A + int64_t(cc) * lda + i0 + tc);
      wc8[u] = *reinterpret_cast<const double2*>(Wp + int64_t(cc) * NB + tc);
    }
  }
  const bool okr = R0 + x < n, okc = C0 + x < n;
  auto stage = [&](const double2 (&ra)[4], bool oka, const double2 (&rb)[4], bool okb) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool ok0 = t0 + 2 * u < pb, ok1 = t0 + 2 * u + 1 < pb;
      opa[t0 + 2 * u][x] = oka && ok0 ? ra[u].x : 0.0;
      opa[t0 + 2 * u + 1][x] = oka && ok1 ? ra[u].y : 0.0;
      opb[t0 + 2 * u][x] = okb && ok0 ? rb[u].x : 0.0;
      opb[t0 + 2 * u + 1][x] = okb && ok1 ? rb[u].y : 0.0;
    }
  };
  f64x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
  auto mma = [&]() {
#pragma unroll
    for (int kk = 0; kk < NB; kk += 4) {
      double a[2], bb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = opa[kk + lq][wr * 32 + i * 16 + l16];
#pragma unroll
      for (int j = 0; j < 2; ++j) bb[j] = opb[kk + lq][wc * 32 + j * 16 + l16];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], bb[j], acc[i][j], 0, 0, 0);
    }
  };
  stage(vr, okr, wc8, okc);   // V_r W_c^T
  __syncthreads();
  mma();
  __syncthreads();
  stage(wr8, okr, vc, okc);   // W_r V_c^T
  __syncthreads();
  mma();
  // Tiles of the first column block also start the next panel (what the column-start
  // kernel does for the first panel): column j1, now up to date, as the contiguous vector
  // xv, d[j1], x0 = A[j1 + 1][j1] and the block's squared-norm partial over rows >= j1 + 2
  // (NPB partials per 64-row block: the sum, then zeros).  Its values sit in lanes
  // l16 = 0 of the waves with wc = 0 (j = 0), rows wr 32 + i 16 + lq + 4 e.
  double sq = 0.0;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int lr = wr * 32 + i * 16 + lq + 4 * e, lc = wc * 32 + j * 16 + l16;
        const int r = R0 + lr, cc = C0 + lc;
        const double val = old[i][j][e] - acc[i][j][e];
        if (r < n && cc < n && (b != c || lr >= lc)) A[int64_t(r) * lda + cc] = val;
        if (c == 0 && lc == 0 && r < n) {
          xv[r] = val;
          if (r == j1) d[j1] = val;
          if (r == j1 + 1) *x0 = val;
          if (r >= j1 + 2) sq += val * val;
        }
      }
  if (c == 0) {
    // lanes 0, 16, 32, 48 of waves 0 and 2 hold partial sums; fixed-order total
    if (wc == 0 && l16 == 0) sqp[wr * 4 + lq] = sq;
    __syncthreads();
    if (tid < NPB) npart[NPB * b + tid] = tid == 0 ? ((sqp[0] + sqp[1]) + (sqp[2] + sqp[3])) +
                                                        ((sqp[4] + sqp[5]) + (sqp[6] + sqp[7]))
                                                  : 0.0;
  }
}


// ---- 1e. the last columns (trailing matrix of at most TT rows, already fully updated at
// a panel boundary) in one workgroup: the whole trailing matrix lives in LDS (full
// symmetric storage), and each column is reduced unblocked, H A H = A - v w^T - w v^T with
// w = tau A v - tau^2/2 (v^T A v) v.  Writes the same d, e, tau and reflectors (column i
// below the diagonal, v[i+1] = 1) as the panel path; one launch instead of two per column.
constexpr int TT = 128;          // rows of the trailing matrix handled this way
constexpr int TTP = TT + 1;      // LDS pitch (doubles)

__device__ __forceinline__ double block_sum4w(double v, double* red) {
  // sum over 256 threads: wave butterflies, then the four wave results in order
  v = wave_sum(v);
  __syncthreads();   // red may still be read from the previous call
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void tri_tail_kernel(double* __restrict__ A, int64_t lda, int n, int t0,
                                                       double* __restrict__ d, double* __restrict__ e,
                                                       double* __restrict__ tau_out, int64_t sA, int64_t wsi) {
  {   // slice blockIdx.y of a batch
    const int64_t it = blockIdx.y;
    A += it * sA;
    d += it * wsi;
    e += it * wsi;
    tau_out += it * wsi;
  }
  __shared__ double T[TT][TTP];
  __shared__ double vv[TT], yy[TT];
  __shared__ double red[4];
  const int tid = threadIdx.x;
  const int nt = n - t0;   // <= TT
  // load the lower triangle of the trailing matrix and mirror it
  for (int q = tid; q < nt * nt; q += 256) {
    const int r = q / nt, c = q % nt;
    if (c <= r) {
      const double val = A[int64_t(t0 + r) * lda + t0 + c];
      T[r][c] = val;
      T[c][r] = val;
    }
  }
  __syncthreads();
  for (int li = 0; li < nt - 1; ++li) {
    const int i = t0 + li;
    const int m = nt - 1 - li;   // length of the column below the diagonal
    const int b0 = li + 1;       // first trailing row / column
    // reflector of column li: x = T[b0.., li]
    const double x0 = T[b0][li];
    double sq = 0.0;
    for (int r = tid + 1; r < m; r += 256) sq += T[b0 + r][li] * T[b0 + r][li];
    const double xn2 = block_sum4w(sq, red);
    double tau, beta, scale;
    house_from_sum(xn2, x0, tau, beta, scale);
    if (tid == 0) {
      d[i] = T[li][li];
      e[i] = beta;
      tau_out[i] = tau;
    }
    for (int r = tid; r < m; r += 256) {
      const double v = r == 0 ? 1.0 : T[b0 + r][li] * scale;
      vv[r] = v;
      A[int64_t(b0 + t0 + r) * lda + i] = v;
    }
    __syncthreads();
    // y = T_trailing v (four threads per row, the quad adding in a fixed order)
    double vy_part = 0.0;
    {
      const int part = tid & 3;
      for (int r0 = tid >> 2; r0 < m; r0 += 64) {
        double acc = 0.0;
        for (int c = part; c < m; c += 4) acc += T[b0 + r0][b0 + c] * vv[c];
        acc = quad_sum(acc);
        if (part == 0) {
          yy[r0] = acc;
          vy_part += acc * vv[r0];
        }
      }
    }
    const double vy = block_sum4w(vy_part, red);   // barrier: also publishes yy
    const double alpha = -0.5 * tau * tau * vy;
    // T_trailing -= v w^T + w v^T, w = tau y + alpha v (16 x 16 threads, strided)
    {
      const int tr = tid >> 4, tc = tid & 15;
      for (int r = tr; r < m; r += 16) {
        const double vr = vv[r], wr = tau * yy[r] + alpha * vr;
        for (int c = tc; c < m; c += 16) {
          const double vc = vv[c], wc = tau * yy[c] + alpha * vc;
          T[b0 + r][b0 + c] -= vr * wc + wr * vc;
        }
      }
    }
    __syncthreads();
  }
  if (tid == 0) d[n - 1] = T[nt - 1][nt - 1];
}

// ---- 2. eigenvalues of T
// bounds: [0] gl, [1] gu, [2] pivmin, [3] ||T|| (max |Gershgorin end|)
__global__ __launch_bounds__(256) void tri_bounds_kernel(const double* __restrict__ d, const double* __restrict__ e,
                                                         int n, double* __restrict__ bounds, int64_t wsi) {
  {   // slice blockIdx.y of a batch: d, e in its loop block, 4 bounds per slice
    const int64_t it = blockIdx.y;
    d += it * wsi;
    e += it * wsi;
    bounds += 4 * it;
  }
  __shared__ double rl[256], rh[256], re[256];
  const int tid = threadIdx.x;
  double lo = 1e300, hi = -1e300, em = 0.0;
  for (int k = tid; k < n; k += 256) {
    const double el = k > 0 ? fabs(e[k - 1]) : 0.0, er = k < n - 1 ? fabs(e[k]) : 0.0;
    lo = fmin(lo, d[k] - el - er);
    hi = fmax(hi, d[k] + el + er);
    if (k < n - 1) em = fmax(em, e[k] * e[k]);
  }
  rl[tid] = lo;
  rh[tid] = hi;
  re[tid] = em;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) {
      rl[tid] = fmin(rl[tid], rl[tid + s]);
      rh[tid] = fmax(rh[tid], rh[tid + s]);
      re[tid] = fmax(re[tid], re[tid + s]);
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double pivmin = 2.2250738585072014e-308 * fmax(1.0, re[0]);
    const double tnorm = fmax(fabs(rl[0]), fabs(rh[0]));
    const double fudge = 2.1 * (EPS * tnorm * double(n) + 2.0 * pivmin);
    bounds[0] = rl[0] - fudge;
    bounds[1] = rh[0] + fudge;
    bounds[2] = pivmin;
    bounds[3] = fmax(tnorm, 2.2250738585072014e-308);
  }
}

// 16 eigenvalues per workgroup, 16 Sturm points each; lam ascending.
// The Sturm count at x is the number of negative ratios q_k = p_k / p_{k-1} of the leading
// principal minors p_k of T - x I.  The minors follow p_{k+1} = (d_k - x) p_k - e_{k-1}^2
// p_{k-1} with no division (the ratio form needs one per step, whose latency bound the
// recurrence); a sign change between p_{k-1} and p_k is a negative q_k.  T is scaled by a
// power of two to norm in [1, 2) (exact), a |q_k| below 2^-60 is replaced by -2^-60 (a
// perturbation of d_k far below the n eps ||T|| accuracy of any count), and the pair
// (p_{k-1}, p_k) is rescaled by a power of two every 8 steps, which keeps both inside the
// fp64 range (each step changes max(|p_k|, |p_{k-1}|) by at most a factor 8 up or 2^-60
// down).
__global__ __launch_bounds__(256) void tri_bisect_kernel(const double* __restrict__ d, const double* __restrict__ e,
                                                         int n, const double* __restrict__ bounds,
                                                         double* __restrict__ lam, int64_t wsi) {
  {   // slice blockIdx.y of a batch: d, e in its loop block, its bounds and n eigenvalues
    const int64_t it = blockIdx.y;
    d += it * wsi;
    e += it * wsi;
    bounds += 4 * it;
    lam += it * int64_t(n);
  }
  __shared__ double sd[BIS_STAGE], se2[BIS_STAGE];
  const int tid = threadIdx.x;
  const int grp = tid >> 4, pt = tid & 15;
  const int mi = blockIdx.x * 16 + grp;   // ascending index
  double lo = bounds[0], hi = bounds[1];
  // 2^-ex with ||T|| = bounds[3] in [2^(ex-1), 2^ex)
  int ex;
  (void)frexp(bounds[3], &ex);
  const double sc = ldexp(1.0, -ex);
  for (int it = 0; it < BIS_ITERS; ++it) {
    const double x = lo + (hi - lo) * (double(pt + 1) / double(BIS_PTS + 1));
    const double xs = x * sc;
    int cnt = 0;
    double pa = 0.0, pb = 1.0;   // p_{k-1}, p_k (p_{-1} = 0, p_0 = 1)
    auto step = [&](double dk, double e2k) {
      double p = fma(dk - xs, pb, -(e2k * pa));
      const double fl = ldexp(fabs(pb), -60);
      p = fabs(p) < fl ? -ldexp(pb, -60) : p;
      cnt += (__double2hiint(p) ^ __double2hiint(pb)) < 0;
      pa = pb;
      pb = p;
    };
    auto rescale = [&]() {
      int eb;
      (void)frexp(pb, &eb);
      pa = ldexp(pa, -eb);
      pb = ldexp(pb, -eb);
    };
    for (int k0 = 0; k0 < n; k0 += BIS_STAGE) {
      const int kn = min(BIS_STAGE, n - k0);
      __syncthreads();
      for (int k = tid; k < kn; k += 256) {
        sd[k] = d[k0 + k] * sc;
        const double es = (k0 + k > 0) ? e[k0 + k - 1] * sc : 0.0;
        se2[k] = es * es;
      }
      __syncthreads();
      int k = 0;
      // LDS operands are read 8 steps at a time, off the recurrence's critical path
      for (; k + 8 <= kn; k += 8) {
        double dk[8], ek[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          dk[u] = sd[k + u];
          ek[u] = se2[k + u];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) step(dk[u], ek[u]);
        rescale();
      }
      for (; k < kn; ++k) step(sd[k], se2[k]);
      rescale();
    }
    // smallest point whose count exceeds mi bounds the eigenvalue from above
    const unsigned long long bal = __ballot(cnt > mi);
    const unsigned gbits = unsigned((bal >> ((tid & 63) & ~15)) & 0xFFFFull);
    const int first = gbits ? __builtin_ctz(gbits) : BIS_PTS;
    const double w = hi - lo;
    const double nlo = first == 0 ? lo : lo + w * (double(first) / double(BIS_PTS + 1));
    const double nhi = first == BIS_PTS ? hi : lo + w * (double(first + 1) / double(BIS_PTS + 1));
    lo = nlo;
    hi = nhi;
  }
  if (pt == 0 && mi < n) lam[mi] = 0.5 * (lo + hi);
}

// ---- 3. clusters among the wanted eigenvalues (descending order j = 0 .. ncols-1): the
// length at each cluster's first member (0 at the others), and the first members of the
// clusters longer than CL_MAX in a list (in any order: each is processed on its own)
__global__ void tri_cluster_kernel(const double* __restrict__ lam, int n, int ncols,
                                   const double* __restrict__ bounds, int* __restrict__ clen,
                                   int* __restrict__ nbig, int* __restrict__ big) {
  {   // slice blockIdx.y of a batch (every array holds one block per slice)
    const int64_t it = blockIdx.y;
    lam += it * n;
    bounds += 4 * it;
    clen += it * ncols;
    nbig += it;
    big += it * ncols;
  }
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= ncols) return;
  const double ctol = CL_TOL * bounds[3];
  const bool start = j == 0 || (lam[n - j] - lam[n - 1 - j] > ctol);
  if (!start) {
    clen[j] = 0;
    return;
  }
  int len = 1;
  while (j + len < ncols && !(lam[n - j - len] - lam[n - 1 - j - len] > ctol)) ++len;
  clen[j] = len;
  if (len > CL_MAX) big[atomicAdd(nbig, 1)] = j;
}

__device__ __forceinline__ double start_value(int j, int k) {
  // deterministic pseudo-random start vector in [-1, 1) (integer hash)
  uint32_t h = uint32_t(j) * 0x9E3779B1u ^ (uint32_t(k) * 0x85EBCA77u + 0x165667B1u);
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  h *= 0x297A2D39u;
  h ^= h >> 15;
  return double(h) * (2.0 / 4294967296.0) - 1.0;
}

// Inverse iteration on T for the wanted eigenvalues, in two kernels:
//  A) one lane per vector (64 vectors per wave): LU with partial pivoting of T - lambda I
//     (the lambda of a cluster member is lowered to stay at least 10 eps ||T|| below the
//     previous member's), with the first solve's forward elimination of a pseudo-random
//     start vector done in the same pass.  Every lane runs its own vector's recurrence,
//     so a step costs one wave instruction per operation with no cross-lane traffic; d
//     and e are wave-uniform operands, loaded a batch of steps ahead, and the results are
//     only stored, so no memory latency enters the recurrence;
//  B) one wave per cluster (a lone eigenvalue is a cluster of one), members in order:
//     the first solve's back-substitution, orthogonalise the iterate against the
//     cluster's finished vectors (modified Gram-Schmidt), normalise, second solve,
//     orthogonalise again, normalise.  These recurrences read back what A stored; with
//     one wave per vector there are enough waves in flight to cover that latency
//     (one lane per vector measured latency-bound: 4.5 ms against 2.8 ms).
// The divisions are a hardware reciprocal refined by a Newton step, the quotient then
// corrected by its residual.  The arrays are step major, one column per vector: LU
// records Rt[k][j] = {1/pivot, u1, u2, multiplier} (32 B), row-interchange flags
// PVt[k][j] and the iterates in Z[k][j] (n x ncols, the layout the back-transformation
// reads), so the lanes of a wave touch consecutive addresses at every step.  Kernel B's
// orthogonalisation and scaling passes use all lanes (sums per lane in row order, then a
// fixed butterfly); its solves run on lane 0 out of LDS chunks the whole wave stages.

// 1 / b: hardware reciprocal refined by one Newton step
__device__ __forceinline__ double recip(double b) {
  double r = __builtin_amdgcn_rcp(b);
  return fma(r, fma(-b, r, 1.0), r);
}

// a / b from r ~ 1 / b, corrected by the residual of the product
__device__ __forceinline__ double quot(double a, double b, double r) {
  const double q = a * r;
  return fma(r, fma(-q, b, a), q);
}

// max over the 64 lanes (exact in any order)
__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}

constexpr int FCH = 256;   // steps per LDS-staged chunk of d, e in kernel A
constexpr int CHL = 256;   // steps per LDS-staged chunk of kernel B's solves
constexpr int CPLL = CHL / 64;

__global__ __launch_bounds__(64) void tri_inviter_a_kernel(const double* __restrict__ d, const double* __restrict__ e,
                                                           int n, const double* __restrict__ lam, int ncols,
                                                           const double* __restrict__ bounds,
                                                           const int* __restrict__ clen,
                                                           double* __restrict__ Rt, uint8_t* __restrict__ PVt,
                                                           double* __restrict__ Z, int64_t wsi) {
  {   // slice blockIdx.y of a batch: d, e in its loop block, the rest one block per slice
    const int64_t it = blockIdx.y;
    const int64_t nc = int64_t(n) * ncols;
    d += it * wsi;
    e += it * wsi;
    lam += it * n;
    bounds += 4 * it;
    clen += it * ncols;
    Rt += it * 4 * nc;
    PVt += it * nc;
    Z += it * nc;
  }
  const int lane = threadIdx.x;
  const int jr = blockIdx.x * 64 + lane;
  const int jv = min(jr, ncols - 1);   // lanes past the last vector repeat it
  int s = jv;   // the cluster's first member (clen is > 0 there, 0 at the others)
  while (s > 0 && clen[s] == 0) --s;
  const double tnorm = bounds[3];
  const double tiny = EPS * tnorm;
  double lmb = lam[n - 1 - s];
  for (int p = s + 1; p <= jv; ++p) lmb = fmin(lam[n - 1 - p], lmb - 10.0 * EPS * tnorm);
  const int nm1 = n - 1;
  double* Rj = Rt + int64_t(jv) * 4;   // record k at Rj + k * rs
  const int64_t rs = int64_t(ncols) * 4;
  uint8_t* Pj = PVt + jv;              // flag k at Pj + k * ncols
  double* zj = Z + jv;                 // entry k at zj + k * ncols

  // ---- factor T - lmb I = P L U (steps k = 0 .. n-2, then the last pivot) and, in the
  //      same pass, y = L^-1 P z0 for the start vector z0 (generated on the fly).
  //      Step k reads e[k], d[k+1], e[k+1], staged through LDS in chunks of FCH steps
  //      (every lane reads the same address: a broadcast), the next chunk's global loads
  //      in flight meanwhile.  Lanes past the last vector compute and store exactly what
  //      that vector's lane does (same bits).
  __shared__ double s_e[2][FCH + 1], s_d[2][FCH];
  double ge[FCH / 64 + 1], gd[FCH / 64];
  auto load_c = [&](int k0) {
#pragma unroll
    for (int u = 0; u < FCH / 64; ++u) {
      ge[u] = e[min(k0 + lane + 64 * u, max(n - 2, 0))];
      gd[u] = d[min(k0 + 1 + lane + 64 * u, n - 1)];
    }
    ge[FCH / 64] = e[min(k0 + FCH, max(n - 2, 0))];
  };
  auto stage_c = [&](int buf) {
#pragma unroll
    for (int u = 0; u < FCH / 64; ++u) {
      s_e[buf][lane + 64 * u] = ge[u];
      s_d[buf][lane + 64 * u] = gd[u];
    }
    if (lane == 0) s_e[buf][FCH] = ge[FCH / 64];
  };
  double cd = d[0] - lmb, cs = n > 1 ? e[0] : 0.0;
  double ycur = start_value(jv, 0);
  const int nchf = (nm1 + FCH - 1) / FCH;
  if (nchf > 0) {
    load_c(0);
    stage_c(0);
  }
  for (int c = 0; c < nchf; ++c) {
    const int buf = c & 1;
    if (c + 1 < nchf) load_c((c + 1) * FCH);
    __syncthreads();   // one wave: the chunk's LDS stores are visible
    const int k0 = c * FCH;
    const int cnt = min(FCH, nm1 - k0);
#pragma unroll 8
    for (int u = 0; u < cnt; ++u) {
      const int k = k0 + u;
      const double sub = s_e[buf][u];
      const double ndk = s_d[buf][u] - lmb;
      const double ns = k + 1 < nm1 ? s_e[buf][u + 1] : 0.0;
      // partial pivoting, branch-free: keep row k (pv = 0) or interchange with row k + 1
      const bool pv = !(fabs(cd) >= fabs(sub));
      double piv_u0 = pv ? sub : (cd == 0.0 ? tiny : cd);
      const double num = pv ? cd : sub;
      double rp = recip(piv_u0);
      const double l = quot(num, piv_u0, rp);
      const double u1 = pv ? ndk : cs;
      const double u2 = pv ? ns : 0.0;
      const double ncd = pv ? cs - l * ndk : ndk - l * cs;
      cs = pv ? -l * ns : ns;
      cd = ncd;
      if (fabs(piv_u0) < tiny) {   // rare: the recorded pivot is clamped to +-tiny
        piv_u0 = piv_u0 < 0.0 ? -tiny : tiny;
        rp = recip(piv_u0);
      }
      // forward elimination of the start vector with this step's multiplier
      const double yn = start_value(jv, k + 1);
      const double yk = pv ? yn : ycur;
      const double ynext = pv ? ycur : yn;
      *reinterpret_cast<f64x2*>(Rj + k * rs) = f64x2{rp, u1};
      *reinterpret_cast<f64x2*>(Rj + k * rs + 2) = f64x2{u2, l};
      Pj[int64_t(k) * ncols] = uint8_t(pv);
      zj[int64_t(k) * ncols] = yk;
      ycur = ynext - l * yk;
    }
    if (c + 1 < nchf) stage_c(buf ^ 1);
  }
  {
    double p0 = cd;
    if (fabs(p0) < tiny) p0 = p0 < 0.0 ? -tiny : tiny;
    *reinterpret_cast<f64x2*>(Rj + nm1 * rs) = f64x2{recip(p0), 0.0};
    *reinterpret_cast<f64x2*>(Rj + nm1 * rs + 2) = f64x2{0.0, 0.0};
    Pj[int64_t(nm1) * ncols] = 0;
    zj[int64_t(nm1) * ncols] = ycur;
  }
}

// back-substitution z <- U^-1 z on one vector (records R[k * rs], iterate z[k * zs]),
// chunks from the end: lane 0 runs the recurrence out of LDS chunks of CHL steps staged by
// the whole wave (the next chunk's loads in flight); returns ||z||^2 (to every lane)
__device__ double inv_usolve_lds(const double* __restrict__ R, int64_t rs, double* __restrict__ z, int64_t zs, int n,
                                 double (*__restrict__ s_in)[CHL][4], double (*__restrict__ s_z)[CHL],
                                 double* __restrict__ s_out, double* __restrict__ s_sc) {
  const int lane = threadIdx.x;
  const int nch = (n + CHL - 1) / CHL;
  double gr[CPLL][4], gz[CPLL];
  auto load = [&](int c) {
#pragma unroll
    for (int u = 0; u < CPLL; ++u) {
      const int k = min(c * CHL + lane + 64 * u, n - 1);
      const f64x2 a = *reinterpret_cast<const f64x2*>(R + int64_t(k) * rs);
      const f64x2 b = *reinterpret_cast<const f64x2*>(R + int64_t(k) * rs + 2);
      gr[u][0] = a[0];
      gr[u][1] = a[1];
      gr[u][2] = b[0];
      gr[u][3] = b[1];
      gz[u] = z[int64_t(k) * zs];
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int u = 0; u < CPLL; ++u) {
      const int i = lane + 64 * u;
#pragma unroll
      for (int t = 0; t < 4; ++t) s_in[buf][i][t] = gr[u][t];
      s_z[buf][i] = gz[u];
    }
  };
  double x1 = 0.0, x2 = 0.0, nrm2 = 0.0;
  load(nch - 1);
  stage((nch - 1) & 1);
  for (int c = nch - 1; c >= 0; --c) {
    const int buf = c & 1;
    if (c > 0) load(c - 1);
    __syncthreads();
    const int cnt = min(CHL, n - c * CHL);
    if (lane == 0) {
      #pragma unroll 8
      for (int i = cnt - 1; i >= 0; --i) {
        // the older x2 term first: only one fma and the scaling wait for x1
        const double t = fma(-s_in[buf][i][2], x2, s_z[buf][i]);
        const double xk = fma(-s_in[buf][i][1], x1, t) * s_in[buf][i][0];
        s_out[i] = xk;
        nrm2 += xk * xk;
        x2 = x1;
        x1 = xk;
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < CPLL; ++u) {
      const int i = lane + 64 * u;
      if (i < cnt) z[int64_t(c * CHL + i) * zs] = s_out[i];
    }
    if (c > 0) stage(buf ^ 1);
  }
  if (lane == 0) s_sc[0] = nrm2;
  __syncthreads();
  return s_sc[0];
}

// Helpers of the per-vector and per-cluster kernels (one wave each); vector p's entry k
// is Z[k * ncols + p].
// 1 / ||z||, or for a badly scaled z 1 / ||z|| taken after scaling by its largest entry
__device__ double inv_unit_scale(const double* __restrict__ z, int64_t zs, int n, double nrm2) {
  if (nrm2 > 0.0 && nrm2 < 1e300) return 1.0 / sqrt(nrm2);
  const int lane = threadIdx.x;
  double mx = 0.0;
  for (int k = lane; k < n; k += 64) mx = fmax(mx, fabs(z[int64_t(k) * zs]));
  mx = wave_max(mx);
  const double inv_mx = mx > 0.0 && mx < 1e308 ? 1.0 / mx : 1.0;
  double s2 = 0.0;
  for (int k = lane; k < n; k += 64) {
    const double v = z[int64_t(k) * zs] * inv_mx;
    s2 += v * v;
  }
  s2 = wave_sum(s2);
  return s2 > 0.0 ? inv_mx / sqrt(s2) : 1.0;
}

// z *= sc, in batches of 8 entries per lane (loads first, so their latencies overlap)
__device__ void inv_scale(double* __restrict__ z, int64_t zs, int n, double sc) {
  const int lane = threadIdx.x;
  for (int k0 = lane; k0 < n; k0 += 64 * 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + 64 * u;
      v[u] = k < n ? z[int64_t(k) * zs] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + 64 * u;
      if (k < n) z[int64_t(k) * zs] = v[u] * sc;
    }
  }
}

// first solve's back-substitution, one wave per vector; its squared norm to nrm[j]
__global__ __launch_bounds__(64) void tri_inviter_u_kernel(int n, int ncols, const double* __restrict__ Rt,
                                                           double* __restrict__ Z, double* __restrict__ nrm) {
  {   // slice blockIdx.y of a batch
    const int64_t it = blockIdx.y, nc = int64_t(n) * ncols;
    Rt += it * 4 * nc;
    Z += it * nc;
    nrm += it * ncols;
  }
  __shared__ double s_in[2][CHL][4];
  __shared__ double s_z[2][CHL];
  __shared__ double s_out[CHL];
  __shared__ double s_sc[1];
  const int jv = blockIdx.x;
  const double n1 = inv_usolve_lds(Rt + int64_t(jv) * 4, int64_t(ncols) * 4, Z + jv, ncols, n, s_in, s_z, s_out, s_sc);
  if (threadIdx.x == 0) nrm[jv] = n1;
}

// one wave per cluster of two to CL_MAX members (final = 0) or of at most CL_MAX members
// (final = 1): members in order, orthogonalise against the cluster's earlier members
// (modified Gram-Schmidt, those already normalised) and normalise (scl = 1).  A lone
// vector's final normalisation is left to the output kernel: scl = 1 / ||z|| from the
// squared norm its solve recorded (scaling commutes with the back-transformation); only a
// norm outside [1e-100, 1e100] is applied here.  Longer clusters: tri_inviter_obig_kernel.
__global__ __launch_bounds__(64) void tri_inviter_o_kernel(int n, int ncols, int final, const int* __restrict__ clen,
                                                           double* __restrict__ Z, const double* __restrict__ nrm,
                                                           double* __restrict__ scl) {
  {   // slice blockIdx.y of a batch
    const int64_t it = blockIdx.y;
    clen += it * ncols;
    Z += it * int64_t(n) * ncols;
    nrm += it * ncols;
    scl += it * ncols;
  }
  const int j = blockIdx.x;
  const int len = clen[j];
  if (len == 0 || len > CL_MAX || (len == 1 && !final)) return;
  const int lane = threadIdx.x;
  if (len == 1) {
    const double s2 = nrm[j];
    double sv = 1.0;
    if (s2 > 1e-200 && s2 < 1e200)
      sv = 1.0 / sqrt(s2);
    else
      inv_scale(Z + j, ncols, n, inv_unit_scale(Z + j, ncols, n, s2));
    if (lane == 0) scl[j] = sv;
    return;
  }
  for (int q = 0; q < len; ++q) {
    const int jv = j + q;
    double* z = Z + jv;
    double s2 = nrm[jv];
    if (q > 0) {
      for (int p = j; p < jv; ++p) {
        const double* zp = Z + p;
        double dot = 0.0;
#pragma unroll 8
        for (int k = lane; k < n; k += 64) dot += zp[int64_t(k) * ncols] * z[int64_t(k) * ncols];
        dot = wave_sum(dot);
        for (int k = lane; k < n; k += 64) z[int64_t(k) * ncols] -= dot * zp[int64_t(k) * ncols];
      }
      s2 = 0.0;
#pragma unroll 8
      for (int k = lane; k < n; k += 64) s2 += z[int64_t(k) * ncols] * z[int64_t(k) * ncols];
      s2 = wave_sum(s2);
    }
    inv_scale(z, ncols, n, inv_unit_scale(z, ncols, n, s2));
    if (lane == 0 && final) scl[jv] = 1.0;
    __syncthreads();   // the normalised member is read by the next members' passes
  }
}

constexpr int OB_T = 1024;          // threads per long cluster (16 waves)
constexpr int OB_W = OB_T / 64;
constexpr int OB_CH = 256;          // earlier members per chunk of a Gram-Schmidt pass
constexpr int OB_U = OB_CH / 64;

// sum (op 0) or max (op 1) over the workgroup, the same value to every thread; waves'
// results combined in wave order
__device__ double ob_reduce(double v, int op, double* __restrict__ red) {
  v = op == 0 ? wave_sum(v) : wave_max(v);
  __syncthreads();   // red is free
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = red[0];
  for (int w = 1; w < OB_W; ++w) r = op == 0 ? r + red[w] : fmax(r, red[w]);
  return r;
}

// one workgroup per cluster of more than CL_MAX members (first members listed in big[]):
// members in order, each orthogonalised against the cluster's earlier, already normalised
// members by two block Gram-Schmidt passes (chunks of OB_CH earlier members: all the
// chunk's projections from one set of dot products, chunks in order), then normalised
// (scl = 1 when final).  The cluster occupies contiguous columns of Z, so a wave reading
// the chunk's entries of one row reads consecutive addresses.  Dot products: wave w sums
// rows w, w + 16, ..., the 16 wave partials are added in wave order.
__global__ __launch_bounds__(OB_T) void tri_inviter_obig_kernel(int n, int ncols, int final,
                                                               const int* __restrict__ clen,
                                                               const int* __restrict__ nbig,
                                                               const int* __restrict__ big, double* __restrict__ Z,
                                                               double* __restrict__ scl) {
  {   // slice blockIdx.y of a batch
    const int64_t it = blockIdx.y;
    clen += it * ncols;
    nbig += it;
    big += it * ncols;
    Z += it * int64_t(n) * ncols;
    scl += it * ncols;
  }
  __shared__ double part[OB_W][OB_CH];
  __shared__ double dots[OB_CH];
  __shared__ double red[OB_W];
  if (int(blockIdx.x) >= *nbig) return;
  const int j = big[blockIdx.x];
  const int len = clen[j];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int q = 0; q < len; ++q) {
    const int jq = j + q;
    for (int pass = 0; pass < 2 && q > 0; ++pass) {
      for (int p0 = 0; p0 < q; p0 += OB_CH) {
        const int pc = min(OB_CH, q - p0);
        double acc[OB_U];
#pragma unroll
        for (int u = 0; u < OB_U; ++u) acc[u] = 0.0;
        for (int k = wv; k < n; k += OB_W) {
          const double* row = Z + int64_t(k) * ncols + j + p0;
          const double zk = Z[int64_t(k) * ncols + jq];
#pragma unroll
          for (int u = 0; u < OB_U; ++u) {
            const int p = lane + 64 * u;
            if (p < pc) acc[u] = fma(row[p], zk, acc[u]);
          }
        }
#pragma unroll
        for (int u = 0; u < OB_U; ++u) part[wv][lane + 64 * u] = acc[u];
        __syncthreads();
        if (tid < pc) {
          double t = part[0][tid];
          for (int w = 1; w < OB_W; ++w) t += part[w][tid];
          dots[tid] = t;
        }
        __syncthreads();
        for (int k = wv; k < n; k += OB_W) {
          const double* row = Z + int64_t(k) * ncols + j + p0;
          double t = 0.0;
#pragma unroll
          for (int u = 0; u < OB_U; ++u) {
            const int p = lane + 64 * u;
            if (p < pc) t = fma(dots[p], row[p], t);
          }
          t = wave_sum(t);
          if (lane == 0) Z[int64_t(k) * ncols + jq] -= t;
        }
        __syncthreads();   // the updated member is read by the next chunk or pass
      }
    }
    double s2 = 0.0;
    for (int k = tid; k < n; k += OB_T) {
      const double v = Z[int64_t(k) * ncols + jq];
      s2 = fma(v, v, s2);
    }
    s2 = ob_reduce(s2, 0, red);
    double sc;
    if (s2 > 0.0 && s2 < 1e300) {
      sc = 1.0 / sqrt(s2);
    } else {   // badly scaled: the norm after scaling by the largest entry
      double mx = 0.0;
      for (int k = tid; k < n; k += OB_T) mx = fmax(mx, fabs(Z[int64_t(k) * ncols + jq]));
      mx = ob_reduce(mx, 1, red);
      const double inv_mx = mx > 0.0 && mx < 1e308 ? 1.0 / mx : 1.0;
      double t2 = 0.0;
      for (int k = tid; k < n; k += OB_T) {
        const double v = Z[int64_t(k) * ncols + jq] * inv_mx;
        t2 = fma(v, v, t2);
      }
      t2 = ob_reduce(t2, 0, red);
      sc = t2 > 0.0 ? inv_mx / sqrt(t2) : 1.0;
    }
    for (int k = tid; k < n; k += OB_T) Z[int64_t(k) * ncols + jq] *= sc;
    if (tid == 0 && final) scl[jq] = 1.0;
    __syncthreads();   // the normalised member is read by the next members' passes
  }
}

// second solve, one wave per vector: y = L^-1 P (sc z), then U^-1 y; its squared norm to
// nrm[j].  A lone vector's iterate is normalised on the fly (sc from its recorded norm);
// cluster members were normalised by the cluster kernel (sc = 1).
__global__ __launch_bounds__(64) void tri_inviter_s_kernel(int n, int ncols, const int* __restrict__ clen,
                                                           const double* __restrict__ Rt,
                                                           const uint8_t* __restrict__ PVt,
                                                           double* __restrict__ Z, double* __restrict__ nrm) {
  {   // slice blockIdx.y of a batch
    const int64_t it = blockIdx.y, nc = int64_t(n) * ncols;
    clen += it * ncols;
    Rt += it * 4 * nc;
    PVt += it * nc;
    Z += it * nc;
    nrm += it * ncols;
  }
  __shared__ double s_in[2][CHL][4];
  __shared__ double s_z[2][CHL];
  __shared__ double s_out[CHL];
  __shared__ uint8_t s_piv[2][CHL];
  __shared__ double s_zx[2];
  __shared__ double s_sc[1];
  const int jv = blockIdx.x;
  const int lane = threadIdx.x;
  const int nm1 = n - 1;
  const int nch = (n + CHL - 1) / CHL;
  const double* R = Rt + int64_t(jv) * 4;   // record k at R + k * rs
  const int64_t rs = int64_t(ncols) * 4;
  const uint8_t* PV = PVt + jv;               // flag k at PV + k * ncols
  double* z = Z + jv;                         // entry k at z + k * ncols
  const bool lone = clen[jv] == 1;
  const double sc = lone ? inv_unit_scale(z, ncols, n, nrm[jv]) : 1.0;
  // ---- y = L^-1 P (sc z): chunk c stages z[c CHL .. c CHL + CHL] (one past, for the
  //      interchange), the multipliers and the flags
  double gz[CPLL], gl[CPLL], gx = 0.0;
  uint8_t gp[CPLL];
  auto load = [&](int c) {
#pragma unroll
    for (int u = 0; u < CPLL; ++u) {
      const int k = min(c * CHL + lane + 64 * u, n - 1);
      gz[u] = z[int64_t(k) * ncols] * sc;
      gl[u] = R[int64_t(k) * rs + 3];
      gp[u] = PV[int64_t(k) * ncols];
    }
    gx = z[int64_t(min(c * CHL + CHL, n - 1)) * ncols] * sc;
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int u = 0; u < CPLL; ++u) {
      const int i = lane + 64 * u;
      s_z[buf][i] = gz[u];
      s_in[buf][i][3] = gl[u];
      s_piv[buf][i] = gp[u];
    }
    if (lane == 0) s_zx[buf] = gx;
  };
  load(0);
  stage(0);
  double ycur = z[0] * sc;
  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    if (c + 1 < nch) load(c + 1);
    __syncthreads();
    const int cnt = min(CHL, nm1 - c * CHL);   // elimination steps in this chunk
    if (lane == 0) {
      #pragma unroll 8
      for (int i = 0; i < cnt; ++i) {
        const double yn = i + 1 < CHL ? s_z[buf][i + 1] : s_zx[buf];
        const bool sw = s_piv[buf][i];
        const double yk = sw ? yn : ycur;
        const double ynext = sw ? ycur : yn;
        s_out[i] = yk;
        ycur = fma(-s_in[buf][i][3], yk, ynext);
      }
      if (c == nch - 1) s_out[max(cnt, 0)] = ycur;   // the last element
    }
    __syncthreads();
    const int nw = min(CHL, n - c * CHL);   // elements written by this chunk
#pragma unroll
    for (int u = 0; u < CPLL; ++u) {
      const int i = lane + 64 * u;
      if (i < nw) z[int64_t(c * CHL + i) * ncols] = s_out[i];
    }
    if (c + 1 < nch) stage(buf ^ 1);
  }
  __syncthreads();
  const double n2 = inv_usolve_lds(R, rs, z, ncols, n, s_in, s_z, s_out, s_sc);
  if (lane == 0) nrm[jv] = n2;
}

// ---- 4. back-transformation.  Block g holds reflectors g*BW .. g*BW+BW-1; reflector t
// of the block lives in column g0 + t, rows > g0 + t.
__device__ __forceinline__ double refl(const double* __restrict__ A, int64_t lda, int nref, int g0, int r, int t) {
  return (g0 + t < nref && r > g0 + t) ? A[int64_t(r) * lda + g0 + t] : 0.0;
}

// partial V^T V of block g over one row chunk
// element strides between the slices of a batch in the back-transformation's arrays
struct BtStrides {
  int64_t a;    // the matrix holding the reflectors
  int64_t wsi;  // a slice's loop block (tau)
  int64_t gp, t, yp, y;   // V^T V partials, the T factors, V^T Z partials, V^T Z and T V^T Z
  int64_t z;    // eigenvectors of T (n x ncols)
  int64_t qt;   // output rows
};

__global__ __launch_bounds__(256) void bt_gram_kernel(const double* __restrict__ A, int64_t lda, int n, int nref,
                                                      int ngc, double* __restrict__ Gp, BtStrides bs) {
  A += blockIdx.z * bs.a;   // slice blockIdx.z of a batch
  Gp += blockIdx.z * bs.gp;
  __shared__ double sv[32][BW + 1];
  const int tid = threadIdx.x;
  const int g = blockIdx.x, ch = blockIdx.y;
  const int g0 = g * BW;
  const int r0 = max(g0 + 1, ch * G_CHUNK), r1 = min(n, (ch + 1) * G_CHUNK);
  const int ty = tid >> 4, tx = tid & 15;   // 8 x 8 outputs: rows ty*8.., cols tx*8..
  double acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[a][q] = 0.0;
  for (int rb = r0; rb < r1; rb += 32) {
    __syncthreads();
    for (int q = tid; q < 32 * BW; q += 256) {
      const int x = q / BW, t = q % BW;
      const int r = rb + x;
      sv[x][t] = r < r1 ? refl(A, lda, nref, g0, r, t) : 0.0;
    }
    __syncthreads();
    for (int x = 0; x < 32; ++x) {
      double a8[8], b8[8];
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        a8[a] = sv[x][ty * 8 + a];
        b8[a] = sv[x][tx * 8 + a];
      }
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[a][q] += a8[a] * b8[q];
    }
  }
  double* out = Gp + (int64_t(g) * ngc + ch) * BW * BW;
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int q = 0; q < 8; ++q) out[(ty * 8 + a) * BW + tx * 8 + q] = acc[a][q];
}

// the row-chunk partials of each group's V^T V summed in chunk order into its first partial
__global__ __launch_bounds__(256) void bt_gsum_kernel(double* __restrict__ Gp, int ngc, BtStrides bs) {
  Gp += blockIdx.z * bs.gp;   // slice blockIdx.z
  const int g = blockIdx.y;
  const int q = blockIdx.x * 256 + threadIdx.x;   // < BW * BW
  double* base = Gp + int64_t(g) * ngc * BW * BW + q;
  double s = 0.0;
  for (int ch = 0; ch < ngc; ++ch) s += base[int64_t(ch) * BW * BW];
  base[0] = s;
}

// T of block g (upper triangular): T[j][j] = tau_j, T[0:j, j] = -tau_j T[0:j,0:j] G[0:j, j];
// thread i owns row i of T, kept in LDS.  G = V^T V is symmetric, so its column j is
// row j (one coalesced load per column, the next column's load in flight).
__global__ __launch_bounds__(BW) void bt_t_kernel(const double* __restrict__ Gp, int ngc, int nsum, int nref,
                                                  const double* __restrict__ tau, double* __restrict__ Tm,
                                                  BtStrides bs) {
  Gp += blockIdx.y * bs.gp;   // slice blockIdx.y
  tau += blockIdx.y * bs.wsi;
  Tm += blockIdx.y * bs.t;
  __shared__ double Ts[BW][BW + 1];
  __shared__ double gcol[2][BW];
  const int tid = threadIdx.x;
  const int g = blockIdx.x, g0 = g * BW;
  // column j of G (entries 0..j-1 used), summed over the first nsum row-chunk partials in
  // chunk order (ngc partials per group in the layout)
  auto load_col = [&](int j) {
    double s = 0.0;
    for (int ch = 0; ch < nsum; ++ch) s += Gp[(int64_t(g) * ngc + ch) * BW * BW + int64_t(j) * BW + tid];
    return s;
  };
  const int i = tid;
  double nxt = load_col(0);
  for (int jcol = 0; jcol < BW; ++jcol) {
    gcol[jcol & 1][tid] = nxt;
    __syncthreads();
    if (jcol + 1 < BW) nxt = load_col(jcol + 1);
    const double tj = g0 + jcol < nref ? tau[g0 + jcol] : 0.0;
    double v = 0.0;
    if (i < jcol) {
      double s = 0.0;
      for (int l = i; l < jcol; ++l) s += Ts[i][l] * gcol[jcol & 1][l];
      v = -tj * s;
    } else if (i == jcol) {
      v = tj;
    }
    Ts[i][jcol] = v;
  }
  __syncthreads();
  double* T = Tm + int64_t(g) * BW * BW;
  for (int q = tid; q < BW * BW; q += BW) T[q] = Ts[q / BW][q % BW];
}

// Yp[ch][a][c] = sum over the chunk's rows of V[r][a] Z[r][c]   (64 columns per workgroup)
// on fp64 MFMA: four waves of 32 reflectors x 64 columns, rows staged 32 at a time through
// LDS (the next rows' loads in flight during the MFMAs)
constexpr int BVP = BW + 2;   // LDS pitch of the staged reflector rows
constexpr int BZP = 64 + 2;   // LDS pitch of the staged Z rows

__global__ __launch_bounds__(256) void bt_vtz_kernel(const double* __restrict__ A, int64_t lda, int n, int nref,
                                                     int g0, const double* __restrict__ Z, int ncols,
                                                     double* __restrict__ Yp, BtStrides bs) {
  A += blockIdx.z * bs.a;   // slice blockIdx.z
  Z += blockIdx.z * bs.z;
  Yp += blockIdx.z * bs.yp;
  __shared__ double sv[32][BVP];
  __shared__ double sz[32][BZP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lq = lane >> 4;
  const int c0 = blockIdx.x * 64, ch = blockIdx.y;
  const int rbase = g0 + 1 + ch * BT_CHUNK;
  const int rend = min(n, rbase + BT_CHUNK);
  // staging: V element (row x, reflector t) with x = tid / 8 .. (4 rows apart? no: one row),
  // t = (tid % 8) * 16 + u; Z element (row x, column cc) with x = tid / 8, cc = (tid % 8) * 8 + u
  const int sx = tid >> 3, st16 = (tid & 7) * 16, sc8 = (tid & 7) * 8;
  double gv[16], gz[8];
  auto load = [&](int rb) {
    const int r = min(rb + sx, n - 1);
#pragma unroll
    for (int u = 0; u < 16; ++u) gv[u] = A[int64_t(r) * lda + min(g0 + st16 + u, nref - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) gz[u] = Z[int64_t(r) * ncols + min(c0 + sc8 + u, ncols - 1)];
  };
  auto store = [&](int rb) {
    const int r = rb + sx;
    const bool okr = r < rend;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int t = st16 + u;
      sv[sx][t] = (okr && g0 + t < nref && r > g0 + t) ? gv[u] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) sz[sx][sc8 + u] = (okr && c0 + sc8 + u < ncols) ? gz[u] : 0.0;
  };
  f64x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
  load(rbase);
  for (int rb = rbase; rb < rend; rb += 32) {
    __syncthreads();
    store(rb);
    __syncthreads();
    if (rb + 32 < rend) load(rb + 32);
#pragma unroll
    for (int kk = 0; kk < 32; kk += 4) {
      double a[2], b[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = sv[kk + lq][wave * 32 + i * 16 + l16];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sz[kk + lq][j * 16 + l16];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  // fp64 16 x 16 output: lane l, element e -> row l / 16 + 4 e, column l % 16
  double* out = Yp + int64_t(ch) * BW * ncols;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int a = wave * 32 + i * 16 + lq + 4 * e, cc = c0 + j * 16 + l16;
        if (cc < ncols) out[int64_t(a) * ncols + cc] = acc[i][j][e];
      }
}

// Y[a][c] = sum_ch Yp[ch][a][c]  (one element per thread, partials in order)
__global__ __launch_bounds__(256) void bt_reduce_kernel(const double* __restrict__ Yp, int nch, int ncols,
                                                        double* __restrict__ Y, BtStrides bs) {
  Yp += blockIdx.y * bs.yp;   // slice blockIdx.y
  Y += blockIdx.y * bs.y;
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t tot = int64_t(BW) * ncols;
  if (e >= tot) return;
  double t[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) t[u] = Yp[int64_t(min(u, nch - 1)) * tot + e];
  double sacc = 0.0;
#pragma unroll
  for (int u = 0; u < 16; ++u) sacc += u < nch ? t[u] : 0.0;
  for (int ch = 16; ch < nch; ++ch) sacc += Yp[int64_t(ch) * tot + e];
  Y[e] = sacc;
}

// Y2 = T Y for 16 rows x 64 columns per workgroup (T upper triangular)
__global__ __launch_bounds__(256) void bt_ty_kernel(const double* __restrict__ Y, const double* __restrict__ T,
                                                    int ncols, double* __restrict__ Y2, BtStrides bs) {
  Y += blockIdx.z * bs.y;   // slice blockIdx.z
  T += blockIdx.z * bs.t;
  Y2 += blockIdx.z * bs.y;
  __shared__ double sy[BW][64 + 1];
  __shared__ double st[16][BW + 1];
  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * 64, a0 = blockIdx.y * 16;
  // every load first (clamped addresses), then the LDS stores with the masks
  constexpr int NY = BW * 64 / 256, NT = 16 * BW / 256;
  double gy[NY], gt[NT];
  const int ccy = tid & 63, ccl = min(c0 + ccy, ncols - 1);
#pragma unroll
  for (int u = 0; u < NY; ++u) gy[u] = Y[int64_t((tid >> 6) + 4 * u) * ncols + ccl];
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int q = tid + 256 * u;
    gt[u] = T[(a0 + q / BW) * BW + q % BW];
  }
#pragma unroll
  for (int u = 0; u < NY; ++u) sy[(tid >> 6) + 4 * u][ccy] = c0 + ccy < ncols ? gy[u] : 0.0;
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int q = tid + 256 * u;
    st[q / BW][q % BW] = gt[u];
  }
  __syncthreads();
  const int ar = tid >> 4, cq = (tid & 15) * 4;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int l = a0 + ar; l < BW; ++l) {
    const double t = st[ar][l];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] += t * sy[l][cq + q];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int cc = c0 + cq + q;
    if (cc < ncols) Y2[int64_t(a0 + ar) * ncols + cc] = acc[q];
  }
}

// Z[r][c] -= sum_a V[r][a] Y2[a][c]   (64 x 64 tile of rows g0+1.. per workgroup) on fp64
// MFMA: four waves of 32 x 32, reflectors staged 32 at a time; the tile's old Z values are
// loaded at the start
constexpr int BUP = 32 + 1;   // LDS pitch of the staged V rows (odd: column reads spread over banks)

__global__ __launch_bounds__(256) void bt_update_kernel(const double* __restrict__ A, int64_t lda, int n, int nref,
                                                        int g0, const double* __restrict__ Y2, int ncols,
                                                        double* __restrict__ Z, BtStrides bs) {
  A += blockIdx.z * bs.a;   // slice blockIdx.z
  Y2 += blockIdx.z * bs.y;
  Z += blockIdx.z * bs.z;
  __shared__ double sv[64][BUP];
  __shared__ double sy[32][BZP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int l16 = lane & 15, lq = lane >> 4;
  const int r0 = g0 + 1 + blockIdx.x * 64, c0 = blockIdx.y * 64;
  double old[2][2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = min(r0 + wr * 32 + i * 16 + lq + 4 * e, n - 1);
        const int cc = min(c0 + wc * 32 + j * 16 + l16, ncols - 1);
        old[i][j][e] = Z[int64_t(r) * ncols + cc];
      }
  // staging: V (row x = tid / 4, reflectors k0 + (tid % 4) * 8 + u), Y2 (reflector row
  // t = tid / 8, columns (tid % 8) * 8 + u)
  const int vx = tid >> 2, vt = (tid & 3) * 8, yt = tid >> 3, yc = (tid & 7) * 8;
  double gv[8], gy[8];
  auto load = [&](int k0) {
    const int r = min(r0 + vx, n - 1);
#pragma unroll
    for (int u = 0; u < 8; ++u) gv[u] = A[int64_t(r) * lda + min(g0 + k0 + vt + u, nref - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) gy[u] = Y2[int64_t(k0 + yt) * ncols + min(c0 + yc + u, ncols - 1)];
  };
  auto store = [&](int k0) {
    const int r = r0 + vx;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = k0 + vt + u;
      sv[vx][vt + u] = (r < n && g0 + t < nref && r > g0 + t) ? gv[u] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) sy[yt][yc + u] = c0 + yc + u < ncols ? gy[u] : 0.0;
  };
  f64x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
  load(0);
  for (int k0 = 0; k0 < BW; k0 += 32) {
    __syncthreads();
    store(k0);
    __syncthreads();
    if (k0 + 32 < BW) load(k0 + 32);
#pragma unroll
    for (int kk = 0; kk < 32; kk += 4) {
      double a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = sv[wr * 32 + i * 16 + l16][kk + lq];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = sy[kk + lq][wc * 32 + j * 16 + l16];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = r0 + wr * 32 + i * 16 + lq + 4 * e, cc = c0 + wc * 32 + j * 16 + l16;
        if (r < n && cc < ncols) Z[int64_t(r) * ncols + cc] = old[i][j][e] - acc[i][j][e];
      }
}

// ---- outputs: sigma (all k, descending) and Qt rows = eigenvectors, sign-fixed, fp32
__global__ void tri_sigma_kernel(const double* __restrict__ lam, int n, float* __restrict__ sigma, int64_t s_sigma) {
  lam += int64_t(blockIdx.y) * n;     // slice blockIdx.y
  sigma += int64_t(blockIdx.y) * s_sigma;
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m < n) sigma[m] = float(sqrt(fmax(lam[n - 1 - m], 0.0)));
}

__global__ __launch_bounds__(256) void tri_out_kernel(const double* __restrict__ Z, const double* __restrict__ scl,
                                                      int n, int ncols, float* __restrict__ Qt, BtStrides bs) {
  Z += blockIdx.y * bs.z;   // slice blockIdx.y
  scl += int64_t(blockIdx.y) * ncols;
  Qt += blockIdx.y * bs.qt;
  __shared__ double bv[256];
  __shared__ int bi[256];
  const int j = blockIdx.x, tid = threadIdx.x;
  double best = -1.0;
  int bidx = 0;
  for (int k = tid; k < n; k += 256) {
    const double a = fabs(Z[int64_t(k) * ncols + j]);
    if (a > best) {
      best = a;
      bidx = k;
    }
  }
  bv[tid] = best;
  bi[tid] = bidx;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) {
      const double o = bv[tid + s];
      const int oi = bi[tid + s];
      if (o > bv[tid] || (o == bv[tid] && oi < bi[tid])) {
        bv[tid] = o;
        bi[tid] = oi;
      }
    }
    __syncthreads();
  }
  // the vector's pending normalisation (positive: the sign choice is unaffected)
  const double sgn = (Z[int64_t(bi[0]) * ncols + j] < 0.0 ? -1.0 : 1.0) * scl[j];
  for (int k = tid; k < n; k += 256) Qt[int64_t(j) * n + k] = float(sgn * Z[int64_t(k) * ncols + j]);
}

struct TWs {
  // the reduction loop's arrays: one block of `istride` doubles per slice of a batch,
  // these pointers into slice 0's block
  double *P, *S, *SV, *SW, *npart, *x0, *xv, *d, *e, *tau, *Wp;
  int64_t istride;
  // the later stages: one block per slice of each array (lam n, bounds 4, the inverse
  // iteration's factors, iterates and clusters, the back-transformation's partials)
  double *lam, *bounds, *U, *Z, *nrm, *scl, *Gp, *T, *Yp, *Yr, *Y2;
  int *clen, *nbig, *big;
  uint8_t* piv;
};

TWs carve_tri(Carve& cv, int64_t n, int64_t ncols, int64_t batch) {
  const int64_t nbt = cdiv(n, TS);
  const int64_t nref = std::max<int64_t>(n - 1, 0);
  const int64_t ngroups = std::max<int64_t>(cdiv(nref, BW), 1);
  const int64_t ngc = cdiv(n, G_CHUNK);
  const int64_t nbc = cdiv(n, BT_CHUNK);
  TWs w;
  // per-slice loop block: every array starts on a 256-byte boundary
  int64_t o = 0;
  auto put = [&](int64_t len) {
    const int64_t at = o;
    o += (len + 31) / 32 * 32;
    return at;
  };
  const int64_t oP = put(nbt * nbt * TS), oS = put(nbt * (nbt + 1) / 2), oSV = put(nbt * NB), oSW = put(nbt * NB);
  const int64_t onp = put(2 * NPB * nbt);   // two columns' partials, NPB per row block
  const int64_t ox0 = put(2), oxv = put(2 * n);   // two columns as contiguous vectors
  const int64_t od = put(n), oe = put(n), otau = put(n), oWp = put(n * NB);
  w.istride = o;
  double* loop = cv.take<double>(size_t(std::max<int64_t>(batch, 1) * o));
  w.P = loop + oP;
  w.S = loop + oS;
  w.SV = loop + oSV;
  w.SW = loop + oSW;
  w.npart = loop + onp;
  w.x0 = loop + ox0;
  w.xv = loop + oxv;
  w.d = loop + od;
  w.e = loop + oe;
  w.tau = loop + otau;
  w.Wp = loop + oWp;
  // eigenvalues and spectrum bounds of every slice (found for the whole batch at once)
  w.lam = cv.take<double>(size_t(std::max<int64_t>(batch, 1) * n));
  w.bounds = cv.take<double>(size_t(4 * std::max<int64_t>(batch, 1)));
  // inverse iteration: one block of each array per slice (the batch is solved at once)
  const int64_t nbat = std::max<int64_t>(batch, 1);
  w.U = cv.take<double>(size_t(nbat * 4 * n * ncols));
  w.piv = cv.take<uint8_t>(size_t(nbat * n * ncols));
  w.Z = cv.take<double>(size_t(nbat * n * ncols));
  // back-transformation: one block of each array per slice (the batch is transformed at once)
  w.Gp = cv.take<double>(size_t(nbat * ngroups * ngc * BW * BW));
  w.T = cv.take<double>(size_t(nbat * ngroups * BW * BW));
  w.Yp = cv.take<double>(size_t(nbat * nbc * BW * ncols));
  w.Yr = cv.take<double>(size_t(nbat * BW * ncols));
  w.Y2 = cv.take<double>(size_t(nbat * BW * ncols));
  w.nrm = cv.take<double>(size_t(nbat * ncols));
  w.scl = cv.take<double>(size_t(nbat * ncols));
  w.clen = cv.take<int>(size_t(nbat * ncols));
  w.nbig = cv.take<int>(size_t(nbat));
  w.big = cv.take<int>(size_t(nbat * ncols));
  return w;
}

__global__ void zero_int_kernel(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Householder tridiagonalisation of the lower triangles of a batch of matrices (n x n,
// pitch lda, slice b at A + b sA) in place: every launch covers all slices (grid y), so a
// column's fixed launch and latency costs are paid once for the batch; d, e, tau and the
// reflectors (below the subdiagonal) land in each slice's loop block and matrix.
lrc_status tri_reduce(hipStream_t st, double* A, int64_t sA, int n, int64_t lda, int batch, const TWs& w) {
  const int64_t wsi = w.istride;
  // panels up to t0 (a multiple of NB), then the last n - t0 <= TT columns in one workgroup
  const int t0 = n <= TT ? 0 : int(cdiv(n - TT, NB) * NB);
  for (int i0 = 0; i0 < t0; i0 += NB) {
    const int pb = std::min(NB, n - 1 - i0);
    if (i0 == 0) {   // later panels are started by the previous panel's rank-2 update
      const unsigned g = unsigned(cdiv(n - i0, TS));
      tri_colstart_kernel<<<dim3(g, unsigned(batch)), 256, 0, st>>>(
          A, lda, n, i0, w.npart + (i0 & 1) * NPB * cdiv(n, TS), w.x0 + (i0 & 1), w.d, w.xv + (i0 & 1) * n, sA, wsi);
      LRC_LAUNCHED();
    }
    for (int jj = 0; jj < pb; ++jj) {
      const int i = i0 + jj;
      const int m = n - i - 1;
      const int nbt = int(cdiv(n - blk_origin(i + 1), TS));   // blocks from the aligned origin
      const int par = i & 1, npar = (i + 1) & 1;
      double* np_cur = w.npart + par * NPB * cdiv(n, TS);
      double* np_next = w.npart + npar * NPB * cdiv(n, TS);
      {
        ProfKernel pk("tri_symv_kernel", 2.0 * double(m) * double(m) * batch, 8.0 * double(m) * double(m + 1) / 2 * batch);
        // 16-byte pairs need an even matrix pitch and base; tiles start at 16-column
        // boundaries (rows and columns before s0 are masked)
        const double* xv = w.xv + par * n;
        // the tiles, then (inside the panel) one workgroup per row block for V^T x, W^T x
        const dim3 grid(unsigned(nbt * (nbt + 1) / 2 + (jj > 0 ? nbt : 0)), unsigned(batch));
        hipExtLaunchKernelGGL(tri_symv_kernel, grid, dim3(256), 0, st, pk.start, pk.stop, 0, (const double*)A, lda, n, i,
                              i0, jj, (const double*)w.Wp, xv, w.P, w.S, w.SV, w.SW, sA, wsi);
        LRC_LAUNCHED();
      }
      {
        // bytes: the symv partials, the panel rows of V and W, column i (and i+1) read and
        // written, the new column of W
        ProfKernel pk("tri_w_kernel", 4.0 * double(m) * (jj + 1) * batch,
                      8.0 * (double(nbt) * nbt * TS + 2.0 * double(m) * jj + 5.0 * double(m)) * batch);
        const int do_next = jj + 1 < pb ? 1 : 0;
        // columns i, i + 1 form an aligned pair when i is even
        hipExtLaunchKernelGGL(i % 2 == 0 ? tri_w_kernel<true> : tri_w_kernel<false>,
                              dim3(unsigned(WPB * nbt), unsigned(batch)), dim3(256), 0, st, pk.start, pk.stop, 0, A,
                              lda, n, i, i0, jj, do_next, w.Wp, (const double*)np_cur, (const double*)(w.x0 + par),
                              (const double*)w.P, (const double*)w.S, (const double*)w.SV, (const double*)w.SW,
                              np_next, w.x0 + npar, w.d, w.e, w.tau, w.xv + npar * n, sA, wsi);
        LRC_LAUNCHED();
      }
    }
    const int j1 = i0 + pb;
    if (j1 < n) {
      const int nt = int(cdiv(n - j1, TS));
      ProfScope scope("tri_syr2k_kernel", st, 2.0 * double(n - j1) * double(n - j1 + 1) * pb * batch, 0.0);
      // j1 is the next panel's first column (i0 + NB): its start-of-panel state goes to the
      // buffers of its parity
      tri_syr2k_kernel<<<dim3(unsigned(nt * (nt + 1) / 2), unsigned(batch)), 256, 0, st>>>(
          A, lda, n, i0, pb, j1, w.Wp, w.npart + (j1 & 1) * NPB * cdiv(n, TS), w.x0 + (j1 & 1), w.d,
          w.xv + (j1 & 1) * n, sA, wsi);
      LRC_LAUNCHED();
    }
  }
  tri_tail_kernel<<<dim3(1, unsigned(batch)), 256, 0, st>>>(A, lda, n, t0, w.d, w.e, w.tau, sA, wsi);
  LRC_LAUNCHED();
  return LRC_OK;
}

}  // namespace

size_t tridiag_workspace(int64_t k, int64_t ncols, int64_t batch) {
  Carve cv(nullptr);
  carve_tri(cv, k, std::max<int64_t>(ncols, 1), std::max<int64_t>(batch, 1));
  return cv.bytes();
}


// the back-transformation of the eigenvectors of every reduced slice of a batch (found by
// inverse iteration): slice b's reflectors in A + b sA, its scalars in its loop block,
// its eigenvectors of T and their pending scales in its blocks of w.Z / w.scl; every
// launch covers the batch (grid z or y)
static lrc_status tri_backtransform(hipStream_t st, double* A, int64_t sA, int n, int64_t lda, int ncols, int batch,
                                    const TWs& w, float* Qt, int64_t s_qt) {
  const int nref = n - 1;
  const int ngroups = int(cdiv(std::max(nref, 1), BW));
  const int ngc = int(cdiv(n, G_CHUNK));
  const int nbc = int(cdiv(n, BT_CHUNK));
  BtStrides bs;
  bs.a = sA;
  bs.wsi = w.istride;
  bs.gp = int64_t(ngroups) * ngc * BW * BW;
  bs.t = int64_t(ngroups) * BW * BW;
  bs.yp = int64_t(nbc) * BW * ncols;
  bs.y = int64_t(BW) * ncols;
  bs.z = int64_t(n) * ncols;
  bs.qt = s_qt;
  const unsigned nb = unsigned(batch);
  if (nref > 0) {
    bt_gram_kernel<<<dim3(unsigned(ngroups), unsigned(ngc), nb), 256, 0, st>>>(A, lda, n, nref, ngc, w.Gp, bs);
    LRC_LAUNCHED();
    bt_gsum_kernel<<<dim3(unsigned(BW * BW / 256), unsigned(ngroups), nb), 256, 0, st>>>(w.Gp, ngc, bs);
    LRC_LAUNCHED();
    bt_t_kernel<<<dim3(unsigned(ngroups), nb), BW, 0, st>>>(w.Gp, ngc, 1, nref, w.tau, w.T, bs);
    LRC_LAUNCHED();
    const unsigned ctiles = unsigned(cdiv(ncols, 64));
    for (int g = ngroups - 1; g >= 0; --g) {
      const int g0 = g * BW;
      const int rows = n - 1 - g0;
      const int nch = int(cdiv(rows, BT_CHUNK));
      const double fl = 2.0 * double(rows) * BW * double(ncols) * batch;
      {
        ProfScope scope("bt_vtz_kernel", st, fl, 0.0);
        bt_vtz_kernel<<<dim3(ctiles, unsigned(nch), nb), 256, 0, st>>>(A, lda, n, nref, g0, w.Z, ncols, w.Yp, bs);
        LRC_LAUNCHED();
      }
      bt_reduce_kernel<<<dim3(unsigned(cdiv(int64_t(BW) * ncols, 256)), nb), 256, 0, st>>>(w.Yp, nch, ncols, w.Yr,
                                                                                          bs);
      LRC_LAUNCHED();
      bt_ty_kernel<<<dim3(ctiles, BW / 16, nb), 256, 0, st>>>(w.Yr, w.T + int64_t(g) * BW * BW, ncols, w.Y2, bs);
      LRC_LAUNCHED();
      {
        ProfScope scope("bt_update_kernel", st, fl, 0.0);
        bt_update_kernel<<<dim3(unsigned(cdiv(rows, 64)), ctiles, nb), 256, 0, st>>>(A, lda, n, nref, g0, w.Y2,
                                                                                     ncols, w.Z, bs);
        LRC_LAUNCHED();
      }
    }
  }
  tri_out_kernel<<<dim3(unsigned(ncols), nb), 256, 0, st>>>(w.Z, w.scl, n, ncols, Qt, bs);
  LRC_LAUNCHED();
  return LRC_OK;
}

lrc_status tridiag_eig(hipStream_t st, double* A, int64_t sA, int64_t k, int64_t lda, int64_t ncols_in, int64_t batch,
                       float* sigma, int64_t s_sigma, float* Qt, int64_t s_qt, void* ws) {
  // the symv kernel reads 16-byte column pairs: even pitch, 16-byte base (every slice),
  // padding after an odd last column
  if (lda % 2 != 0 || (k % 2 != 0 && lda < k + 1) || reinterpret_cast<uintptr_t>(A) % 16 != 0 ||
      (batch > 1 && sA % 2 != 0) || batch < 1 || batch > 65535)
    return LRC_EINVAL;
  const int n = int(k);
  const int ncols = int(std::max<int64_t>(ncols_in, 1));
  Carve cv(ws);
  const TWs w0 = carve_tri(cv, n, ncols, batch);

  // 1. tridiagonalisation of every slice, one launch per step for the batch
  LRC_TRY(tri_reduce(st, A, sA, n, lda, int(batch), w0));

  // 2. all eigenvalues of every slice: one launch per kernel for the batch (each
  // slice's bisection is latency-bound on one wave per SIMD, so the slices run side by
  // side at the cost of one)
  const unsigned nb = unsigned(batch);
  tri_bounds_kernel<<<dim3(1, nb), 256, 0, st>>>(w0.d, w0.e, n, w0.bounds, w0.istride);
  LRC_LAUNCHED();
  {
    ProfScope scope("tri_bisect_kernel", st, 0.0, 0.0);
    tri_bisect_kernel<<<dim3(unsigned(cdiv(n, 16)), nb), 256, 0, st>>>(w0.d, w0.e, n, w0.bounds, w0.lam,
                                                                       w0.istride);
    LRC_LAUNCHED();
  }
  tri_sigma_kernel<<<dim3(unsigned(cdiv(n, 256)), nb), 256, 0, st>>>(w0.lam, n, sigma, s_sigma);
  LRC_LAUNCHED();

  // 3. clusters and inverse iteration for every slice at once (one wave per vector or
  // cluster, so the slices' latency-bound recurrences run side by side)
  zero_int_kernel<<<unsigned(cdiv(batch, 256)), 256, 0, st>>>(w0.nbig, int(batch));
  LRC_LAUNCHED();
  tri_cluster_kernel<<<dim3(unsigned(cdiv(ncols, 256)), nb), 256, 0, st>>>(w0.lam, n, ncols, w0.bounds, w0.clen,
                                                                          w0.nbig, w0.big);
  LRC_LAUNCHED();
  {
    ProfScope scope("tri_inviter_a_kernel", st, 0.0, 0.0);
    tri_inviter_a_kernel<<<dim3(unsigned(cdiv(ncols, 64)), nb), 64, 0, st>>>(w0.d, w0.e, n, w0.lam, ncols,
                                                                             w0.bounds, w0.clen, w0.U, w0.piv,
                                                                             w0.Z, w0.istride);
    LRC_LAUNCHED();
  }
  {
    // the solve and orthogonalisation launches together; clusters longer than CL_MAX
    // (at most ncols / (CL_MAX + 1) of them per slice) get a workgroup each
    ProfScope scope("tri_inviter_u_o_s_kernels", st, 0.0, 0.0);
    const int max_big = ncols / (CL_MAX + 1);
    tri_inviter_u_kernel<<<dim3(unsigned(ncols), nb), 64, 0, st>>>(n, ncols, w0.U, w0.Z, w0.nrm);
    LRC_LAUNCHED();
    for (int fin = 0; fin < 2; ++fin) {
      if (fin == 1) {
        tri_inviter_s_kernel<<<dim3(unsigned(ncols), nb), 64, 0, st>>>(n, ncols, w0.clen, w0.U, w0.piv, w0.Z,
                                                                       w0.nrm);
        LRC_LAUNCHED();
      }
      tri_inviter_o_kernel<<<dim3(unsigned(ncols), nb), 64, 0, st>>>(n, ncols, fin, w0.clen, w0.Z, w0.nrm, w0.scl);
      LRC_LAUNCHED();
      if (max_big > 0) {
        tri_inviter_obig_kernel<<<dim3(unsigned(max_big), nb), OB_T, 0, st>>>(n, ncols, fin, w0.clen, w0.nbig,
                                                                             w0.big, w0.Z, w0.scl);
        LRC_LAUNCHED();
      }
    }
  }

  // 4. the back-transformation of every slice, one launch per step for the batch
  LRC_TRY(tri_backtransform(st, A, sA, n, lda, ncols, int(batch), w0, Qt, s_qt));
  return LRC_OK;
}

}  // namespace lrc
