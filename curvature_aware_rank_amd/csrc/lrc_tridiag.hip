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
//   2. All eigenvalues of T by Sturm-count multisection (16 points per step, 14 steps).
//   3. Eigenvectors of the wanted (largest) eigenvalues by inverse iteration on T with
//      partial pivoting, one thread per vector; eigenvalues closer than 1e-7 ||T|| form a
//      cluster whose vectors one thread computes in turn, orthogonalised against each
//      other (modified Gram-Schmidt).  Clusters larger than 32 are reported to the caller,
//      which then uses the Jacobi solver.
//   4. Back-transformation Z <- Q Z in blocks of 128 reflectors, I - V T V^T (T from the
//      forward columnwise recurrence on V^T V).
// Every reduction has a fixed order, so equal inputs give equal bits.
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

#include "lrc_dense.h"

namespace lrc {
namespace {

constexpr int NB = 32;          // tridiagonalisation panel width
constexpr int TS = 64;          // tile and row-block size of the symv / w kernels
constexpr int BW = 128;         // reflectors per back-transformation block
constexpr int BT_CHUNK = 256;   // rows per partial of V^T Z
constexpr int G_CHUNK = 1024;   // rows per partial of V^T V
constexpr int BIS_PTS = 16;     // Sturm points per eigenvalue per multisection step
constexpr int BIS_ITERS = 14;   // 17^14 > 2^57: the interval shrinks below fp64 resolution
constexpr int BIS_STAGE = 2048; // d, e^2 staged through LDS in chunks of this many
constexpr int CL_MAX = 32;      // largest cluster inverse iteration handles
constexpr double CL_TOL = 1e-7; // eigenvalues closer than CL_TOL ||T|| share a cluster
constexpr int INV_ITERS = 3;    // inverse-iteration solves per vector
constexpr double EPS = 2.220446049250313e-16;

__device__ __forceinline__ void tile_of(int t, int& b, int& c) {
  // t = b (b + 1) / 2 + c, 0 <= c <= b
  int bb = int((sqrt(8.0 * double(t) + 1.0) - 1.0) * 0.5);
  while ((bb + 1) * (bb + 2) / 2 <= t) ++bb;
  while (bb * (bb + 1) / 2 > t) --bb;
  b = bb;
  c = t - bb * (bb + 1) / 2;
}

// Householder scalars of column i from its squared-norm partials (rows >= i + 2) and
// x0 = C[i+1][i]: H = I - tau v v^T, H x = beta e1, v = [1, x2 * scale].
__device__ __forceinline__ void house_scalars(const double* __restrict__ npart, int np, double x0, double& tau,
                                              double& beta, double& scale) {
  double xn2 = 0.0;
  for (int b = 0; b < np; ++b) xn2 += npart[b];
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

// ---- 1a. first column of a panel: d[i], x0, squared-norm partials (no deferred updates)
__global__ __launch_bounds__(256) void tri_colstart_kernel(const double* __restrict__ A, int64_t lda, int n, int i,
                                                           double* __restrict__ npart, double* __restrict__ x0,
                                                           double* __restrict__ d) {
  __shared__ double red[256];
  const int tid = threadIdx.x;
  const int r = i + blockIdx.x * TS + tid;
  double sq = 0.0;
  if (tid < TS && r < n) {
    const double val = A[int64_t(r) * lda + i];
    if (r == i) d[i] = val;
    if (r == i + 1) *x0 = val;
    if (r >= i + 2) sq = val * val;
  }
  const double s = block_sum256(sq, red);
  if (tid == 0) npart[blockIdx.x] = s;
}

// ---- 1b. symv over the trailing matrix (rows/cols i+1 .. n-1), one 64 x 64 lower tile
// per workgroup.  P[x][y][*]: contribution to y-block x from the tile pairing x and y.
__global__ __launch_bounds__(256) void tri_symv_kernel(const double* __restrict__ A, int64_t lda, int n, int i, int i0,
                                                       int jj, const double* __restrict__ Wp,
                                                       const double* __restrict__ npart, const double* __restrict__ x0p,
                                                       double* __restrict__ P, double* __restrict__ S,
                                                       double* __restrict__ SV, double* __restrict__ SW,
                                                       double* __restrict__ e, double* __restrict__ tau_out) {
  __shared__ double T[TS][TS + 1];
  __shared__ double vb[TS], vc[TS], rs[TS], cs[TS];
  __shared__ double red[8][2][NB];
  __shared__ double sc[3];
  const int tid = threadIdx.x;
  const int s0 = i + 1;
  const int m = n - s0;
  const int nbt = (m + TS - 1) / TS;
  int b, c;
  tile_of(blockIdx.x, b, c);
  if (tid == 0) {
    double tau, beta, scale;
    house_scalars(npart, (n - i + TS - 1) / TS, *x0p, tau, beta, scale);
    sc[0] = tau;
    sc[1] = beta;
    sc[2] = scale;
    if (blockIdx.x == 0) {
      e[i] = beta;
      tau_out[i] = tau;
    }
  }
  __syncthreads();
  const double scale = sc[2];
  const int R0 = s0 + b * TS, C0 = s0 + c * TS;
  if (tid < TS) {
    const int r = R0 + tid;
    vb[tid] = r >= n ? 0.0 : (r == s0 ? 1.0 : A[int64_t(r) * lda + i] * scale);
  } else if (tid < 2 * TS) {
    const int r = C0 + tid - TS;
    vc[tid - TS] = r >= n ? 0.0 : (r == s0 ? 1.0 : A[int64_t(r) * lda + i] * scale);
  }
  const bool diag = b == c;
  for (int q = tid; q < TS * TS; q += 256) {
    const int lr = q / TS, lc = q % TS;
    const int r = R0 + lr, cc = C0 + lc;
    const bool ok = r < n && cc < n && (!diag || lr >= lc);
    T[lr][lc] = ok ? A[int64_t(r) * lda + cc] : 0.0;
  }
  __syncthreads();
  {
    const int x = tid >> 2, part = tid & 3;
    double srow = 0.0, scol = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int q = part * 16 + j;
      srow += T[x][q] * vc[q];
      // column sums: strictly lower rows in a diagonal tile
      const double tv = (diag && q == x) ? 0.0 : T[q][x];
      scol += tv * vb[q];
    }
    srow += __shfl_xor(srow, 1);
    srow += __shfl_xor(srow, 2);
    scol += __shfl_xor(scol, 1);
    scol += __shfl_xor(scol, 2);
    if (part == 0) {
      rs[x] = srow;
      cs[x] = scol;
    }
  }
  __syncthreads();
  if (tid < TS) {
    if (diag) {
      P[(int64_t(b) * nbt + b) * TS + tid] = rs[tid] + cs[tid];
    } else {
      P[(int64_t(b) * nbt + c) * TS + tid] = rs[tid];
      P[(int64_t(c) * nbt + b) * TS + tid] = cs[tid];
    }
  }
  if (tid == 0) {
    double s = 0.0;
    if (diag) {
      for (int x = 0; x < TS; ++x) s += vb[x] * (rs[x] + cs[x]);
    } else {
      for (int x = 0; x < TS; ++x) s += vb[x] * rs[x];
      s *= 2.0;
    }
    S[blockIdx.x] = s;
  }
  if (diag && jj > 0) {
    // panel products over this row block: V^T v and W^T v
    const int cc = tid & 31, g = tid >> 5;
    double sv = 0.0, sw = 0.0;
    if (cc < jj) {
      for (int q = 0; q < 8; ++q) {
        const int x = g * 8 + q;
        const int r = R0 + x;
        if (r < n) {
          sv += A[int64_t(r) * lda + i0 + cc] * vb[x];
          sw += Wp[int64_t(r) * NB + cc] * vb[x];
        }
      }
    }
    red[g][0][cc] = sv;
    red[g][1][cc] = sw;
    __syncthreads();
    if (tid < jj) {
      double a0 = 0.0, a1 = 0.0;
      for (int q = 0; q < 8; ++q) {
        a0 += red[q][0][tid];
        a1 += red[q][1][tid];
      }
      SV[b * NB + tid] = a0;
      SW[b * NB + tid] = a1;
    }
  }
}

// y of trailing row r (block xb, local xl): partial sums, then the panel corrections
__device__ __forceinline__ double tri_yrow(const double* __restrict__ A, int64_t lda, int i0, int jj,
                                           const double* __restrict__ Wp, const double* __restrict__ P, int nbt,
                                           int r, int xb, int xl, const double* sv, const double* sw) {
  double y = 0.0;
  for (int c = 0; c < nbt; ++c) y += P[(int64_t(xb) * nbt + c) * TS + xl];
  double corr = 0.0;
  for (int c = 0; c < jj; ++c) corr += Wp[int64_t(r) * NB + c] * sv[c] + A[int64_t(r) * lda + i0 + c] * sw[c];
  return y - corr;
}

// ---- 1c. w = tau y + alpha v for one 64-row block of the trailing rows; store v and w;
// then bring column i+1 up to date with the panel's reflectors 0..jj (if it is in the panel)
__global__ __launch_bounds__(256) void tri_w_kernel(double* __restrict__ A, int64_t lda, int n, int i, int i0, int jj,
                                                    int do_next, double* __restrict__ Wp,
                                                    const double* __restrict__ npart, const double* __restrict__ x0p,
                                                    const double* __restrict__ P, const double* __restrict__ S,
                                                    const double* __restrict__ SV, const double* __restrict__ SW,
                                                    double* __restrict__ npart_next, double* __restrict__ x0_next,
                                                    double* __restrict__ d) {
  __shared__ double sv[NB], sw[NB], vrow[TS], wrow[TS];
  __shared__ double vn[NB + 1], wn[NB + 1];
  __shared__ double red[256];
  __shared__ double sc[4];
  const int tid = threadIdx.x;
  const int s0 = i + 1;
  const int m = n - s0;
  const int nbt = (m + TS - 1) / TS;
  const int ntile = nbt * (nbt + 1) / 2;
  const int b = blockIdx.x;
  const int R0 = s0 + b * TS;
  if (tid < jj) {
    double a0 = 0.0, a1 = 0.0;
    for (int q = 0; q < nbt; ++q) {
      a0 += SV[q * NB + tid];
      a1 += SW[q * NB + tid];
    }
    sv[tid] = a0;
    sw[tid] = a1;
  }
  // v^T C v: fixed-order sum of the tile partials
  double part = 0.0;
  for (int t = tid; t < ntile; t += 256) part += S[t];
  const double vav = block_sum256(part, red);   // (contains the barrier that publishes sv, sw)
  if (tid == 0) {
    double tau, beta, scale;
    house_scalars(npart, (n - i + TS - 1) / TS, *x0p, tau, beta, scale);
    double dsw = 0.0;
    for (int c = 0; c < jj; ++c) dsw += sv[c] * sw[c];
    const double yv = vav - 2.0 * dsw;
    sc[0] = tau;
    sc[1] = scale;
    sc[2] = -0.5 * tau * tau * yv;   // alpha
    // w of row s0 (needed by every block for the next column's update)
    const double y0 = tri_yrow(A, lda, i0, jj, Wp, P, nbt, s0, 0, 0, sv, sw);
    sc[3] = tau * y0 + sc[2];
  }
  __syncthreads();
  const double tau = sc[0], scale = sc[1], alpha = sc[2];
  if (tid < TS) {
    const int r = R0 + tid;
    if (r < n) {
      const double y = tri_yrow(A, lda, i0, jj, Wp, P, nbt, r, b, tid, sv, sw);
      const double v = r == s0 ? 1.0 : A[int64_t(r) * lda + i] * scale;
      const double w = tau * y + alpha * v;
      vrow[tid] = v;
      wrow[tid] = w;
    }
  }
  if (do_next && tid <= jj) {
    // row s0 of the panel's V and W, reflectors 0..jj
    vn[tid] = tid == jj ? 1.0 : A[int64_t(s0) * lda + i0 + tid];
    wn[tid] = tid == jj ? sc[3] : Wp[int64_t(s0) * NB + tid];
  }
  __syncthreads();
  if (tid < TS) {
    const int r = R0 + tid;
    if (r < n) {
      Wp[int64_t(r) * NB + jj] = wrow[tid];
      A[int64_t(r) * lda + i] = vrow[tid];
    }
  }
  if (!do_next) return;
  // column i' = s0: rows s0.., C[r][i'] -= sum_c V[r][c] W[i'][c] + W[r][c] V[i'][c]
  double sq = 0.0;
  if (tid < TS) {
    const int r = R0 + tid;
    if (r < n) {
      double corr = 0.0;
      for (int c = 0; c < jj; ++c)
        corr += A[int64_t(r) * lda + i0 + c] * wn[c] + Wp[int64_t(r) * NB + c] * vn[c];
      corr += vrow[tid] * wn[jj] + wrow[tid] * vn[jj];
      const double val = A[int64_t(r) * lda + s0] - corr;
      A[int64_t(r) * lda + s0] = val;
      if (r == s0) d[s0] = val;
      if (r == s0 + 1) *x0_next = val;
      if (r >= s0 + 2) sq = val * val;
    }
  }
  const double s = block_sum256(sq, red);
  if (tid == 0) npart_next[b] = s;
}

// ---- 1d. trailing rank-2 panel update, lower tiles of rows/cols j1 .. n-1:
// C -= V W^T + W V^T  (V rows in C's panel columns i0 .. i0+pb-1)
__global__ __launch_bounds__(256) void tri_syr2k_kernel(double* __restrict__ A, int64_t lda, int n, int i0, int pb,
                                                        int j1, const double* __restrict__ Wp) {
  __shared__ double Vr[TS][NB + 1], Wr[TS][NB + 1], Vc[TS][NB + 1], Wc[TS][NB + 1];
  const int tid = threadIdx.x;
  int b, c;
  tile_of(blockIdx.x, b, c);
  const int R0 = j1 + b * TS, C0 = j1 + c * TS;
  for (int q = tid; q < TS * NB; q += 256) {
    const int x = q / NB, t = q % NB;
    const int r = R0 + x, cc = C0 + x;
    const bool tr = t < pb;
    Vr[x][t] = (tr && r < n) ? A[int64_t(r) * lda + i0 + t] : 0.0;
    Wr[x][t] = (tr && r < n) ? Wp[int64_t(r) * NB + t] : 0.0;
    Vc[x][t] = (tr && cc < n) ? A[int64_t(cc) * lda + i0 + t] : 0.0;
    Wc[x][t] = (tr && cc < n) ? Wp[int64_t(cc) * NB + t] : 0.0;
  }
  __syncthreads();
  const int ty = tid >> 4, tx = tid & 15;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[a][q] = 0.0;
  for (int t = 0; t < NB; ++t) {
    double vr[4], wr[4], vc[4], wc[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      vr[a] = Vr[ty * 4 + a][t];
      wr[a] = Wr[ty * 4 + a][t];
      vc[a] = Vc[tx * 4 + a][t];
      wc[a] = Wc[tx * 4 + a][t];
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[a][q] += vr[a] * wc[q] + wr[a] * vc[q];
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int lr = ty * 4 + a, r = R0 + lr;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int lc = tx * 4 + q, cc = C0 + lc;
      if (r < n && cc < n && (b != c || lr >= lc)) A[int64_t(r) * lda + cc] -= acc[a][q];
    }
  }
}

// ---- 2. eigenvalues of T
// bounds: [0] gl, [1] gu, [2] pivmin, [3] ||T|| (max |Gershgorin end|)
__global__ __launch_bounds__(256) void tri_bounds_kernel(const double* __restrict__ d, const double* __restrict__ e,
                                                         int n, double* __restrict__ bounds) {
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

// 16 eigenvalues per workgroup, 16 Sturm points each; lam ascending
__global__ __launch_bounds__(256) void tri_bisect_kernel(const double* __restrict__ d, const double* __restrict__ e,
                                                         int n, const double* __restrict__ bounds,
                                                         double* __restrict__ lam) {
  __shared__ double sd[BIS_STAGE], se2[BIS_STAGE];
  const int tid = threadIdx.x;
  const int grp = tid >> 4, pt = tid & 15;
  const int mi = blockIdx.x * 16 + grp;   // ascending index
  const double pivmin = bounds[2];
  double lo = bounds[0], hi = bounds[1];
  for (int it = 0; it < BIS_ITERS; ++it) {
    const double x = lo + (hi - lo) * (double(pt + 1) / double(BIS_PTS + 1));
    int cnt = 0;
    double q = 1.0;
    for (int k0 = 0; k0 < n; k0 += BIS_STAGE) {
      const int kn = min(BIS_STAGE, n - k0);
      __syncthreads();
      for (int k = tid; k < kn; k += 256) {
        sd[k] = d[k0 + k];
        se2[k] = (k0 + k > 0) ? e[k0 + k - 1] * e[k0 + k - 1] : 0.0;
      }
      __syncthreads();
      for (int k = 0; k < kn; ++k) {
        q = (k0 + k == 0) ? sd[k] - x : (sd[k] - x) - se2[k] / q;
        if (fabs(q) < pivmin) q = -pivmin;
        cnt += q < 0.0;
      }
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

// ---- 3. clusters among the wanted eigenvalues (descending order j = 0 .. ncols-1)
__global__ void tri_cluster_kernel(const double* __restrict__ lam, int n, int ncols,
                                   const double* __restrict__ bounds, int* __restrict__ clen,
                                   int* __restrict__ flag) {
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
  if (len > CL_MAX) atomicMax(flag, len);
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

// one thread per cluster: LU (partial pivoting) of T - lambda I, INV_ITERS solves, MGS
// within the cluster; Z[k][j] (n x ncols) receives eigenvector j of T
__global__ __launch_bounds__(64) void tri_inviter_kernel(const double* __restrict__ d, const double* __restrict__ e,
                                                         int n, const double* __restrict__ lam, int ncols,
                                                         const double* __restrict__ bounds,
                                                         const int* __restrict__ clen, const int* __restrict__ flag,
                                                         double* __restrict__ U, uint8_t* __restrict__ piv,
                                                         double* __restrict__ Z) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= ncols || *flag) return;
  const int len = clen[j];
  if (len == 0) return;
  const double tnorm = bounds[3];
  const double tiny = EPS * tnorm;
  const int64_t nc = ncols;
  double* u0 = U;
  double* u1 = U + int64_t(n) * nc;
  double* u2 = U + 2 * int64_t(n) * nc;
  double* ml = U + 3 * int64_t(n) * nc;
  double lprev = 0.0;
  for (int q = 0; q < len; ++q) {
    const int jv = j + q;
    double lmb = lam[n - 1 - jv];
    if (q > 0) lmb = fmin(lmb, lprev - 10.0 * EPS * tnorm);
    lprev = lmb;
    // factor T - lmb I = P L U, U with two superdiagonals
    double cd = d[0] - lmb, cs = n > 1 ? e[0] : 0.0;
    for (int k = 0; k < n - 1; ++k) {
      const double sub = e[k];
      const double nd = d[k + 1] - lmb;
      const double ns = k + 1 < n - 1 ? e[k + 1] : 0.0;
      const int64_t o = int64_t(k) * nc + j;
      if (fabs(cd) >= fabs(sub)) {
        const double dd = cd == 0.0 ? tiny : cd;
        const double l = sub / dd;
        u0[o] = dd;
        u1[o] = cs;
        u2[o] = 0.0;
        ml[o] = l;
        piv[o] = 0;
        cd = nd - l * cs;
        cs = ns;
      } else {
        const double l = cd / sub;
        u0[o] = sub;
        u1[o] = nd;
        u2[o] = ns;
        ml[o] = l;
        piv[o] = 1;
        cd = cs - l * nd;
        cs = -l * ns;
      }
    }
    u0[int64_t(n - 1) * nc + j] = cd;
    u1[int64_t(n - 1) * nc + j] = 0.0;
    u2[int64_t(n - 1) * nc + j] = 0.0;
    double* z = Z + jv;
    for (int k = 0; k < n; ++k) z[int64_t(k) * nc] = start_value(jv, k);
    for (int it = 0; it < INV_ITERS; ++it) {
      // apply P and L^-1
      for (int k = 0; k < n - 1; ++k) {
        const int64_t o = int64_t(k) * nc + j;
        double yk = z[int64_t(k) * nc], yk1 = z[int64_t(k + 1) * nc];
        if (piv[o]) {
          const double t = yk;
          yk = yk1;
          yk1 = t;
        }
        z[int64_t(k) * nc] = yk;
        z[int64_t(k + 1) * nc] = yk1 - ml[o] * yk;
      }
      // back-substitution with U (tiny pivots replaced by +-tiny)
      double x1 = 0.0, x2 = 0.0;
      for (int k = n - 1; k >= 0; --k) {
        const int64_t o = int64_t(k) * nc + j;
        double p = u0[o];
        if (fabs(p) < tiny) p = p < 0.0 ? -tiny : tiny;
        const double xk = (z[int64_t(k) * nc] - u1[o] * x1 - u2[o] * x2) / p;
        z[int64_t(k) * nc] = xk;
        x2 = x1;
        x1 = xk;
      }
      // orthogonalise against the cluster's earlier vectors, normalise
      for (int p = 0; p < q; ++p) {
        const double* zp = Z + (j + p);
        double dot = 0.0;
        for (int k = 0; k < n; ++k) dot += zp[int64_t(k) * nc] * z[int64_t(k) * nc];
        for (int k = 0; k < n; ++k) z[int64_t(k) * nc] -= dot * zp[int64_t(k) * nc];
      }
      double mx = 0.0;
      for (int k = 0; k < n; ++k) mx = fmax(mx, fabs(z[int64_t(k) * nc]));
      const double inv_mx = mx > 0.0 ? 1.0 / mx : 1.0;
      double nrm2 = 0.0;
      for (int k = 0; k < n; ++k) {
        const double v = z[int64_t(k) * nc] * inv_mx;
        nrm2 += v * v;
      }
      const double sfac = inv_mx / sqrt(nrm2);
      for (int k = 0; k < n; ++k) z[int64_t(k) * nc] *= sfac;
    }
  }
}

// ---- 4. back-transformation.  Block g holds reflectors g*BW .. g*BW+BW-1; reflector t
// of the block lives in column g0 + t, rows > g0 + t.
__device__ __forceinline__ double refl(const double* __restrict__ A, int64_t lda, int nref, int g0, int r, int t) {
  return (g0 + t < nref && r > g0 + t) ? A[int64_t(r) * lda + g0 + t] : 0.0;
}

// partial V^T V of block g over one row chunk
__global__ __launch_bounds__(256) void bt_gram_kernel(const double* __restrict__ A, int64_t lda, int n, int nref,
                                                      int ngc, double* __restrict__ Gp) {
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

// T of block g (upper triangular): T[j][j] = tau_j, T[0:j, j] = -tau_j T[0:j,0:j] G[0:j, j];
// thread i owns row i of T (it alone writes and reads it)
__global__ __launch_bounds__(BW) void bt_t_kernel(const double* __restrict__ Gp, int ngc, int nref,
                                                  const double* __restrict__ tau, double* __restrict__ Tm) {
  __shared__ double G[BW][BW + 1];
  const int tid = threadIdx.x;
  const int g = blockIdx.x, g0 = g * BW;
  for (int q = tid; q < BW * BW; q += BW) {
    double s = 0.0;
    for (int ch = 0; ch < ngc; ++ch) s += Gp[(int64_t(g) * ngc + ch) * BW * BW + q];
    G[q / BW][q % BW] = s;
  }
  __syncthreads();
  double* T = Tm + int64_t(g) * BW * BW;
  const int i = tid;
  for (int jcol = 0; jcol < BW; ++jcol) {
    const double tj = g0 + jcol < nref ? tau[g0 + jcol] : 0.0;
    double v = 0.0;
    if (i < jcol) {
      double s = 0.0;
      for (int l = i; l < jcol; ++l) s += T[i * BW + l] * G[l][jcol];
      v = -tj * s;
    } else if (i == jcol) {
      v = tj;
    }
    T[i * BW + jcol] = v;
  }
}

// Yp[ch][a][c] = sum over the chunk's rows of V[r][a] Z[r][c]   (64 columns per workgroup)
__global__ __launch_bounds__(256) void bt_vtz_kernel(const double* __restrict__ A, int64_t lda, int n, int nref,
                                                     int g0, const double* __restrict__ Z, int ncols,
                                                     double* __restrict__ Yp) {
  __shared__ double sv[32][BW + 1];
  __shared__ double sz[32][64 + 1];
  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * 64, ch = blockIdx.y;
  const int rbase = g0 + 1 + ch * BT_CHUNK;
  const int rend = min(n, rbase + BT_CHUNK);
  const int ty = tid >> 4, tx = tid & 15;   // outputs a = ty*8 .. +7, c = tx*4 .. +3
  double acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[a][q] = 0.0;
  for (int rb = rbase; rb < rend; rb += 32) {
    __syncthreads();
    for (int q = tid; q < 32 * BW; q += 256) {
      const int x = q / BW, t = q % BW;
      const int r = rb + x;
      sv[x][t] = r < rend ? refl(A, lda, nref, g0, r, t) : 0.0;
    }
    for (int q = tid; q < 32 * 64; q += 256) {
      const int x = q / 64, cc = q % 64;
      const int r = rb + x;
      sz[x][cc] = (r < rend && c0 + cc < ncols) ? Z[int64_t(r) * ncols + c0 + cc] : 0.0;
    }
    __syncthreads();
    for (int x = 0; x < 32; ++x) {
      double a8[8], z4[4];
#pragma unroll
      for (int a = 0; a < 8; ++a) a8[a] = sv[x][ty * 8 + a];
#pragma unroll
      for (int q = 0; q < 4; ++q) z4[q] = sz[x][tx * 4 + q];
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[a][q] += a8[a] * z4[q];
    }
  }
  double* out = Yp + int64_t(ch) * BW * ncols;
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cc = c0 + tx * 4 + q;
      if (cc < ncols) out[int64_t(ty * 8 + a) * ncols + cc] = acc[a][q];
    }
}

// Y2 = T * sum_ch Yp[ch]   (64 columns per workgroup)
__global__ __launch_bounds__(256) void bt_ty_kernel(const double* __restrict__ Yp, int nch,
                                                    const double* __restrict__ T, int ncols,
                                                    double* __restrict__ Y2) {
  __shared__ double Y[BW][64 + 1];
  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * 64;
  for (int q = tid; q < BW * 64; q += 256) {
    const int a = q / 64, cc = q % 64;
    double s = 0.0;
    if (c0 + cc < ncols)
      for (int ch = 0; ch < nch; ++ch) s += Yp[(int64_t(ch) * BW + a) * ncols + c0 + cc];
    Y[a][cc] = s;
  }
  __syncthreads();
  const int ty = tid >> 4, tx = tid & 15;   // a = ty*8.., c = tx*4..
  double acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[a][q] = 0.0;
  for (int l = 0; l < BW; ++l) {
    double t8[8], y4[4];
#pragma unroll
    for (int a = 0; a < 8; ++a) t8[a] = T[(ty * 8 + a) * BW + l];
#pragma unroll
    for (int q = 0; q < 4; ++q) y4[q] = Y[l][tx * 4 + q];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[a][q] += t8[a] * y4[q];
  }
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cc = c0 + tx * 4 + q;
      if (cc < ncols) Y2[int64_t(ty * 8 + a) * ncols + cc] = acc[a][q];
    }
}

// Z[r][c] -= sum_a V[r][a] Y2[a][c]   (64 x 64 tile of rows g0+1.. per workgroup)
__global__ __launch_bounds__(256) void bt_update_kernel(const double* __restrict__ A, int64_t lda, int n, int nref,
                                                        int g0, const double* __restrict__ Y2, int ncols,
                                                        double* __restrict__ Z) {
  __shared__ double sv[64][32 + 1];
  __shared__ double sy[32][64 + 1];
  const int tid = threadIdx.x;
  const int r0 = g0 + 1 + blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int ty = tid >> 4, tx = tid & 15;   // rows ty*4.., cols tx*4..
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[a][q] = 0.0;
  for (int k0 = 0; k0 < BW; k0 += 32) {
    __syncthreads();
    for (int q = tid; q < 64 * 32; q += 256) {
      const int x = q / 32, t = q % 32;
      const int r = r0 + x;
      sv[x][t] = r < n ? refl(A, lda, nref, g0, r, k0 + t) : 0.0;
    }
    for (int q = tid; q < 32 * 64; q += 256) {
      const int t = q / 64, cc = q % 64;
      sy[t][cc] = c0 + cc < ncols ? Y2[int64_t(k0 + t) * ncols + c0 + cc] : 0.0;
    }
    __syncthreads();
    for (int t = 0; t < 32; ++t) {
      double v4[4], y4[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) v4[a] = sv[ty * 4 + a][t];
#pragma unroll
      for (int q = 0; q < 4; ++q) y4[q] = sy[t][tx * 4 + q];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[a][q] += v4[a] * y4[q];
    }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int r = r0 + ty * 4 + a;
    if (r >= n) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cc = c0 + tx * 4 + q;
      if (cc < ncols) Z[int64_t(r) * ncols + cc] -= acc[a][q];
    }
  }
}

// ---- outputs: sigma (all k, descending) and Qt rows = eigenvectors, sign-fixed, fp32
__global__ void tri_sigma_kernel(const double* __restrict__ lam, int n, float* __restrict__ sigma) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m < n) sigma[m] = float(sqrt(fmax(lam[n - 1 - m], 0.0)));
}

__global__ __launch_bounds__(256) void tri_out_kernel(const double* __restrict__ Z, int n, int ncols,
                                                      float* __restrict__ Qt) {
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
  const double sgn = Z[int64_t(bi[0]) * ncols + j] < 0.0 ? -1.0 : 1.0;
  for (int k = tid; k < n; k += 256) Qt[int64_t(j) * n + k] = float(sgn * Z[int64_t(k) * ncols + j]);
}

struct TWs {
  double *P, *S, *SV, *SW, *npart, *x0, *d, *e, *tau, *Wp, *lam, *bounds, *U, *Z, *Gp, *T, *Yp, *Y2;
  int *clen, *flag;
  uint8_t* piv;
};

TWs carve_tri(Carve& cv, int64_t n, int64_t ncols) {
  const int64_t nbt = cdiv(n, TS);
  const int64_t nref = std::max<int64_t>(n - 1, 0);
  const int64_t ngroups = std::max<int64_t>(cdiv(nref, BW), 1);
  const int64_t ngc = cdiv(n, G_CHUNK);
  const int64_t nbc = cdiv(n, BT_CHUNK);
  TWs w;
  w.P = cv.take<double>(size_t(nbt * nbt * TS));
  w.S = cv.take<double>(size_t(nbt * (nbt + 1) / 2));
  w.SV = cv.take<double>(size_t(nbt * NB));
  w.SW = cv.take<double>(size_t(nbt * NB));
  w.npart = cv.take<double>(size_t(2 * nbt));
  w.x0 = cv.take<double>(2);
  w.d = cv.take<double>(size_t(n));
  w.e = cv.take<double>(size_t(n));
  w.tau = cv.take<double>(size_t(n));
  w.Wp = cv.take<double>(size_t(n * NB));
  w.lam = cv.take<double>(size_t(n));
  w.bounds = cv.take<double>(4);
  w.U = cv.take<double>(size_t(4 * n * ncols));
  w.piv = cv.take<uint8_t>(size_t(n * ncols));
  w.Z = cv.take<double>(size_t(n * ncols));
  w.Gp = cv.take<double>(size_t(ngroups * ngc * BW * BW));
  w.T = cv.take<double>(size_t(ngroups * BW * BW));
  w.Yp = cv.take<double>(size_t(nbc * BW * ncols));
  w.Y2 = cv.take<double>(size_t(BW * ncols));
  w.clen = cv.take<int>(size_t(ncols));
  w.flag = cv.take<int>(1);
  return w;
}

__global__ void zero_int_kernel(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

size_t tridiag_workspace(int64_t k, int64_t ncols) {
  Carve cv(nullptr);
  carve_tri(cv, k, std::max<int64_t>(ncols, 1));
  return cv.bytes();
}

lrc_status tridiag_eig(hipStream_t st, double* A, int64_t k, int64_t lda, int64_t ncols_in, float* sigma, float* Qt,
                       void* ws, bool* clustered) {
  *clustered = false;
  const int n = int(k);
  const int ncols = int(std::max<int64_t>(ncols_in, 1));
  Carve cv(ws);
  TWs w = carve_tri(cv, n, ncols);

  // 1. tridiagonalisation
  for (int i0 = 0; i0 < n - 1; i0 += NB) {
    const int pb = std::min(NB, n - 1 - i0);
    {
      const unsigned g = unsigned(cdiv(n - i0, TS));
      tri_colstart_kernel<<<g, 256, 0, st>>>(A, lda, n, i0, w.npart + (i0 & 1) * cdiv(n, TS), w.x0 + (i0 & 1), w.d);
      LRC_LAUNCHED();
    }
    for (int jj = 0; jj < pb; ++jj) {
      const int i = i0 + jj;
      const int m = n - i - 1;
      const int nbt = int(cdiv(m, TS));
      const int par = i & 1, npar = (i + 1) & 1;
      double* np_cur = w.npart + par * cdiv(n, TS);
      double* np_next = w.npart + npar * cdiv(n, TS);
      {
        ProfScope scope("tri_symv_kernel", st, 2.0 * double(m) * double(m),
                        8.0 * double(m) * double(m + 1) / 2);
        tri_symv_kernel<<<unsigned(nbt * (nbt + 1) / 2), 256, 0, st>>>(A, lda, n, i, i0, jj, w.Wp, np_cur,
                                                                        w.x0 + par, w.P, w.S, w.SV, w.SW, w.e, w.tau);
        LRC_LAUNCHED();
      }
      tri_w_kernel<<<unsigned(nbt), 256, 0, st>>>(A, lda, n, i, i0, jj, jj + 1 < pb ? 1 : 0, w.Wp, np_cur,
                                                  w.x0 + par, w.P, w.S, w.SV, w.SW, np_next, w.x0 + npar, w.d);
      LRC_LAUNCHED();
    }
    const int j1 = i0 + pb;
    if (j1 < n) {
      const int nt = int(cdiv(n - j1, TS));
      ProfScope scope("tri_syr2k_kernel", st, 2.0 * double(n - j1) * double(n - j1 + 1) * pb, 0.0);
      tri_syr2k_kernel<<<unsigned(nt * (nt + 1) / 2), 256, 0, st>>>(A, lda, n, i0, pb, j1, w.Wp);
      LRC_LAUNCHED();
    }
  }
  {
    // last diagonal entry (and the whole job when n == 1)
    const int i = n - 1;
    tri_colstart_kernel<<<1, 256, 0, st>>>(A, lda, n, i, w.npart + (i & 1) * cdiv(n, TS), w.x0 + (i & 1), w.d);
    LRC_LAUNCHED();
  }

  // 2. eigenvalues
  tri_bounds_kernel<<<1, 256, 0, st>>>(w.d, w.e, n, w.bounds);
  LRC_LAUNCHED();
  {
    ProfScope scope("tri_bisect_kernel", st, 0.0, 0.0);
    tri_bisect_kernel<<<unsigned(cdiv(n, 16)), 256, 0, st>>>(w.d, w.e, n, w.bounds, w.lam);
    LRC_LAUNCHED();
  }
  tri_sigma_kernel<<<unsigned(cdiv(n, 256)), 256, 0, st>>>(w.lam, n, sigma);
  LRC_LAUNCHED();

  // 3. clusters and inverse iteration
  zero_int_kernel<<<1, 64, 0, st>>>(w.flag, 1);
  LRC_LAUNCHED();
  tri_cluster_kernel<<<unsigned(cdiv(ncols, 256)), 256, 0, st>>>(w.lam, n, ncols, w.bounds, w.clen, w.flag);
  LRC_LAUNCHED();
  int flag = 0;
  LRC_HIP(hipMemcpyAsync(&flag, w.flag, sizeof(int), hipMemcpyDeviceToHost, st));
  LRC_HIP(hipStreamSynchronize(st));
  if (flag) {
    *clustered = true;
    return LRC_OK;
  }
  {
    ProfScope scope("tri_inviter_kernel", st, 0.0, 0.0);
    tri_inviter_kernel<<<unsigned(cdiv(ncols, 64)), 64, 0, st>>>(w.d, w.e, n, w.lam, ncols, w.bounds, w.clen, w.flag,
                                                                 w.U, w.piv, w.Z);
    LRC_LAUNCHED();
  }

  // 4. back-transformation
  const int nref = n - 1;
  if (nref > 0) {
    const int ngroups = int(cdiv(nref, BW));
    const int ngc = int(cdiv(n, G_CHUNK));
    bt_gram_kernel<<<dim3(unsigned(ngroups), unsigned(ngc)), 256, 0, st>>>(A, lda, n, nref, ngc, w.Gp);
    LRC_LAUNCHED();
    bt_t_kernel<<<unsigned(ngroups), BW, 0, st>>>(w.Gp, ngc, nref, w.tau, w.T);
    LRC_LAUNCHED();
    const unsigned ctiles = unsigned(cdiv(ncols, 64));
    for (int g = ngroups - 1; g >= 0; --g) {
      const int g0 = g * BW;
      const int rows = n - 1 - g0;
      const int nch = int(cdiv(rows, BT_CHUNK));
      const double fl = 2.0 * double(rows) * BW * double(ncols);
      {
        ProfScope scope("bt_vtz_kernel", st, fl, 0.0);
        bt_vtz_kernel<<<dim3(ctiles, unsigned(nch)), 256, 0, st>>>(A, lda, n, nref, g0, w.Z, ncols, w.Yp);
        LRC_LAUNCHED();
      }
      bt_ty_kernel<<<ctiles, 256, 0, st>>>(w.Yp, nch, w.T + int64_t(g) * BW * BW, ncols, w.Y2);
      LRC_LAUNCHED();
      {
        ProfScope scope("bt_update_kernel", st, fl, 0.0);
        bt_update_kernel<<<dim3(unsigned(cdiv(rows, 64)), ctiles), 256, 0, st>>>(A, lda, n, nref, g0, w.Y2, ncols,
                                                                                 w.Z);
        LRC_LAUNCHED();
      }
    }
  }
  tri_out_kernel<<<unsigned(ncols), 256, 0, st>>>(w.Z, n, ncols, Qt);
  LRC_LAUNCHED();
  return LRC_OK;
}

}  // namespace lrc
