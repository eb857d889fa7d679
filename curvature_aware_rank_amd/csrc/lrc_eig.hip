// Symmetric eigensolver for the Gram of the whitened weight: two-sided block Jacobi in
// fp64 (Swift-SVD technical summary 2A: one eigendecomposition of the aggregated output
// covariance yields the singular values and vectors of the whitened weight).
//
// The k x k Gram (lower triangle stored) is padded to kp = multiple of 64 with
// decoupled diagonal entries -(trace + 1) (they stay exactly decoupled and sort last),
// cut into 32-wide blocks, and swept with a round-robin (circle) ordering of block pairs.
// Per round:
//   * one workgroup per pair loads the 64 x 64 pair block into LDS; if any entry is
//     above threshold it runs one cyclic Jacobi sweep on it (32 disjoint rotations per
//     step, the rotated 2 x 2 entries set exactly), accumulating the pair rotation J,
//     and orders the pair's eigenvalues descending (the larger half to the lower block:
//     fewer outer sweeps, and the blocks end up sorted);
//   * C <- J^T C J and V <- V J are applied tile by tile with fp64 MFMA
//     (v_mfma_f64_16x16x4f64); diagonal pair tiles take the pair solver's result, and
//     a pair that needed nothing contributes the identity.
// A sweep in which no pair needed a rotation ends the iteration; the host reads one
// counter per sweep.  Rotations are skipped when |a_pq| <= max(tol_r sqrt|a_pp a_qq|,
// floor_rel * trace), which bounds what is left off the diagonal.
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "lrc_dense.h"

namespace lrc {
namespace {

constexpr int JB = 32;       // block width
constexpr int PD = 2 * JB;   // pair dimension
constexpr int PP = PD + 1;   // LDS row pitch in doubles
constexpr double TOL_R_DEFAULT = 1e-10;
constexpr double FLOOR_REL_DEFAULT = 1e-12;
constexpr int MAX_SWEEPS = 40;

__device__ __forceinline__ int rr_pos(int pos, int r, int n) { return pos == 0 ? 0 : 1 + ((pos - 1 + r) % (n - 1)); }

__device__ __forceinline__ void pair_of(int pair, int r, int nb, int& p, int& q) {
  const int a = rr_pos(pair, r, nb), b = rr_pos(nb - 1 - pair, r, nb);
  p = min(a, b);
  q = max(a, b);
}

__device__ __forceinline__ int gidx(int i, int p, int q) { return i < JB ? p * JB + i : q * JB + (i - JB); }

// trace, pad value and rotation floor per batch item
__global__ void jacobi_scalars_kernel(const double* __restrict__ A, int k, int kp, int64_t sA, double* __restrict__ pad,
                                      double* __restrict__ floor_v, double floor_rel) {
  __shared__ double red[256];
  const double* a = A + blockIdx.x * sA;
  double s = 0.0;
  for (int i = threadIdx.x; i < k; i += 256) s += fabs(a[int64_t(i) * kp + i]);
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    pad[blockIdx.x] = -(red[0] + 1.0);
    floor_v[blockIdx.x] = floor_rel * red[0];
  }
}

// pad rows/cols beyond k and set V = I
__global__ void jacobi_init_kernel(double* __restrict__ A, double* __restrict__ V, int k, int kp, int64_t sA,
                                   const double* __restrict__ pad) {
  const int i = blockIdx.x;
  double* a = A + blockIdx.y * sA + int64_t(i) * kp;
  double* v = V + blockIdx.y * sA + int64_t(i) * kp;
  const double pv = pad[blockIdx.y];
  for (int j = threadIdx.x; j < kp; j += blockDim.x) {
    if (i >= k || j >= k) a[j] = (i == j) ? pv : 0.0;
    v[j] = (i == j) ? 1.0 : 0.0;
  }
}

__global__ void zero_i32_kernel(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ __launch_bounds__(256) void pair_eig_kernel(const double* __restrict__ Ad, int kp, int64_t sA, int nb,
                                                       int round, double* __restrict__ Jbuf, double* __restrict__ Sbuf,
                                                       int* __restrict__ changed, int* __restrict__ sweep_count,
                                                       const double* __restrict__ floors, double tol_r,
                                                       int max_inner) {
  __shared__ double S[PD][PP];
  __shared__ double J[PD][PP];
  __shared__ double rc[32], rs[32], rt[32], rapp[32], raqq[32], rapq[32];
  __shared__ int rp[32], rq[32], ract[32];
  __shared__ int nrot[2];
  __shared__ int perm[PD];
  const int pair = blockIdx.x, bt = blockIdx.y, tid = threadIdx.x;
  const int npairs = nb / 2;
  const double* A = Ad + bt * sA;
  int p, q;
  pair_of(pair, round, nb, p, q);
  // the pair block's lower triangle is stored (p < q keeps local and global order equal)
  for (int e = tid; e < PD * PD; e += 256) {
    const int i = e / PD, j = e % PD;
    if (i >= j) {
      const double v = A[int64_t(gidx(i, p, q)) * kp + gidx(j, p, q)];
      S[i][j] = v;
      S[j][i] = v;
    }
  }
  __syncthreads();
  const double floor_v = floors[bt];
  // nothing to do when every off-diagonal entry is below its threshold and the
  // diagonal is already descending
  int need = 0;
  for (int e = tid; e < PD * PD; e += 256) {
    const int i = e / PD, j = e % PD;
    if (i > j) need |= fabs(S[i][j]) > fmax(tol_r * sqrt(fabs(S[i][i] * S[j][j])), floor_v);
  }
  if (tid < PD - 1) need |= S[tid][tid] < S[tid + 1][tid + 1];
  need = __syncthreads_or(need);
  if (!need) {
    if (tid == 0) changed[bt * npairs + pair] = 0;
    return;
  }
  for (int e = tid; e < PD * PD; e += 256) J[e / PD][e % PD] = (e / PD == e % PD) ? 1.0 : 0.0;
  __syncthreads();
  // update role: wave wv owns rotations 8*wv .. 8*wv+7; lane = row / column index
  const int lane = tid & 63, wv = tid >> 6;
  for (int sw = 0; sw < max_inner; ++sw) {
    int sweep_rot = 0;
    for (int r = 0; r < PD - 1; ++r) {
      if (tid < 32) {
        const int a = rr_pos(tid, r, PD), c = rr_pos(PD - 1 - tid, r, PD);
        const int pi = min(a, c), qi = max(a, c);
        const double apq = S[pi][qi], app = S[pi][pi], aqq = S[qi][qi];
        const double thr = fmax(tol_r * sqrt(fabs(app * aqq)), floor_v);
        const bool act = fabs(apq) > thr;
        double t = 0.0, cc = 1.0, ss = 0.0;
        if (act) {
          const double tau = (aqq - app) / (2.0 * apq);
          t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
          cc = 1.0 / sqrt(1.0 + t * t);
          ss = t * cc;
        }
        rp[tid] = pi; rq[tid] = qi; rc[tid] = cc; rs[tid] = ss; rt[tid] = t;
        rapp[tid] = app; raqq[tid] = aqq; rapq[tid] = apq; ract[tid] = act ? 1 : 0;
        const unsigned long long bal = __ballot(act);
        if (tid == 0) nrot[r & 1] = __popcll(bal);
      }
      __syncthreads();
      const int nr = nrot[r & 1];
      if (nr == 0) continue;
      sweep_rot += nr;
      // rows p, q of S (lane = column)
      for (int u = 0; u < 8; ++u) {
        const int w = wv * 8 + u;
        if (!ract[w]) continue;
        const int pw = rp[w], qw = rq[w];
        const double cw = rc[w], sn = rs[w];
        const double sp = S[pw][lane], sq = S[qw][lane];
        S[pw][lane] = cw * sp - sn * sq;
        S[qw][lane] = sn * sp + cw * sq;
      }
      __syncthreads();
      // columns p, q of S and J (lane = row)
      for (int u = 0; u < 8; ++u) {
        const int w = wv * 8 + u;
        if (!ract[w]) continue;
        const int pw = rp[w], qw = rq[w];
        const double cw = rc[w], sn = rs[w];
        const double sp = S[lane][pw], sq = S[lane][qw];
        S[lane][pw] = cw * sp - sn * sq;
        S[lane][qw] = sn * sp + cw * sq;
        const double jp = J[lane][pw], jq = J[lane][qw];
        J[lane][pw] = cw * jp - sn * jq;
        J[lane][qw] = sn * jp + cw * jq;
      }
      __syncthreads();
      // the rotated 2x2 entries exactly (same wave computes the next round's rotations)
      if (tid < 32 && ract[tid]) {
        const int pi = rp[tid], qi = rq[tid];
        S[pi][qi] = 0.0;
        S[qi][pi] = 0.0;
        S[pi][pi] = rapp[tid] - rt[tid] * rapq[tid];
        S[qi][qi] = raqq[tid] + rt[tid] * rapq[tid];
      }
    }
    if (sweep_rot == 0) break;
  }
  __syncthreads();
  // eigenvalues of the pair descending: the larger half moves to the lower block index
  if (tid < PD) {
    const double di = S[tid][tid];
    int rank = 0;
    for (int j = 0; j < PD; ++j) {
      const double dj = S[j][j];
      rank += (dj > di) || (dj == di && j < tid);
    }
    perm[rank] = tid;
  }
  __syncthreads();
  const int64_t slot = (int64_t(bt) * npairs + pair) * (PD * PD);
  for (int e = tid; e < PD * PD; e += 256) {
    const int i = e / PD, j = e % PD;
    Jbuf[slot + e] = J[i][perm[j]];
    Sbuf[slot + e] = S[perm[i]][perm[j]];
  }
  if (tid == 0) {
    changed[bt * npairs + pair] = 1;
    atomicAdd(&sweep_count[bt], 1);
  }
}

// D(64x64) = op(X) * Y with X, Y in LDS (pitch PP).  transX: X element (i,k) read as X[k][i].
// Wave w computes the 32 x 32 quadrant (w>>1, w&1) as 2 x 2 blocks of 16 x 16.
// Fragment layout of v_mfma_f64_16x16x4f64 (checked on gfx950): A[i = l%16][k = l/16],
// B[k = l/16][j = l%16], element r of lane l = D[4*r + l/16][l%16] (unlike the fp32
// 16x16x4 form, whose element r sits in row 4*(l/16) + r).
template <bool TRANS_X>
__device__ __forceinline__ void mm64(const double (*X)[PP], const double (*Y)[PP], f64x4 (&acc)[2][2]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wi = w >> 1, wj = w & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
  for (int kq = 0; kq < PD; kq += 4) {
    const int kk = kq + (lane >> 4);
    double a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ii = wi * 32 + i * 16 + (lane & 15);
      a[i] = TRANS_X ? X[kk][ii] : X[ii][kk];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = Y[kk][wj * 32 + j * 16 + (lane & 15)];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

__device__ __forceinline__ void acc_to_lds(const f64x4 (&acc)[2][2], double (*D)[PP]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wi = w >> 1, wj = w & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) D[wi * 32 + i * 16 + 4 * r + (lane >> 4)][wj * 32 + j * 16 + (lane & 15)] = acc[i][j][r];
}

// Block (bp, bq) of the symmetric matrix whose lower triangle is stored: element (i, j)
// of a 32 x 32 sub-block lives at row max, column min of its global indices.  Sub-blocks
// of two different blocks are wholly above or below the diagonal, so each is read or
// written in one orientation with the contiguous index running fastest.
template <bool LOAD>
__device__ __forceinline__ void sym_tile_io(double* __restrict__ A, int kp, int p1, int p2, int q1, int q2,
                                            double (*T)[PP]) {
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    const int a = sb >> 1, b = sb & 1;
    const int bp = a ? p2 : p1, bq = b ? q2 : q1;
    const bool direct = bp > bq;
    for (int e = threadIdx.x; e < JB * JB; e += 256) {
      const int u = e / JB, v = e % JB;                 // v runs fastest
      const int i = direct ? u : v, j = direct ? v : u;   // local row in P, local col in Q
      const int gi = bp * JB + i, gj = bq * JB + j;
      double* cell = direct ? &A[int64_t(gi) * kp + gj] : &A[int64_t(gj) * kp + gi];
      if (LOAD) T[a * JB + i][b * JB + j] = *cell;
      else *cell = T[a * JB + i][b * JB + j];
    }
  }
}

__global__ __launch_bounds__(256) void jacobi_apply_kernel(double* __restrict__ Ad, double* __restrict__ Vd, int kp,
                                                           int64_t sA, int nb, int round,
                                                           const double* __restrict__ Jbuf,
                                                           const double* __restrict__ Sbuf,
                                                           const int* __restrict__ changed, int n_ctiles) {
  __shared__ double T0[PD][PP];
  __shared__ double T1[PD][PP];
  const int bt = blockIdx.y, tid = threadIdx.x;
  const int npairs = nb / 2;
  double* A = Ad + bt * sA;
  double* V = Vd + bt * sA;
  const int64_t jbase = int64_t(bt) * npairs * (PD * PD);
  int t = blockIdx.x;
  f64x4 acc[2][2];
  if (t < n_ctiles) {
    int P = 0;
    while (t > P) { t -= P + 1; ++P; }
    const int Q = t;
    const int chP = changed[bt * npairs + P], chQ = changed[bt * npairs + Q];
    if (!chP && !chQ) return;
    int p1, p2, q1, q2;
    pair_of(P, round, nb, p1, p2);
    pair_of(Q, round, nb, q1, q2);
    if (P == Q) {
      // the pair solver's rotated block; its lower triangle is stored
      const double* s = Sbuf + jbase + int64_t(P) * PD * PD;
      for (int e = tid; e < PD * PD; e += 256) {
        const int i = e / PD, j = e % PD;
        if (i >= j) A[int64_t(gidx(i, p1, p2)) * kp + gidx(j, p1, p2)] = s[e];
      }
      return;
    }
    sym_tile_io<true>(A, kp, p1, p2, q1, q2, T0);
    if (chQ) {
      const double* jq = Jbuf + jbase + int64_t(Q) * PD * PD;
      for (int e = tid; e < PD * PD; e += 256) T1[e / PD][e % PD] = jq[e];
      __syncthreads();
      mm64<false>(T0, T1, acc);   // C_PQ J_Q
      __syncthreads();
      acc_to_lds(acc, T0);
    }
    if (chP) {
      const double* jp = Jbuf + jbase + int64_t(P) * PD * PD;
      for (int e = tid; e < PD * PD; e += 256) T1[e / PD][e % PD] = jp[e];
      __syncthreads();
      mm64<true>(T1, T0, acc);    // J_P^T (C_PQ J_Q)
      __syncthreads();
      acc_to_lds(acc, T0);
    }
    __syncthreads();
    sym_tile_io<false>(A, kp, p1, p2, q1, q2, T0);
  } else {
    t -= n_ctiles;
    const int rb = t / npairs, Q = t % npairs;
    if (!changed[bt * npairs + Q]) return;
    int q1, q2;
    pair_of(Q, round, nb, q1, q2);
    const double* jq = Jbuf + jbase + int64_t(Q) * PD * PD;
    for (int e = tid; e < PD * PD; e += 256) {
      const int i = e / PD, j = e % PD;
      T0[i][j] = V[int64_t(rb * 64 + i) * kp + gidx(j, q1, q2)];
      T1[i][j] = jq[e];
    }
    __syncthreads();
    mm64<false>(T0, T1, acc);
    __syncthreads();
    acc_to_lds(acc, T0);
    __syncthreads();
    for (int e = tid; e < PD * PD; e += 256) {
      const int i = e / PD, j = e % PD;
      V[int64_t(rb * 64 + i) * kp + gidx(j, q1, q2)] = T0[i][j];
    }
  }
}

// diagonal -> dvec (all kp positions: the in-pair sorting moves the decoupled padding
// entries around, and they rank last because they are below every eigenvalue of the
// positive semi-definite Gram); rank descending, index breaks ties -> perm, sigma
__global__ void diag_kernel(const double* __restrict__ A, int kp, int64_t sA, double* __restrict__ dvec) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < kp) dvec[int64_t(blockIdx.y) * kp + i] = A[blockIdx.y * sA + int64_t(i) * kp + i];
}

__global__ void rank_kernel(const double* __restrict__ dvec, int k, int kp, int* __restrict__ perm,
                            float* __restrict__ sigma) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const double* d = dvec + int64_t(blockIdx.y) * kp;
  if (i >= kp) return;
  const double di = d[i];
  int rank = 0;
  for (int j = 0; j < kp; ++j) {
    const double dj = d[j];
    rank += (dj > di) || (dj == di && j < i);
  }
  if (rank < k) {
    perm[int64_t(blockIdx.y) * k + rank] = i;
    sigma[int64_t(blockIdx.y) * k + rank] = float(sqrt(fmax(di, 0.0)));
  }
}

__global__ void transpose_f64_kernel(const double* __restrict__ S, double* __restrict__ D, int n, int64_t sS) {
  __shared__ double t[32][33];
  const double* s = S + blockIdx.z * sS;
  double* d = D + blockIdx.z * sS;
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  for (int i = threadIdx.y; i < 32; i += 8) t[i][threadIdx.x] = s[int64_t(r0 + i) * n + c0 + threadIdx.x];
  __syncthreads();
  for (int i = threadIdx.y; i < 32; i += 8) d[int64_t(c0 + i) * n + r0 + threadIdx.x] = t[threadIdx.x][i];
}

// row c of Qt = eigenvector perm[c] (a row of V^T), sign-fixed, fp32
__global__ __launch_bounds__(256) void gather_sign_kernel(const double* __restrict__ VT, int k, int kp, int64_t sV,
                                                          const int* __restrict__ perm, float* __restrict__ Qt,
                                                          int ncols) {
  __shared__ double bv[256];
  __shared__ int bi[256];
  const int c = blockIdx.x, bt = blockIdx.y;
  const double* v = VT + bt * sV + int64_t(perm[int64_t(bt) * k + c]) * kp;
  double best = -1.0;
  int besti = 0x7fffffff;
  for (int j = threadIdx.x; j < k; j += 256) {
    const double a = fabs(v[j]);
    if (a > best) { best = a; besti = j; }   // j increases: the first maximum is kept
  }
  bv[threadIdx.x] = best;
  bi[threadIdx.x] = besti;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      const double ob = bv[threadIdx.x + o];
      const int oi = bi[threadIdx.x + o];
      if (ob > bv[threadIdx.x] || (ob == bv[threadIdx.x] && oi < bi[threadIdx.x])) {
        bv[threadIdx.x] = ob;
        bi[threadIdx.x] = oi;
      }
    }
    __syncthreads();
  }
  const double sgn = (v[bi[0]] < 0.0) ? -1.0 : 1.0;
  float* out = Qt + (int64_t(bt) * ncols + c) * k;
  for (int j = threadIdx.x; j < k; j += 256) out[j] = float(sgn * v[j]);
}

struct JWs {
  double *V, *J, *S, *pad, *floor_v, *dvec;
  int *changed, *count, *perm;
};

JWs carve_jacobi(Carve& cv, int64_t k, int64_t batch) {
  const int64_t kp = jacobi_padded(k);
  const int64_t npairs = kp / PD;
  JWs w;
  w.V = cv.take<double>(size_t(batch * kp * kp));
  w.J = cv.take<double>(size_t(batch * npairs * PD * PD));
  w.S = cv.take<double>(size_t(batch * npairs * PD * PD));
  w.pad = cv.take<double>(size_t(batch));
  w.floor_v = cv.take<double>(size_t(batch));
  w.dvec = cv.take<double>(size_t(batch * kp));
  w.changed = cv.take<int>(size_t(batch * npairs));
  w.count = cv.take<int>(size_t(batch));
  w.perm = cv.take<int>(size_t(batch * k));
  return w;
}

// tuning overrides (measurement only): LRC_JACOBI_TOL, LRC_JACOBI_FLOOR, LRC_JACOBI_INNER
double env_double(const char* name, double dflt) {
  const char* e = getenv(name);
  const double v = e ? atof(e) : 0.0;
  return v > 0.0 ? v : dflt;
}

int inner_sweeps() {
  const char* e = getenv("LRC_JACOBI_INNER");
  const int v = e ? atoi(e) : 0;
  return v > 0 ? v : 1;
}

}  // namespace

int64_t jacobi_padded(int64_t k) { return cdiv(k, PD) * PD; }

size_t jacobi_workspace(int64_t k, int64_t batch) {
  Carve cv(nullptr);
  carve_jacobi(cv, k, batch);
  return cv.bytes();
}

lrc_status jacobi_eig(hipStream_t st, double* A, int64_t k, int64_t batch, int64_t ncols, float* sigma, float* Qt,
                      int32_t* info, void* ws) {
  Carve cv(ws);
  JWs w = carve_jacobi(cv, k, batch);
  const int64_t kp = jacobi_padded(k);
  const int nb = int(kp / JB);
  const int npairs = nb / 2;
  const int64_t sA = kp * kp;
  const int n_ctiles = npairs * (npairs + 1) / 2;
  const int n_vtiles = int(kp / 64) * npairs;
  const int max_inner = inner_sweeps();
  const double tol_r = env_double("LRC_JACOBI_TOL", TOL_R_DEFAULT);
  const double floor_rel = env_double("LRC_JACOBI_FLOOR", FLOOR_REL_DEFAULT);
  const bool debug = getenv("LRC_DEBUG") != nullptr;

  jacobi_scalars_kernel<<<unsigned(batch), 256, 0, st>>>(A, int(k), int(kp), sA, w.pad, w.floor_v, floor_rel);
  LRC_LAUNCHED();
  jacobi_init_kernel<<<dim3(unsigned(kp), unsigned(batch)), 256, 0, st>>>(A, w.V, int(k), int(kp), sA, w.pad);
  LRC_LAUNCHED();

  std::vector<int> counts(size_t(batch), 0);
  bool converged = false;
  for (int sweep = 0; sweep < MAX_SWEEPS; ++sweep) {
    zero_i32_kernel<<<unsigned(cdiv(batch, 256)), 256, 0, st>>>(w.count, int(batch));
    LRC_LAUNCHED();
    for (int r = 0; r < nb - 1; ++r) {
      pair_eig_kernel<<<dim3(unsigned(npairs), unsigned(batch)), 256, 0, st>>>(A, int(kp), sA, nb, r, w.J, w.S,
                                                                              w.changed, w.count, w.floor_v, tol_r,
                                                                              max_inner);
      LRC_LAUNCHED();
      jacobi_apply_kernel<<<dim3(unsigned(n_ctiles + n_vtiles), unsigned(batch)), 256, 0, st>>>(
          A, w.V, int(kp), sA, nb, r, w.J, w.S, w.changed, n_ctiles);
      LRC_LAUNCHED();
    }
    LRC_HIP(hipMemcpyAsync(counts.data(), w.count, sizeof(int) * size_t(batch), hipMemcpyDeviceToHost, st));
    LRC_HIP(hipStreamSynchronize(st));
    bool any = false;
    for (int c : counts) any |= (c != 0);
    if (debug) fprintf(stderr, "lrc jacobi k=%lld sweep %d: pairs rotated %d (item 0)\n", (long long)k, sweep, counts[0]);
    if (!any) {
      converged = true;
      break;
    }
  }

  diag_kernel<<<dim3(unsigned(cdiv(kp, 256)), unsigned(batch)), 256, 0, st>>>(A, int(kp), sA, w.dvec);
  LRC_LAUNCHED();
  rank_kernel<<<dim3(unsigned(cdiv(kp, 256)), unsigned(batch)), 256, 0, st>>>(w.dvec, int(k), int(kp), w.perm,
                                                                            sigma);
  LRC_LAUNCHED();
  // V^T into A's storage (A is no longer needed)
  transpose_f64_kernel<<<dim3(unsigned(kp / 32), unsigned(kp / 32), unsigned(batch)), dim3(32, 8), 0, st>>>(w.V, A,
                                                                                                        int(kp), sA);
  LRC_LAUNCHED();
  gather_sign_kernel<<<dim3(unsigned(ncols), unsigned(batch)), 256, 0, st>>>(A, int(k), int(kp), sA, w.perm, Qt,
                                                                             int(ncols));
  LRC_LAUNCHED();
  if (!converged) {
    // mark every item that still rotated in the last sweep
    std::vector<int32_t> inf(size_t(batch), 0);
    for (int64_t b = 0; b < batch; ++b) inf[size_t(b)] = counts[size_t(b)] ? -1 : 0;
    LRC_HIP(hipMemcpyAsync(info, inf.data(), sizeof(int32_t) * size_t(batch), hipMemcpyHostToDevice, st));
    LRC_HIP(hipStreamSynchronize(st));
    return LRC_ENOCONV;
  }
  return LRC_OK;
}

}  // namespace lrc
