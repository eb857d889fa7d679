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
// A sweep in which no pair needed a rotation ends the iteration: a per-item flag set on
// the device at the end of that sweep turns every later launch for the item into an
// immediate return, so the host enqueues a fixed number of sweeps and never waits.  An
// item still rotating after the last sweep gets info = -1.  Rotations are skipped when
// |a_pq| <= max(tol_r sqrt|a_pp a_qq|, floor_rel * trace), which bounds what is left off
// the diagonal.
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
constexpr int MAX_SWEEPS = 40;   // sweeps enqueued per call (LRC_JACOBI_MAX_SWEEPS overrides, for tests)

// work counters, filled only while measurement is on (see lrc_profile_start)
enum : int { PROF_ROTATIONS, PROF_PAIRS_ACTIVE, PROF_V_TILES, PROF_C_TILES, PROF_C_PRODUCTS, PROF_C_DIAG, PROF_N };
// algorithmic work: a plane rotation of a pair block updates two rows and two columns of the
// 64 x 64 block and two columns of its 64 x 64 accumulated rotation, 3 flops per element
// (2 multiplies, 1 add); a 64 x 64 x 64 tile product is 2 * 64^3 flops
constexpr double FLOPS_PER_ROTATION = 3.0 * 2 * PD * 3;
constexpr double FLOPS_PER_TILE_PRODUCT = 2.0 * PD * PD * PD;
constexpr double TILE_BYTES = 8.0 * PD * PD;

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

// end of a sweep: an item whose sweep rotated nothing is done; the counters restart
__global__ void jacobi_sweep_end_kernel(int* __restrict__ count, int* __restrict__ done, int batch) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  if (count[b] == 0) done[b] = 1;
  count[b] = 0;
}

// after the last sweep: an item that never finished reports -1 (a Cholesky failure code
// already in info is kept)
__global__ void jacobi_info_kernel(const int* __restrict__ done, int32_t* __restrict__ info, int batch) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch && !done[b] && info[b] == 0) info[b] = -1;
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

struct PairScratch {
  double2 cs[32];            // cos, sin of the round's rotations (identity when inactive)
  int meta[32];              // p | q << 8 | active << 16
  uint16_t sched[PD - 1][32];  // round-robin schedule: p | q << 8 for each round and slot
  int nrot[2];
  int perm[PD];
};

// One pair of a round: load its 64 x 64 block, one cyclic Jacobi sweep if anything is
// above threshold, descending order; writes J, the rotated block and the changed flag.
__device__ __forceinline__ void pair_solve(double (*S)[PP], double (*J)[PP], PairScratch& ps,
                                           const double* __restrict__ Ad, int kp, int64_t sA, int nb, int round,
                                           int pair, double* __restrict__ Jbuf, double* __restrict__ Sbuf,
                                           int* __restrict__ changed, int* __restrict__ sweep_count,
                                           const double* __restrict__ floors, double tol_r, int max_inner,
                                           unsigned long long* __restrict__ prof) {
  int* nrot = ps.nrot; int* perm = ps.perm;
  const int bt = blockIdx.y, tid = threadIdx.x;
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
    if (i > j) {
      const double v = S[i][j];
      need |= (v * v > tol_r * tol_r * fabs(S[i][i] * S[j][j])) && (fabs(v) > floor_v);
    }
  }
  if (tid < PD - 1) need |= S[tid][tid] < S[tid + 1][tid + 1];
  need = __syncthreads_or(need);
  if (!need) {
    if (tid == 0) changed[bt * npairs + pair] = 0;
    return;
  }
  for (int e = tid; e < PD * PD; e += 256) J[e / PD][e % PD] = (e / PD == e % PD) ? 1.0 : 0.0;
  __syncthreads();
  for (int e = tid; e < (PD - 1) * 32; e += 256) {
    const int r = e / 32, i = e % 32;
    const int a = rr_pos(i, r, PD), c = rr_pos(PD - 1 - i, r, PD);
    ps.sched[r][i] = uint16_t(min(a, c) | (max(a, c) << 8));
  }
  __syncthreads();
  int total_rot = 0;
  for (int sw = 0; sw < max_inner; ++sw) {
    int sweep_rot = 0;
    for (int r = 0; r < PD - 1; ++r) {
      if (tid < 32) {
        const int pq = ps.sched[r][tid];
        const int pi = pq & 0xff, qi = pq >> 8;
        const double apq = S[pi][qi], app = S[pi][pi], aqq = S[qi][qi];
        // rotate when |a_pq| > max(tol_r sqrt|a_pp a_qq|, floor)  (squared, no sqrt)
        const bool act = (apq * apq > tol_r * tol_r * fabs(app * aqq)) && (fabs(apq) > floor_v);
        double cc = 1.0, ss = 0.0;
        if (act) {
          // tangent of the angle that zeroes a_pq, t = y sgn(x) / (|x| + sqrt(x^2 + y^2)) with
          // x = a_qq - a_pp, y = 2 a_pq: x and y are formed in fp64 and rescaled, the ratio
          // is taken in fp32 (t to ~1e-7 relative: the rotation then leaves a_pq ~1e-7 of
          // itself, removed by later sweeps); c = 1/sqrt(1+t^2) and s = t c are fp64, so the
          // rotation is orthogonal to fp64 precision and S, J stay consistent.
          const double x = aqq - app, y = 2.0 * apq;
          const double sc = __builtin_amdgcn_rcp(fmax(fabs(x), fabs(y)));
          const float xf = float(x * sc), yf = float(y * sc);
          const float tf = (xf >= 0.f ? yf : -yf) * __builtin_amdgcn_rcpf(fabsf(xf) + __builtin_amdgcn_sqrtf(xf * xf + yf * yf));
          const double t = double(tf);
          // v_rsq_f64 is an approximation: two Newton steps c <- c (3/2 - (u/2) c^2) square its
          // relative error twice, to fp64 rounding
          const double u = 1.0 + t * t, hu = 0.5 * u;
          double c0 = __builtin_amdgcn_rsq(u);
          c0 = c0 * fma(-hu * c0, c0, 1.5);
          c0 = c0 * fma(-hu * c0, c0, 1.5);
          cc = c0;
          ss = t * cc;
        }
        ps.cs[tid] = make_double2(cc, ss);
        ps.meta[tid] = pi | (qi << 8) | (act ? (1 << 16) : 0);
        const unsigned long long bal = __ballot(act);
        if (tid == 0) nrot[r & 1] = __popcll(bal);
      }
      __syncthreads();
      const int nr = nrot[r & 1];
      if (nr == 0) continue;
      sweep_rot += nr;
      // S <- R^T S R: a thread owns whole 2 x 2 groups (rows {p, q} of rotation w, columns
      // {p', q'} of rotation w2), so it reads, rotates on both sides and writes them back
      // with no barrier in between (the pair's own 2 x 2 block included).  Rotation w acts
      // as row p <- c p - s q, q <- s p + c q.
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int combo = tid + 256 * k;
        const int w = combo >> 5, w2 = combo & 31;
        const int m = ps.meta[w], m2 = ps.meta[w2];
        const bool a1 = (m >> 16) & 1, a2 = (m2 >> 16) & 1;
        if (!a1 && !a2) continue;
        const int p = m & 0xff, q = (m >> 8) & 0xff, p2 = m2 & 0xff, q2 = (m2 >> 8) & 0xff;
        const double2 r1 = ps.cs[w], r2 = ps.cs[w2];
        const double spp = S[p][p2], spq = S[p][q2], sqp = S[q][p2], sqq = S[q][q2];
        // rows
        const double tpp = r1.x * spp - r1.y * sqp, tqp = r1.y * spp + r1.x * sqp;
        const double tpq = r1.x * spq - r1.y * sqq, tqq = r1.y * spq + r1.x * sqq;
        // columns
        S[p][p2] = r2.x * tpp - r2.y * tpq;
        S[p][q2] = r2.y * tpp + r2.x * tpq;
        S[q][p2] = r2.x * tqp - r2.y * tqq;
        S[q][q2] = r2.y * tqp + r2.x * tqq;
      }
      // J <- J R (columns p, q; lane = row)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int item = tid + 256 * k;
        const int i = item & 63, w = item >> 6;
        const int m = ps.meta[w];
        if (!((m >> 16) & 1)) continue;
        const int p = m & 0xff, q = (m >> 8) & 0xff;
        const double2 r1 = ps.cs[w];
        const double jp = J[i][p], jq = J[i][q];
        J[i][p] = r1.x * jp - r1.y * jq;
        J[i][q] = r1.y * jp + r1.x * jq;
      }
      __syncthreads();
    }
    total_rot += sweep_rot;
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
    if (prof) {
      atomicAdd(&prof[PROF_ROTATIONS], (unsigned long long)total_rot);
      atomicAdd(&prof[PROF_PAIRS_ACTIVE], 1ull);
    }
  }
}

// V <- V J_Q for one 64-row block of V and one pair of a finished round
__device__ __forceinline__ void v_update(double (*T0)[PP], double (*T1)[PP], double* __restrict__ V, int kp, int nb,
                                         int round, int rb, int Q, const double* __restrict__ jq) {
  int q1, q2;
  pair_of(Q, round, nb, q1, q2);
  const int tid = threadIdx.x;
  for (int e = tid; e < PD * PD; e += 256) {
    const int i = e / PD, j = e % PD;
    T0[i][j] = V[int64_t(rb * 64 + i) * kp + gidx(j, q1, q2)];
    T1[i][j] = jq[e];
  }
  __syncthreads();
  f64x4 acc[2][2];
  mm64<false>(T0, T1, acc);
  __syncthreads();
  acc_to_lds(acc, T0);
  __syncthreads();
  for (int e = tid; e < PD * PD; e += 256) {
    const int i = e / PD, j = e % PD;
    V[int64_t(rb * 64 + i) * kp + gidx(j, q1, q2)] = T0[i][j];
  }
}

// Round g: workgroups [0, npair_wg) solve the pairs of round `round` (buffers *cur);
// the others apply round g-1's rotations to V (buffers *prev).  V is not read by the
// pair solves, so the V work of one round overlaps the pair solves of the next.
__global__ __launch_bounds__(256) void jacobi_pairs_v_kernel(
    const double* __restrict__ Ad, double* __restrict__ Vd, int kp, int64_t sA, int nb, int npair_wg, int round,
    double* __restrict__ Jcur, double* __restrict__ Scur, int* __restrict__ chcur, int prev_round,
    const double* __restrict__ Jprev, const int* __restrict__ chprev, int* __restrict__ sweep_count,
    const int* __restrict__ done, const double* __restrict__ floors, double tol_r, int max_inner,
    unsigned long long* __restrict__ prof) {
  __shared__ double L0[PD][PP];
  __shared__ double L1[PD][PP];
  __shared__ PairScratch ps;
  const int npairs = nb / 2, bt = blockIdx.y;
  const int t = blockIdx.x;
  if (done[bt]) return;   // converged in an earlier sweep: nothing rotates, nothing is pending
  if (t < npair_wg) {
    pair_solve(L0, L1, ps, Ad, kp, sA, nb, round, t, Jcur, Scur, chcur, sweep_count, floors, tol_r, max_inner,
               prof);
    return;
  }
  const int v = t - npair_wg;
  const int rb = v / npairs, Q = v % npairs;
  if (!chprev[bt * npairs + Q]) return;
  const double* jq = Jprev + (int64_t(bt) * npairs + Q) * (PD * PD);
  v_update(L0, L1, Vd + bt * sA, kp, nb, prev_round, rb, Q, jq);
  if (prof && threadIdx.x == 0) atomicAdd(&prof[PROF_V_TILES], 1ull);
}

// C <- J^T C J for the pair tiles (P >= Q) of a round
__global__ __launch_bounds__(256) void jacobi_apply_c_kernel(double* __restrict__ Ad, int kp, int64_t sA, int nb,
                                                             int round, const double* __restrict__ Jbuf,
                                                             const double* __restrict__ Sbuf,
                                                             const int* __restrict__ changed,
                                                             const int* __restrict__ done,
                                                             unsigned long long* __restrict__ prof) {
  __shared__ double T0[PD][PP];
  __shared__ double T1[PD][PP];
  const int bt = blockIdx.y, tid = threadIdx.x;
  if (done[bt]) return;
  const int npairs = nb / 2;
  double* A = Ad + bt * sA;
  const int64_t jbase = int64_t(bt) * npairs * (PD * PD);
  int t = blockIdx.x;
  f64x4 acc[2][2];
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
    const double* sb = Sbuf + jbase + int64_t(P) * PD * PD;
    for (int e = tid; e < PD * PD; e += 256) {
      const int i = e / PD, j = e % PD;
      if (i >= j) A[int64_t(gidx(i, p1, p2)) * kp + gidx(j, p1, p2)] = sb[e];
    }
    if (prof && tid == 0) atomicAdd(&prof[PROF_C_DIAG], 1ull);
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
  if (prof && tid == 0) {
    atomicAdd(&prof[PROF_C_TILES], 1ull);
    atomicAdd(&prof[PROF_C_PRODUCTS], (unsigned long long)(chP + chQ));
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
  // no entry compares above -1 only when every entry is NaN: the index stays in range
  const double sgn = (v[min(bi[0], k - 1)] < 0.0) ? -1.0 : 1.0;
  float* out = Qt + (int64_t(bt) * ncols + c) * k;
  for (int j = threadIdx.x; j < k; j += 256) out[j] = float(sgn * v[j]);
}

struct JWs {
  double *V, *J, *S, *pad, *floor_v, *dvec;
  int *changed, *count, *done, *perm;
  unsigned long long* prof;
};

JWs carve_jacobi(Carve& cv, int64_t k, int64_t batch) {
  const int64_t kp = jacobi_padded(k);
  const int64_t npairs = kp / PD;
  JWs w;
  w.V = cv.take<double>(size_t(batch * kp * kp));
  w.J = cv.take<double>(size_t(2 * batch * npairs * PD * PD));   // by round parity
  w.S = cv.take<double>(size_t(2 * batch * npairs * PD * PD));
  w.pad = cv.take<double>(size_t(batch));
  w.floor_v = cv.take<double>(size_t(batch));
  w.dvec = cv.take<double>(size_t(batch * kp));
  w.changed = cv.take<int>(size_t(2 * batch * npairs));
  w.count = cv.take<int>(size_t(batch));
  w.done = cv.take<int>(size_t(batch));
  w.perm = cv.take<int>(size_t(batch * k));
  w.prof = cv.take<unsigned long long>(PROF_N);
  return w;
}

// tuning overrides (measurement only): LRC_JACOBI_TOL, LRC_JACOBI_FLOOR, LRC_JACOBI_INNER
double env_double(const char* name, double dflt) {
  const char* e = getenv(name);
  const double v = e ? atof(e) : 0.0;
  return v > 0.0 ? v : dflt;
}

int max_sweeps() {
  const char* e = getenv("LRC_JACOBI_MAX_SWEEPS");
  const int v = e ? atoi(e) : 0;
  return v > 0 ? v : MAX_SWEEPS;
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
  const int n_sweeps = max_sweeps();

  const bool prof_on = prof_enabled();
  unsigned long long* prof = prof_on ? w.prof : nullptr;
  if (prof_on) {
    zero_i32_kernel<<<1, 256, 0, st>>>(reinterpret_cast<int*>(w.prof), 2 * PROF_N);
    LRC_LAUNCHED();
  }
  int64_t pair_wgs = 0;  // pair-solve workgroups launched (each reads its pair block)
  jacobi_scalars_kernel<<<unsigned(batch), 256, 0, st>>>(A, int(k), int(kp), sA, w.pad, w.floor_v, floor_rel);
  LRC_LAUNCHED();
  jacobi_init_kernel<<<dim3(unsigned(kp), unsigned(batch)), 256, 0, st>>>(A, w.V, int(k), int(kp), sA, w.pad);
  LRC_LAUNCHED();
  zero_i32_kernel<<<unsigned(cdiv(batch, 256)), 256, 0, st>>>(w.count, int(batch));
  LRC_LAUNCHED();
  zero_i32_kernel<<<unsigned(cdiv(batch, 256)), 256, 0, st>>>(w.done, int(batch));
  LRC_LAUNCHED();

  const size_t jslot = size_t(batch) * npairs * PD * PD;
  const size_t cslot = size_t(batch) * npairs;
  int64_t g = 0;            // rounds launched so far, over all sweeps
  int prev_round = 0;       // round-robin index of round g-1
  auto launch_pairs_v = [&](int npair_wg, int round) -> lrc_status {
    const int cur = int(g & 1), prv = int((g + 1) & 1);
    const int nv = g > 0 ? n_vtiles : 0;
    if (npair_wg + nv == 0) return LRC_OK;
    ProfScope scope("jacobi_pairs_v_kernel", st, 0.0, 0.0);  // work is counted on the device
    jacobi_pairs_v_kernel<<<dim3(unsigned(npair_wg + nv), unsigned(batch)), 256, 0, st>>>(
        A, w.V, int(kp), sA, nb, npair_wg, round, w.J + cur * jslot, w.S + cur * jslot, w.changed + cur * cslot,
        prev_round, w.J + prv * jslot, w.changed + prv * cslot, w.count, w.done, w.floor_v, tol_r, max_inner, prof);
    LRC_LAUNCHED();
    pair_wgs += int64_t(npair_wg) * batch;
    return LRC_OK;
  };
  // a fixed number of sweeps; items that finish early skip the rest on the device
  for (int sweep = 0; sweep < n_sweeps; ++sweep) {
    for (int r = 0; r < nb - 1; ++r) {
      LRC_TRY(launch_pairs_v(npairs, r));
      const int cur = int(g & 1);
      {
        ProfScope scope("jacobi_apply_c_kernel", st, 0.0, 0.0);
        jacobi_apply_c_kernel<<<dim3(unsigned(n_ctiles), unsigned(batch)), 256, 0, st>>>(
            A, int(kp), sA, nb, r, w.J + cur * jslot, w.S + cur * jslot, w.changed + cur * cslot, w.done, prof);
        LRC_LAUNCHED();
      }
      prev_round = r;
      ++g;
    }
    jacobi_sweep_end_kernel<<<unsigned(cdiv(batch, 256)), 256, 0, st>>>(w.count, w.done, int(batch));
    LRC_LAUNCHED();
  }
  // an item still rotating at the end has its last round's rotations pending for V
  LRC_TRY(launch_pairs_v(0, 0));

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
  jacobi_info_kernel<<<unsigned(cdiv(batch, 256)), 256, 0, st>>>(w.done, info, int(batch));
  LRC_LAUNCHED();
  if (prof_on) {
    // the measurement session only: the device-side work counters are read back
    unsigned long long c[PROF_N];
    LRC_HIP(hipMemcpyAsync(c, w.prof, sizeof(c), hipMemcpyDeviceToHost, st));
    LRC_HIP(hipStreamSynchronize(st));
    // pair solves read the lower half of their block; active ones write J and the block;
    // a V tile update reads V and J and writes V; a C tile is read and written, plus one J
    // per product; a diagonal pair block is copied from the solver's output
    const double lower_bytes = 8.0 * PD * (PD + 1) / 2;
    prof_add_work("jacobi_pairs_v_kernel",
                  double(c[PROF_ROTATIONS]) * FLOPS_PER_ROTATION + double(c[PROF_V_TILES]) * FLOPS_PER_TILE_PRODUCT,
                  double(pair_wgs) * lower_bytes + double(c[PROF_PAIRS_ACTIVE]) * 2 * TILE_BYTES +
                      double(c[PROF_V_TILES]) * 3 * TILE_BYTES);
    prof_add_work("jacobi_apply_c_kernel", double(c[PROF_C_PRODUCTS]) * FLOPS_PER_TILE_PRODUCT,
                  double(c[PROF_C_TILES]) * 2 * TILE_BYTES + double(c[PROF_C_PRODUCTS]) * TILE_BYTES +
                      double(c[PROF_C_DIAG]) * 2 * lower_bytes);
  }
  return LRC_OK;
}

}  // namespace lrc
