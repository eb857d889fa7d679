// Internal dense and eigensolver entry points (not part of the C ABI).
#pragma once
#include "lrc_internal.h"

namespace lrc {

// L = chol(lower(S)/cnt + damping*I), fp32, n x n with ld n, strict upper part zero.
// info (device int, must be 0 on entry) receives the 1-based failing pivot.
lrc_status cholesky_f32(hipStream_t st, const float* S, int64_t lds_, int64_t n, int64_t cnt, float damping,
                        float* L, int* info);
// The same for a batch: slice b factors S + b sS into L + b n n, its pivot in info + b sinfo
// (every info must be 0 on entry); each launch covers the batch.
lrc_status cholesky_f32_batched(hipStream_t st, const float* S, int64_t lds_, int64_t sS, int64_t n, int64_t cnt,
                                float damping, float* L, int* info, int sinfo, int64_t batch);

// Solve L^T Y = B in place (L lower n x n, ld n; B n x ncol, ld ldb).
lrc_status trsm_lower_t(hipStream_t st, const float* L, int64_t n, float* Bm, int64_t ldb, int64_t ncol);

// D (cols x rows) = S^T  (S rows x cols)
lrc_status transpose_f32(hipStream_t st, const float* S, int64_t lds_, float* D, int64_t ldd, int64_t rows,
                         int64_t cols);

// Symmetric eigendecomposition of batch fp64 k x k Grams held in A (kp x kp each,
// kp = jacobi_padded(k), Gram in the leading k x k block).  Workspace from `cv`.
// Outputs: lam (batch x k, descending, fp64 -> float sigma = sqrt(max(lam,0))) and
// Qt (batch x ncols x k, fp32): row c = eigenvector c, sign fixed so that its
// largest-magnitude entry (lowest index on ties) is positive.
// Enqueues a fixed number of sweeps (items that converge skip the rest on the device);
// an item still rotating after the last sweep gets info[b] = -1 (written on the device,
// unless info[b] already holds a nonzero code).
int64_t jacobi_padded(int64_t k);
size_t jacobi_workspace(int64_t k, int64_t batch);
lrc_status jacobi_eig(hipStream_t st, double* A, int64_t k, int64_t batch, int64_t ncols, float* sigma,
                      float* Qt, int32_t* info, void* ws);

// Symmetric eigendecompositions of a batch of fp64 k x k Grams (lower triangles of A,
// slice b at A + b sA, leading dimension lda; destroyed): Householder tridiagonalisation
// of all slices at once (every launch covers the batch), Sturm multisection for all
// eigenvalues of every slice (one launch for the batch), then per slice inverse iteration
// for the ncols largest and the blocked back-transformation.  Outputs as jacobi_eig: sigma slice b at sigma + b s_sigma, the
// eigenvectors (ncols x k rows) at Qt + b s_qt.  Enqueues a fixed amount of work and never
// waits.  A must be 16-byte aligned with an even lda and an even sA, and lda > k when k is
// odd (LRC_EINVAL otherwise).
size_t tridiag_workspace(int64_t k, int64_t ncols, int64_t batch);
lrc_status tridiag_eig(hipStream_t st, double* A, int64_t sA, int64_t k, int64_t lda, int64_t ncols, int64_t batch,
                       float* sigma, int64_t s_sigma, float* Qt, int64_t s_qt, void* ws);

}  // namespace lrc
