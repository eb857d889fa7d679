// Alternative component scores for the global allocator.
//
// UniRank technical summary 2.1 (Sorting-and-Truncation, "Aggregation and Truncation"):
// singular triplet i of matrix l scores I_l * sigma_{l,i}^2 / ||Sigma_l||_F^2, the layer's
// global functional importance times the triplet's share of the singular-value energy
// (local structural significance).
// Swift-SVD technical summary, section B (Dynamic Rank Allocation Strategy, "Hybrid
// Scoring"): layer l at rank k scores beta_l^alpha * log(e + eps*_{k,l})^(1 - alpha), with
// eps*_{k,l} = sum_{j > k} sigma_{l,j}^2 the energy the closed-form rank-k solution
// discards; entry k - 1 of the matrix's range holds the score at rank k.
//
// One workgroup per matrix.  Squared singular values and their sums are fp64; each thread
// sums a contiguous segment of the matrix in order, and the segment totals are combined
// in order (from the end for the discarded energies), so equal inputs give equal bits.
#include "lrc_internal.h"

namespace lrc {
namespace {

constexpr int RS_T = 256;

__global__ void zero_info_kernel(int32_t* __restrict__ info) { *info = 0; }

__global__ __launch_bounds__(RS_T) void rank_scores_kernel(const float* __restrict__ sigma,
                                                           const int64_t* __restrict__ offs, int n_mat, int64_t M,
                                                           const float* __restrict__ weight, double alpha, int swift,
                                                           float* __restrict__ scores, int32_t* __restrict__ info) {
  __shared__ double seg[RS_T];
  __shared__ double after[RS_T];
  __shared__ int bad;
  const int m = blockIdx.x, tid = threadIdx.x;
  const int64_t b = offs[m], e = offs[m + 1];
  const double w = double(weight[m]);
  if (tid == 0) {
    bad = 0;
    if (b < 0 || e < b || e > M || (m == 0 && b != 0) || (m == n_mat - 1 && e != M)) bad = int(LRC_EINVAL);
    else if (!isfinite(w)) bad = int(LRC_ENONFINITE);
    else if (w < 0.0 || (swift && w <= 0.0)) bad = int(LRC_EINVAL);
  }
  __syncthreads();
  if (bad) {
    if (tid == 0) atomicMax(info, bad);
    return;
  }
  const int64_t len = e - b;
  const int64_t sl = (len + RS_T - 1) / RS_T;
  const int64_t s0 = b + min<int64_t>(len, tid * sl), s1 = b + min<int64_t>(len, (tid + 1) * sl);
  double part = 0.0;
  bool nonfinite = false;
  for (int64_t j = s0; j < s1; ++j) {
    const float x = sigma[j];
    nonfinite |= !isfinite(x);
    part += double(x) * double(x);
  }
  seg[tid] = part;
  if (nonfinite) atomicMax(&bad, int(LRC_ENONFINITE));
  __syncthreads();
  if (bad) {
    if (tid == 0) atomicMax(info, bad);
    return;
  }
  if (!swift) {
    if (tid == 0) {
      double tot = 0.0;
      for (int t = 0; t < RS_T; ++t) tot += seg[t];
      after[0] = tot;
    }
    __syncthreads();
    const double tot = after[0];
    for (int64_t j = s0; j < s1; ++j) {
      const double x = double(sigma[j]);
      scores[j] = tot > 0.0 ? float(w * (x * x) / tot) : 0.f;
    }
    return;
  }
  // discarded energy after each segment, accumulated from the last segment backwards
  if (tid == 0) {
    double acc = 0.0;
    for (int t = RS_T - 1; t >= 0; --t) {
      after[t] = acc;
      acc += seg[t];
    }
  }
  __syncthreads();
  const double wa = pow(w, alpha);
  double acc = after[tid];
  for (int64_t j = s1 - 1; j >= s0; --j) {
    // rank (j - b + 1) keeps components b .. j and discards the rest
    scores[j] = float(wa * pow(log(M_E + acc), 1.0 - alpha));
    const double x = double(sigma[j]);
    acc += x * x;
  }
}

}  // namespace
}  // namespace lrc

using namespace lrc;

extern "C" lrc_status lrc_rank_scores(const float* sigma, const int64_t* offsets, int64_t n_mat, int64_t n_items,
                                      const float* weight, float alpha, uint32_t mode, float* scores, int32_t* info,
                                      void* stream) {
  if (mode != LRC_RANKSCORE_UNIRANK && mode != LRC_RANKSCORE_SWIFT) return LRC_EDTYPE;
  if (offsets == nullptr || weight == nullptr || info == nullptr) return LRC_EINVAL;
  if (n_mat <= 0 || n_mat > (int64_t(1) << 30) || n_items < 0) return LRC_EINVAL;
  if (n_items > 0 && (sigma == nullptr || scores == nullptr)) return LRC_EINVAL;
  if (mode == LRC_RANKSCORE_SWIFT && !(alpha >= 0.f && alpha <= 1.f)) return LRC_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  zero_info_kernel<<<1, 1, 0, st>>>(info);
  LRC_LAUNCHED();
  ProfScope scope("rank_scores_kernel", st, 0.0, 8.0 * double(n_items));
  rank_scores_kernel<<<unsigned(n_mat), RS_T, 0, st>>>(sigma, offsets, int(n_mat), n_items, weight, double(alpha),
                                                       mode == LRC_RANKSCORE_SWIFT ? 1 : 0, scores, info);
  LRC_LAUNCHED();
  return LRC_OK;
}
