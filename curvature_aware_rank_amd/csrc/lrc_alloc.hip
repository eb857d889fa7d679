// Global sort-and-truncate rank allocation.
//
// LASER technical summary, Methodology 2 (global optimisation: components are chosen
// greedily by importance per parameter cost until the target parameter budget is
// reached) and UniRank technical summary 2.1 (Aggregation and Truncation: every
// component of every matrix in one pool, sorted descending, accumulated while the
// parameter total stays within the budget; one component of an m x n matrix costs m+n).
//
// key_j = fp64(score_j) / fp64(cost_m) (IEEE).  For non-negative doubles the bit pattern
// is monotone, so ~bits sorted ascending is the descending key order.  An LSD radix sort
// with 8-bit digits and a stable scatter (ballot-matched ranks inside a wave, per-wave
// counts in LDS, waves and rounds in input order) keeps equal keys in input order, which
// is (matrix id, component index).  Then an int64 inclusive scan of the sorted costs and
// the longest prefix within the budget.
#include "lrc_internal.h"

namespace lrc {
namespace {

constexpr int RT = 256;        // threads per sort workgroup
constexpr int RR = 16;         // rounds per workgroup
constexpr int RTILE = RT * RR; // items per workgroup
constexpr int SC = 8;          // items per thread in the int64 scan
constexpr int STILE = 256 * SC;

__device__ __forceinline__ int matrix_of(const int64_t* __restrict__ offs, int n_mat, int64_t j) {
  int lo = 0, hi = n_mat - 1;   // largest m with offs[m] <= j
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offs[mid] <= j) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ void alloc_check_kernel(const int64_t* __restrict__ offs, const int64_t* __restrict__ cost, int n_mat,
                                   int64_t M, int32_t* __restrict__ info) {
  // one workgroup: offsets start at 0, end at M, never decrease; every cost is > 0
  __shared__ int bad;
  if (threadIdx.x == 0) bad = (offs[0] != 0 || offs[n_mat] != M) ? 1 : 0;
  __syncthreads();
  for (int m = threadIdx.x; m < n_mat; m += blockDim.x)
    if (offs[m + 1] < offs[m] || cost[m] <= 0) atomicOr(&bad, 1);
  __syncthreads();
  if (threadIdx.x == 0) *info = bad ? int32_t(LRC_EINVAL) : 0;
}

__global__ void key_kernel(const float* __restrict__ scores, const int64_t* __restrict__ offs,
                           const int64_t* __restrict__ cost, int n_mat, int M, uint64_t* __restrict__ keys,
                           uint32_t* __restrict__ vals, int32_t* __restrict__ info) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= M) return;
  vals[j] = uint32_t(j);   // always a valid permutation, whatever the checks find
  if (*info == int32_t(LRC_EINVAL)) {
    keys[j] = 0;
    return;
  }
  const float s = scores[j];
  if (!isfinite(s) || s < 0.f) {
    atomicExch(info, int32_t(LRC_ENONFINITE));
    keys[j] = 0;
    return;
  }
  const int m = matrix_of(offs, n_mat, j);
  const double key = (double(s) + 0.0) / double(cost[m]);   // +0.0 folds -0 into +0
  keys[j] = ~uint64_t(__double_as_longlong(key));
}

__global__ __launch_bounds__(RT) void radix_hist_kernel(const uint64_t* __restrict__ keys, int M, int shift,
                                                        uint32_t* __restrict__ hist, int nblk) {
  __shared__ uint32_t h[256];
  h[threadIdx.x] = 0;
  __syncthreads();
  const int64_t base = int64_t(blockIdx.x) * RTILE;
  for (int r = 0; r < RR; ++r) {
    const int64_t j = base + r * RT + threadIdx.x;
    if (j < M) atomicAdd(&h[(keys[j] >> shift) & 255u], 1u);
  }
  __syncthreads();
  hist[int64_t(threadIdx.x) * nblk + blockIdx.x] = h[threadIdx.x];
}

// exclusive scan of n uint32 values, one workgroup of 1024 threads
__global__ __launch_bounds__(1024) void scan_u32_kernel(uint32_t* __restrict__ a, int64_t n) {
  __shared__ uint32_t part[1024];
  const int64_t per = (n + 1023) / 1024;
  const int64_t b = threadIdx.x * per, e = min<int64_t>(n, b + per);
  uint32_t s = 0;
  for (int64_t i = b; i < e; ++i) s += a[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const uint32_t v = threadIdx.x >= o ? part[threadIdx.x - o] : 0u;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  uint32_t run = threadIdx.x ? part[threadIdx.x - 1] : 0u;
  for (int64_t i = b; i < e; ++i) {
    const uint32_t v = a[i];
    a[i] = run;
    run += v;
  }
}

__global__ __launch_bounds__(RT) void radix_scatter_kernel(const uint64_t* __restrict__ kin,
                                                           const uint32_t* __restrict__ vin,
                                                           uint64_t* __restrict__ kout, uint32_t* __restrict__ vout,
                                                           int M, int shift, const uint32_t* __restrict__ offs,
                                                           int nblk) {
  __shared__ uint32_t run[256];
  __shared__ uint32_t wcnt[4][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  run[tid] = offs[int64_t(tid) * nblk + blockIdx.x];
#pragma unroll
  for (int w = 0; w < 4; ++w) wcnt[w][tid] = 0;
  __syncthreads();
  const uint64_t lt = (uint64_t(1) << lane) - 1;
  const int64_t base = int64_t(blockIdx.x) * RTILE;
  for (int r = 0; r < RR; ++r) {
    const int64_t j = base + r * RT + tid;
    const bool valid = j < M;
    const uint64_t key = valid ? kin[j] : 0;
    const uint32_t d = uint32_t(key >> shift) & 255u;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool on = (d >> bit) & 1u;
      const uint64_t bal = __ballot(valid && on);
      peers &= on ? bal : ~bal;
    }
    const int rank = __popcll(peers & lt);
    if (valid && (peers & lt) == 0) wcnt[wave][d] = uint32_t(__popcll(peers));
    __syncthreads();
    if (valid) {
      uint32_t off = run[d] + uint32_t(rank);
      for (int w = 0; w < wave; ++w) off += wcnt[w][d];
      kout[off] = key;
      vout[off] = vin[j];
    }
    __syncthreads();
    run[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
#pragma unroll
    for (int w = 0; w < 4; ++w) wcnt[w][tid] = 0;
    __syncthreads();
  }
}

__global__ void gather_cost_kernel(const uint32_t* __restrict__ ids, const int64_t* __restrict__ offs,
                                   const int64_t* __restrict__ cost, int n_mat, int M, int64_t* __restrict__ cs,
                                   int32_t* __restrict__ order) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= M) return;
  const uint32_t id = ids[j];
  cs[j] = cost[matrix_of(offs, n_mat, id)];
  order[j] = int32_t(id);
}

__global__ __launch_bounds__(256) void scan_local_i64_kernel(int64_t* __restrict__ a, int M,
                                                             int64_t* __restrict__ bsum) {
  __shared__ int64_t part[256];
  const int64_t base = int64_t(blockIdx.x) * STILE + threadIdx.x * SC;
  int64_t v[SC];
  int64_t s = 0;
#pragma unroll
  for (int i = 0; i < SC; ++i) {
    const int64_t j = base + i;
    v[i] = j < M ? a[j] : 0;
    s += v[i];
    v[i] = s;
  }
  part[threadIdx.x] = s;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int64_t t = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += t;
    __syncthreads();
  }
  const int64_t pre = threadIdx.x ? part[threadIdx.x - 1] : 0;
#pragma unroll
  for (int i = 0; i < SC; ++i) {
    const int64_t j = base + i;
    if (j < M) a[j] = v[i] + pre;
  }
  if (threadIdx.x == 255) bsum[blockIdx.x] = part[255];
}

__global__ __launch_bounds__(1024) void scan_bsum_i64_kernel(int64_t* __restrict__ a, int n) {
  __shared__ int64_t part[1024];
  const int per = (n + 1023) / 1024;
  const int b = threadIdx.x * per, e = min(n, b + per);
  int64_t s = 0;
  for (int i = b; i < e; ++i) s += a[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int64_t v = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int64_t run = threadIdx.x ? part[threadIdx.x - 1] : 0;
  for (int i = b; i < e; ++i) {
    const int64_t v = a[i];
    a[i] = run;
    run += v;
  }
}

__global__ void scan_add_i64_kernel(int64_t* __restrict__ a, int M, const int64_t* __restrict__ bexcl) {
  const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j < M) a[j] += bexcl[j / STILE];
}

__global__ void cut_kernel(const int64_t* __restrict__ cum, int M, int64_t budget, int64_t* __restrict__ n_kept) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (M == 0) {
    if (j == 0) *n_kept = 0;
    return;
  }
  if (j >= M) return;
  const int64_t c = cum[j];
  if (j == 0 && c > budget) *n_kept = 0;
  if (c <= budget && (j == M - 1 || cum[j + 1] > budget)) *n_kept = int64_t(j) + 1;
}

__global__ void mask_kernel(const int32_t* __restrict__ order, int M, const int64_t* __restrict__ n_kept,
                            uint8_t* __restrict__ kept) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j < M) kept[order[j]] = (int64_t(j) < *n_kept) ? 1 : 0;
}

__global__ __launch_bounds__(256) void ranks_kernel(const uint8_t* __restrict__ kept, const int64_t* __restrict__ offs,
                                                    int64_t M, const int32_t* __restrict__ info,
                                                    int32_t* __restrict__ ranks) {
  __shared__ int red[256];
  const int m = blockIdx.x;
  int s = 0;
  if (*info != int32_t(LRC_EINVAL)) {   // offsets validated: every range lies inside [0, M)
    const int64_t b = max<int64_t>(0, offs[m]), e = min<int64_t>(M, offs[m + 1]);
    for (int64_t j = b + threadIdx.x; j < e; j += 256) s += kept[j];
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) ranks[m] = red[0];
}

struct AWs {
  uint64_t *ka, *kb;
  uint32_t *va, *vb, *hist;
  int64_t *cs, *bsum;
};

AWs carve_alloc(Carve& cv, int64_t M) {
  const int64_t nblk = std::max<int64_t>(1, cdiv(M, RTILE));
  const int64_t nsb = std::max<int64_t>(1, cdiv(M, STILE));
  AWs w;
  w.ka = cv.take<uint64_t>(size_t(std::max<int64_t>(M, 1)));
  w.kb = cv.take<uint64_t>(size_t(std::max<int64_t>(M, 1)));
  w.va = cv.take<uint32_t>(size_t(std::max<int64_t>(M, 1)));
  w.vb = cv.take<uint32_t>(size_t(std::max<int64_t>(M, 1)));
  w.hist = cv.take<uint32_t>(size_t(256 * nblk));
  w.cs = cv.take<int64_t>(size_t(std::max<int64_t>(M, 1)));
  w.bsum = cv.take<int64_t>(size_t(nsb));
  return w;
}

}  // namespace
}  // namespace lrc

using namespace lrc;

extern "C" size_t lrc_allocate_ranks_workspace(int64_t n_mat, int64_t n_items) {
  (void)n_mat;
  if (n_items < 0) return 0;
  Carve cv(nullptr);
  carve_alloc(cv, n_items);
  return cv.bytes();
}

extern "C" lrc_status lrc_allocate_ranks(const float* scores, const int64_t* offsets, const int64_t* cost,
                                         int64_t n_mat, int64_t n_items, int64_t budget, int32_t* order,
                                         int64_t* n_kept, int32_t* ranks, uint8_t* kept_mask, int32_t* info,
                                         void* ws, size_t ws_bytes, void* stream) {
  if (offsets == nullptr || cost == nullptr || n_kept == nullptr || ranks == nullptr || info == nullptr)
    return LRC_EINVAL;
  if (n_mat <= 0 || n_mat > (int64_t(1) << 30) || n_items < 0 || n_items >= (int64_t(1) << 31) || budget < 0)
    return LRC_EINVAL;
  if (n_items > 0 && (scores == nullptr || order == nullptr || kept_mask == nullptr)) return LRC_EINVAL;
  const size_t need = lrc_allocate_ranks_workspace(n_mat, n_items);
  if (ws == nullptr || ws_bytes < need) return LRC_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Carve cv(ws);
  AWs w = carve_alloc(cv, n_items);
  const int M = int(n_items);
  const int nm = int(n_mat);

  alloc_check_kernel<<<1, 256, 0, st>>>(offsets, cost, nm, n_items, info);
  LRC_LAUNCHED();
  if (M > 0) {
    const unsigned g = unsigned(cdiv(M, 256));
    key_kernel<<<g, 256, 0, st>>>(scores, offsets, cost, nm, M, w.ka, w.va, info);
    LRC_LAUNCHED();
    const int nblk = int(cdiv(M, RTILE));
    uint64_t *kin = w.ka, *kout = w.kb;
    uint32_t *vin = w.va, *vout = w.vb;
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = pass * 8;
      radix_hist_kernel<<<unsigned(nblk), RT, 0, st>>>(kin, M, shift, w.hist, nblk);
      LRC_LAUNCHED();
      scan_u32_kernel<<<1, 1024, 0, st>>>(w.hist, int64_t(256) * nblk);
      LRC_LAUNCHED();
      radix_scatter_kernel<<<unsigned(nblk), RT, 0, st>>>(kin, vin, kout, vout, M, shift, w.hist, nblk);
      LRC_LAUNCHED();
      std::swap(kin, kout);
      std::swap(vin, vout);
    }
    gather_cost_kernel<<<g, 256, 0, st>>>(vin, offsets, cost, nm, M, w.cs, order);
    LRC_LAUNCHED();
    const int nsb = int(cdiv(M, STILE));
    scan_local_i64_kernel<<<unsigned(nsb), 256, 0, st>>>(w.cs, M, w.bsum);
    LRC_LAUNCHED();
    scan_bsum_i64_kernel<<<1, 1024, 0, st>>>(w.bsum, nsb);
    LRC_LAUNCHED();
    scan_add_i64_kernel<<<g, 256, 0, st>>>(w.cs, M, w.bsum);
    LRC_LAUNCHED();
  }
  cut_kernel<<<unsigned(std::max<int64_t>(1, cdiv(M, 256))), 256, 0, st>>>(w.cs, M, budget, n_kept);
  LRC_LAUNCHED();
  if (M > 0) {
    mask_kernel<<<unsigned(cdiv(M, 256)), 256, 0, st>>>(order, M, n_kept, kept_mask);
    LRC_LAUNCHED();
  }
  ranks_kernel<<<unsigned(nm), 256, 0, st>>>(kept_mask, offsets, n_items, info, ranks);
  LRC_LAUNCHED();
  return LRC_OK;
}
