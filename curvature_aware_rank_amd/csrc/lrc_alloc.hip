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
// with 8-bit digits keeps equal keys in input order, which is (matrix id, component
// index).  Each pass: per-workgroup digit counts, a scan per digit row, and a stable
// scatter that ranks a tile per wave (ballot-matched equal digits, waves and rounds in
// input order), stages it in LDS in digit order and writes contiguous runs.  The cut
// sums the sorted costs per block of positions (int64, exact), finds the block where the
// running total first exceeds the budget, and resolves the position inside it; the mask
// is then written in item order by comparing each item's (key, id) with that of the first
// excluded item.  Matrix costs are looked up per 4096-item bucket.
//
// A caller that needs no order gets the same cut without sorting: the first excluded item
// E is found by a radix select weighted by cost.  Level 0 sums the costs of every item per
// top 8-bit digit of its key bits; the digit whose bucket carries the running total past
// the budget is fixed, the cost of every lower bucket is carried, and the next level sums
// the next 8 bits over the items of that bucket only.  After eight levels the bucket holds
// the items whose key equals E's; among them E is the first, in id order, at which the
// running total exceeds the budget, found by four more such levels over the 32-bit id.
// Only the first three levels read every key; the third also lists the items of its
// bucket, and the later levels read only that list.
#include <mutex>

#include "lrc_internal.h"

// ---- scratch of the allocation-free variant (lrc_allocate_ranks_noalloc): one array per
// GPU, held until the process ends.  carve_alloc at NOALLOC_MAX_ITEMS needs 24 B per item
// (two key and two id buffers) plus about 1.6 MB of histogram, lookup, cut and select
// tables; the entry point checks the carve against the array's size at run time.
constexpr int64_t NOALLOC_MAX_ITEMS = int64_t(1) << 21;
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(24) * NOALLOC_MAX_ITEMS + (size_t(2) << 20);
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace lrc {
namespace {

constexpr int RT = 256;        // threads per sort workgroup (4 waves)
// items per thread (each wave: RR rounds of 64 consecutive items) and per tile: 16 (4096-item
// tiles) for large pools, 4 (1024-item tiles) when 4096-item tiles would give fewer than two
// workgroups per compute unit -- more, shorter workgroups at small sizes
constexpr int RR_BIG = 16, RR_SMALL = 4;
constexpr int MAX_SORT_BLOCKS = 4096;   // sort workgroups per pass; each takes a run of tiles
constexpr int SC = 8;          // items per thread in the int64 scan
constexpr int STILE = 256 * SC;
constexpr int MB_SHIFT = 12;   // item ids per bucket of the matrix lookup table (log2)

__device__ __forceinline__ int matrix_of(const int64_t* __restrict__ offs, int n_mat, int64_t j) {
  int lo = 0, hi = n_mat - 1;   // largest m with offs[m] <= j
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offs[mid] <= j) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// mtab[b] = matrix of item b << MB_SHIFT (n_mat - 1 past the end), so that the matrix
// of item j lies in [mtab[j >> MB_SHIFT], mtab[(j >> MB_SHIFT) + 1]];
// ctab[b] = the cost of bucket b's items when they all belong to one matrix, else -1
__global__ void mtab_kernel(const int64_t* __restrict__ offs, const int64_t* __restrict__ cost, int n_mat,
                            int64_t M, int nbk, int32_t* __restrict__ mtab, int64_t* __restrict__ ctab) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b > nbk) return;
  const int64_t j = int64_t(b) << MB_SHIFT;
  const int m0 = j < M ? matrix_of(offs, n_mat, j) : n_mat - 1;
  mtab[b] = m0;
  if (b < nbk) {
    const int m1 = matrix_of(offs, n_mat, min<int64_t>(j + (1 << MB_SHIFT), M) - 1);
    ctab[b] = m0 == m1 ? cost[m0] : -1;
  }
}

__device__ __forceinline__ int matrix_of_item(const int64_t* __restrict__ offs, const int32_t* __restrict__ mtab,
                                              int64_t j) {
  const int64_t b = j >> MB_SHIFT;
  int lo = mtab[b], hi = mtab[b + 1];
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offs[mid] <= j) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// an id read back from the sorted order, kept inside [0, M) so that a lookup can never
// leave the tables (the sort writes a permutation; this only guards the reads)
__device__ __forceinline__ int32_t order_id(const int32_t* __restrict__ order, int64_t p, int M) {
  const int32_t id = order[p];
  return id < 0 ? 0 : (id >= M ? M - 1 : id);
}

// Tables of the item -> matrix -> cost lookup
struct CostLookup {
  const int64_t* offs;
  const int32_t* mtab;
  const int64_t* ctab;
  const int64_t* cost;
  __device__ __forceinline__ int64_t operator()(int64_t j) const {
    const int64_t c = ctab[j >> MB_SHIFT];
    return c >= 0 ? c : cost[matrix_of_item(offs, mtab, j)];
  }
};

// sort key of a score at a cost: ~bits(fp64(score) / fp64(cost)); 0 (first in the order)
// for a NaN, infinite or negative score, whose call reports an error and keeps nothing
__device__ __forceinline__ uint64_t score_key(float sc, int64_t c, bool& nonfinite) {
  nonfinite = false;
  if (!isfinite(sc) || sc < 0.f) {
    nonfinite = true;
    return 0;
  }
  const double key = (double(sc) + 0.0) / double(c);   // +0.0: -0 -> +0
  return ~uint64_t(__double_as_longlong(key));
}

// sort key of item j (0 for every item when the offsets or costs were rejected)
__device__ __forceinline__ uint64_t item_key(const float* __restrict__ scores, const CostLookup& cl, int64_t j,
                                             bool inputs_bad, bool& nonfinite) {
  nonfinite = false;
  if (inputs_bad) return 0;
  return score_key(scores[j], cl(j), nonfinite);
}

// argument checks on the device, in two launches: the offsets start at 0 and end at M
// (info = 0 or LRC_EINVAL), then one thread per matrix: offsets never decrease and every
// cost is > 0 (a wave that finds a failure sets LRC_EINVAL once)
__global__ void alloc_check_ends_kernel(const int64_t* __restrict__ offs, int n_mat, int64_t M,
                                        int32_t* __restrict__ info) {
  *info = (offs[0] != 0 || offs[n_mat] != M) ? int32_t(LRC_EINVAL) : 0;
}
__global__ __launch_bounds__(256) void alloc_check_kernel(const int64_t* __restrict__ offs,
                                                          const int64_t* __restrict__ cost, int n_mat,
                                                          int32_t* __restrict__ info) {
  const int64_t m = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const bool bad = m < n_mat && (offs[m + 1] < offs[m] || cost[m] <= 0);
  if (__ballot(bad) != 0 && (threadIdx.x & 63) == 0) atomicExch(info, int32_t(LRC_EINVAL));
}

// KEY_PER items per workgroup, consecutive lanes on consecutive items
constexpr int KEY_PER = 256 * 8;
__global__ __launch_bounds__(256) void key_kernel(const float* __restrict__ scores, CostLookup cl, int M,
                                                  uint64_t* __restrict__ keys, uint32_t* __restrict__ vals,
                                                  int32_t* __restrict__ info) {
  const bool bad = *info == int32_t(LRC_EINVAL);
  const int64_t base = int64_t(blockIdx.x) * KEY_PER;
  bool any_nf = false;
#pragma unroll
  for (int i = 0; i < KEY_PER / 256; ++i) {
    const int64_t j = base + i * 256 + int(threadIdx.x);
    if (j < M) {
      vals[j] = uint32_t(j);   // always a valid permutation, whatever the checks find
      bool nf;
      keys[j] = item_key(scores, cl, j, bad, nf);
      any_nf |= nf;
    }
  }
  if (any_nf) atomicExch(info, int32_t(LRC_ENONFINITE));
}

// Stable ranking of one wave's items by 8-bit digit: lanes whose digits are equal are
// found with eight ballots; `below` is the number of such lanes with a lower lane index.
__device__ __forceinline__ uint64_t digit_peers(uint32_t d, bool valid) {
  uint64_t peers = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const bool on = (d >> bit) & 1u;
    const uint64_t bal = __ballot(valid && on);
    peers &= on ? bal : ~bal;
  }
  return peers;
}

// exclusive scan of one value per thread over a 256-thread workgroup (4 waves)
__device__ __forceinline__ uint32_t block_exscan256(uint32_t v, uint32_t* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t pre = 0;
  for (int w = 0; w < wave; ++w) pre += wsum[w];
  __syncthreads();
  return pre + inc - v;
}

// Digit counts of each sort block's run of tiles, digit-major: cnt[d * nblk + block].
// Block b takes tiles [b * tpb, min((b + 1) * tpb, ntiles)); wave w of a tile owns its
// contiguous items [w * RR * 64, (w + 1) * RR * 64).
template <int RR>
__global__ __launch_bounds__(RT) void radix_hist_kernel(const uint64_t* __restrict__ keys, int M, int shift,
                                                        int tpb, uint32_t* __restrict__ cnt, int nblk) {
  constexpr int RTILE = RT * RR;
  __shared__ uint32_t h[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  h[tid] = 0;
  __syncthreads();
  const uint64_t lt = (uint64_t(1) << lane) - 1;
  const int64_t t_end = min<int64_t>(int64_t(blockIdx.x + 1) * tpb, (int64_t(M) + RTILE - 1) / RTILE);
  for (int64_t t = int64_t(blockIdx.x) * tpb; t < t_end; ++t) {
    const int64_t base = t * RTILE + int64_t(wave) * (RR * 64);
    uint64_t k[RR];
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      const int64_t j = min<int64_t>(base + r * 64 + lane, M - 1);
      k[r] = keys[j];
    }
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      const bool valid = base + r * 64 + lane < M;
      const uint32_t d = uint32_t(k[r] >> shift) & 255u;
      const uint64_t peers = digit_peers(d, valid);
      if (valid && (peers & lt) == 0) atomicAdd(&h[d], uint32_t(__popcll(peers)));
    }
  }
  __syncthreads();
  cnt[int64_t(tid) * nblk + blockIdx.x] = h[tid];
}

// In-place exclusive scan of each digit row cnt[d * nblk .. + nblk); rowtot[d] = row sum.
// One workgroup per digit, 1024 entries per step with 16-byte loads.
__global__ __launch_bounds__(256) void radix_rowscan_kernel(uint32_t* __restrict__ cnt, int nblk,
                                                            uint32_t* __restrict__ rowtot) {
  __shared__ uint32_t wsum[4];
  uint32_t* row = cnt + int64_t(blockIdx.x) * nblk;
  uint32_t carry = 0;
  for (int c0 = 0; c0 < nblk; c0 += 1024) {
    uint32_t v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = c0 + threadIdx.x * 4 + q;
      v[q] = j < nblk ? row[j] : 0u;
    }
    const uint32_t s = v[0] + v[1] + v[2] + v[3];
    uint32_t run = carry + block_exscan256(s, wsum);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = c0 + threadIdx.x * 4 + q;
      if (j < nblk) row[j] = run;
      run += v[q];
    }
    // the last thread's run is the new carry; share it through the scan's own workspace
    if (threadIdx.x == 255) wsum[0] = run;
    __syncthreads();
    carry = wsum[0];
    __syncthreads();
  }
  if (threadIdx.x == 0) rowtot[blockIdx.x] = carry;
}

// Stable scatter of a sort block's run of tiles, one tile at a time: ranks by (digit,
// input position) are computed per wave, the tile is staged in LDS in digit order and
// written out in that order, so the items of one digit leave as contiguous runs.  The
// next tile's keys are loaded while the current one is ranked and written.
template <int RR>
__global__ __launch_bounds__(RT) void radix_scatter_kernel(const uint64_t* __restrict__ kin,
                                                           const uint32_t* __restrict__ vin,
                                                           uint64_t* __restrict__ kout, uint32_t* __restrict__ vout,
                                                           int M, int shift, int tpb, const uint32_t* __restrict__ cnt,
                                                           const uint32_t* __restrict__ rowtot, int nblk) {
  constexpr int RTILE = RT * RR;
  __shared__ uint64_t skey[RTILE];
  __shared__ uint32_t sval[RTILE];
  __shared__ uint32_t wc[4][256];
  __shared__ uint32_t tstart[256];
  __shared__ int64_t gofs[256];
  __shared__ uint32_t wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt = (uint64_t(1) << lane) - 1;
  // running global position of this thread's digit (tid) over the block's tiles
  const uint32_t db = block_exscan256(rowtot[tid], wsum);
  int64_t run = int64_t(db) + cnt[int64_t(tid) * nblk + blockIdx.x];
  const int64_t t0 = int64_t(blockIdx.x) * tpb;
  const int64_t t_end = min<int64_t>(t0 + tpb, (int64_t(M) + RTILE - 1) / RTILE);
  uint64_t k[RR];
  uint32_t v[RR];
  auto load_tile = [&](int64_t t) {
    const int64_t base = t * RTILE + int64_t(wave) * (RR * 64);
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      const int64_t j = min<int64_t>(base + r * 64 + lane, M - 1);
      k[r] = kin[j];
      v[r] = vin[j];
    }
  };
  if (t0 < t_end) load_tile(t0);
  for (int64_t t = t0; t < t_end; ++t) {
    const int64_t tile0 = t * RTILE;
    const int64_t base = tile0 + int64_t(wave) * (RR * 64);
#pragma unroll
    for (int w = 0; w < 4; ++w) wc[w][tid] = 0;
    __syncthreads();
    uint32_t rk[RR];
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      const bool valid = base + r * 64 + lane < M;
      const uint32_t d = uint32_t(k[r] >> shift) & 255u;
      const uint64_t peers = digit_peers(d, valid);
      const uint32_t below = uint32_t(__popcll(peers & lt));
      const uint32_t before = wc[wave][d];
      rk[r] = before + below;
      if (valid && below == 0) wc[wave][d] = before + uint32_t(__popcll(peers));
    }
    __syncthreads();
    // per digit (thread tid = digit): wave offsets inside the tile, tile start, global offset
    uint32_t tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t c = wc[w][tid];
      wc[w][tid] = tot;
      tot += c;
    }
    const uint32_t ts = block_exscan256(tot, wsum);
    tstart[tid] = ts;
    gofs[tid] = run - int64_t(ts);
    run += tot;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      if (base + r * 64 + lane < M) {
        const uint32_t d = uint32_t(k[r] >> shift) & 255u;
        const uint32_t slot = tstart[d] + wc[wave][d] + rk[r];
        skey[slot] = k[r];
        sval[slot] = v[r];
      }
    }
    __syncthreads();
    if (t + 1 < t_end) load_tile(t + 1);
    const int64_t nt = min<int64_t>(RTILE, int64_t(M) - tile0);
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      const int p = r * RT + tid;
      if (p < nt) {
        const uint64_t key = skey[p];
        const int64_t dst = gofs[uint32_t(key >> shift) & 255u] + p;
        kout[dst] = key;
        vout[dst] = sval[p];
      }
    }
    __syncthreads();
  }
}

// Sum of the costs of each block of STILE sorted positions (int64, exact).
__global__ __launch_bounds__(256) void cost_bsum_kernel(const int32_t* __restrict__ order, CostLookup cl, int M,
                                                        int64_t* __restrict__ bsum) {
  __shared__ int64_t red[4];
  const int64_t base = int64_t(blockIdx.x) * STILE;
  int32_t id[SC];
#pragma unroll
  for (int i = 0; i < SC; ++i) {
    const int64_t p = min<int64_t>(base + i * 256 + int(threadIdx.x), M - 1);
    id[i] = order_id(order, p, M);
  }
  int64_t c[SC];
#pragma unroll
  for (int i = 0; i < SC; ++i) c[i] = cl.ctab[id[i] >> MB_SHIFT];
  int64_t s = 0;
#pragma unroll
  for (int i = 0; i < SC; ++i) {
    if (c[i] < 0) c[i] = cl.cost[matrix_of_item(cl.offs, cl.mtab, id[i])];
    s += base + i * 256 + int(threadIdx.x) < M ? c[i] : 0;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) bsum[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

// One workgroup: scan the block sums and find the block in which the running cost first
// exceeds the budget.  cut[0] = that block (-1 if everything fits, and then n_kept = M),
// cut[1] = the cost of all positions before it.
__global__ __launch_bounds__(1024) void cost_cut_block_kernel(const int64_t* __restrict__ bsum, int nsb, int M,
                                                              int64_t budget, int64_t* __restrict__ cut,
                                                              int64_t* __restrict__ n_kept) {
  __shared__ int64_t wsum[16];
  __shared__ int64_t carry_s;
  __shared__ int found;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) found = 0;
  int64_t carry = 0;
  __syncthreads();
  for (int c0 = 0; c0 < nsb; c0 += 1024) {
    const int c = c0 + tid;
    const int64_t v = c < nsb ? bsum[c] : 0;
    int64_t inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t t = __shfl_up(inc, o);
      if (lane >= o) inc += t;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int64_t pre = carry;
    for (int w = 0; w < wave; ++w) pre += wsum[w];
    const int64_t excl = pre + inc - v;
    // the running total only grows (every cost is positive): exactly one block crosses
    if (c < nsb && excl <= budget && excl + v > budget) {
      cut[0] = c;
      cut[1] = excl;
      found = 1;
    }
    if (tid == 1023) carry_s = pre + inc;
    __syncthreads();
    carry = carry_s;
    if (found) break;
    __syncthreads();
  }
  if (tid == 0 && !found) {
    cut[0] = -1;
    *n_kept = M;
  }
}

// One workgroup: inside the cut block, the first position whose running cost exceeds the
// budget is the number of kept components.
__global__ __launch_bounds__(256) void cost_cut_kernel(const int32_t* __restrict__ order, CostLookup cl, int M,
                                                       int64_t budget,
                                                       const int64_t* __restrict__ cut,
                                                       int64_t* __restrict__ n_kept) {
  __shared__ int64_t wsum[4];
  __shared__ int first;
  const int64_t cb = cut[0];
  if (cb < 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) first = STILE;
  // thread tid takes the SC consecutive positions base + tid * SC ...
  const int64_t base = cb * STILE + int64_t(tid) * SC;
  int64_t c[SC];
  int64_t s = 0;
#pragma unroll
  for (int i = 0; i < SC; ++i) {
    const int64_t p = base + i;
    c[i] = p < M ? cl(order_id(order, p, M)) : 0;
    s += c[i];
  }
  int64_t inc = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int64_t run = cut[1] + inc - s;
  for (int w = 0; w < wave; ++w) run += wsum[w];
  bool done = false;
#pragma unroll
  for (int i = 0; i < SC; ++i) {
    run += c[i];
    if (!done && base + i < M && run > budget) {
      atomicMin(&first, tid * SC + i);
      done = true;
    }
  }
  __syncthreads();
  if (tid == 0) *n_kept = cb * STILE + first;
}

__global__ void set_i64_kernel(int64_t* __restrict__ p, int64_t v) { *p = v; }
__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* __restrict__ p, int n) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// The cut for the mask: key bits and id of the first excluded item E, so that the kept
// items are exactly those whose (key bits, id) pair is below E's.  (~0, M) keeps every
// item, (0, 0) none.  A call whose inputs were rejected (info != 0: a score NaN, infinite
// or negative, or inconsistent offsets or costs) keeps nothing: n_kept = 0, and the mask
// and ranks come out zero.
__global__ void cut_key_kernel(const float* __restrict__ scores, CostLookup cl,
                               const int32_t* __restrict__ order, int M, int64_t* __restrict__ n_kept,
                               const int32_t* __restrict__ info, uint64_t* __restrict__ cutkey) {
  if (*info != 0) {
    *n_kept = 0;
    cutkey[0] = 0;
    cutkey[1] = 0;
    return;
  }
  const int64_t nk = *n_kept;
  if (nk >= M) {
    cutkey[0] = ~uint64_t(0);
    cutkey[1] = uint64_t(M);
    return;
  }
  bool nf;
  const int32_t id = order_id(order, nk < 0 ? 0 : nk, M);
  cutkey[0] = item_key(scores, cl, id, false, nf);
  cutkey[1] = uint64_t(id);
}

// kept_mask in item order: an item is kept when its (key bits, id) pair is below the cut's.
// The key is recomputed here so that the mask is written in item order rather than
// scattered through the order.  With part given, part[workgroup] = its kept count, and the
// kept items are also counted into rank_acc (zeroed before) per matrix: a workgroup's
// items are one bucket of the cost table, so a bucket inside one matrix adds its count
// with one atomic, and a bucket across matrix boundaries adds each kept item to its own
// matrix.  MASK_PER items per workgroup, consecutive lanes on consecutive items.
constexpr int MASK_PER = 256 * 16;
static_assert(MASK_PER == (1 << MB_SHIFT), "a mask workgroup is one bucket of the cost table");
__global__ __launch_bounds__(256) void mask_kernel(const float* __restrict__ scores, CostLookup cl, int M,
                                                   const uint64_t* __restrict__ cutkey,
                                                   const int32_t* __restrict__ info, uint8_t* __restrict__ kept,
                                                   int64_t* __restrict__ part, int32_t* __restrict__ rank_acc) {
  const uint64_t ck = cutkey[0];
  const int64_t cid = int64_t(cutkey[1]);
  const bool bad = *info == int32_t(LRC_EINVAL);
  const int64_t base = int64_t(blockIdx.x) * MASK_PER;
  int nk = 0;
  uint32_t kbits = 0;   // which of this thread's items were kept
  // every score of the thread loaded before any is used; the workgroup's items are one
  // bucket of the cost table, so their cost is looked up once when they share a matrix
  float sv[MASK_PER / 256];
#pragma unroll
  for (int i = 0; i < MASK_PER / 256; ++i) {
    const int64_t j = base + i * 256 + threadIdx.x;
    sv[i] = j < M ? scores[j] : 0.f;
  }
  const int64_t ct = bad ? 0 : cl.ctab[blockIdx.x];
#pragma unroll
  for (int i = 0; i < MASK_PER / 256; ++i) {
    const int64_t j = base + i * 256 + threadIdx.x;
    if (j < M) {
      bool nf = false;
      const uint64_t key = bad ? 0 : score_key(sv[i], ct >= 0 ? ct : cl(j), nf);
      const bool k = key < ck || (key == ck && j < cid);
      kept[j] = k ? 1 : 0;
      nk += k;
      kbits |= uint32_t(k) << i;
    }
  }
  if (part != nullptr) {
    __shared__ int wn[4];
    const bool one_matrix = ct >= 0;
    if (!one_matrix && kbits != 0) {
      for (int i = 0; i < MASK_PER / 256; ++i)
        if ((kbits >> i) & 1u)
          atomicAdd(&rank_acc[matrix_of_item(cl.offs, cl.mtab, base + i * 256 + threadIdx.x)], 1);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) nk += __shfl_xor(nk, o);
    if ((threadIdx.x & 63) == 0) wn[threadIdx.x >> 6] = nk;
    __syncthreads();
    if (threadIdx.x == 0) {
      const int tot = wn[0] + wn[1] + wn[2] + wn[3];
      part[blockIdx.x] = tot;
      if (one_matrix && tot != 0) atomicAdd(&rank_acc[cl.mtab[blockIdx.x]], tot);
    }
  }
}

// ---- radix select of the first excluded item (the call without an order)
// Select state: sel[0] = the key bits fixed so far (8 per level), sel[1] = the cost of every
// item whose key lies below that bucket, sel[2] = 1 when the whole pool fits the budget.
// Id state (the items whose key equals the selected key): seli[0] = the id bits fixed so
// far, seli[1] = the cost of every item below that id bucket.
// Select workgroup b takes SEL_PER-item tiles b, b + gridDim.x, ..., consecutive lanes on
// consecutive items.  Levels 0 to 2 read every score and recompute its key (4 bytes read
// per item instead of 8, and no key array written); level 2 also writes the items of its
// bucket (the 16 fixed bits: a few percent of a realistic pool) to the candidate list:
// wave w of a tile, which owns 1024 of its items, fills the quarter w of the tile's range,
// placing its matches by ballot, and records their count (so the list needs no more room
// than the tiles and no global counter or barrier).  Key levels 3 to 7 and the four id
// levels read only the candidates.  A thread sums the costs of its consecutive equal
// digits before one LDS atomic (the top digits of a realistic pool take few values).
// Every sum is an integer add, so none depends on order.
constexpr int SEL_PER = 256 * 16;
constexpr int SEL_RR = SEL_PER / 256;
constexpr int SEL_MAX_BLOCKS = 2048;
static_assert(SEL_PER == (1 << MB_SHIFT), "a select tile is one bucket of the cost table");

__device__ __forceinline__ void sel_run_add(unsigned long long* hc, uint32_t& cd, unsigned long long& cc,
                                            uint32_t d, int64_t c) {
  if (d != cd) {
    if (cc != 0) atomicAdd(&hc[cd], cc);
    cd = d;
    cc = 0;
  }
  cc += (unsigned long long)c;
}

// the workgroup's digit sums into the level's histogram (atomics: for levels whose
// workgroups fill few digits), or stored as the workgroup's row of a table that
// sel_reduce_kernel sums (levels whose workgroups fill many digits: the atomics of 2048
// workgroups on one 2 KB histogram serialise)
__device__ __forceinline__ void sel_flush(unsigned long long* hc, uint32_t cd, unsigned long long cc,
                                          unsigned long long* __restrict__ hist) {
  if (cc != 0) atomicAdd(&hc[cd], cc);
  __syncthreads();
  const unsigned long long v = hc[threadIdx.x];
  if (v != 0) atomicAdd(&hist[threadIdx.x], v);
}
__device__ __forceinline__ void sel_flush_row(unsigned long long* hc, uint32_t cd, unsigned long long cc,
                                              unsigned long long* __restrict__ rows) {
  if (cc != 0) atomicAdd(&hc[cd], cc);
  __syncthreads();
  rows[int64_t(blockIdx.x) * 256 + threadIdx.x] = hc[threadIdx.x];
}

// the level histogram from the rows of nrows workgroups: workgroup g sums rows g,
// g + gridDim.x, ... and adds its 256 sums
constexpr int SEL_REDUCE_BLOCKS = 64;
__global__ __launch_bounds__(256) void sel_reduce_kernel(const unsigned long long* __restrict__ rows, int nrows,
                                                         const uint64_t* __restrict__ sel,
                                                         unsigned long long* __restrict__ hist) {
  if (sel[2] != 0) return;
  unsigned long long v = 0;
  for (int r = blockIdx.x; r < nrows; r += gridDim.x) v += rows[int64_t(r) * 256 + threadIdx.x];
  if (v != 0) atomicAdd(&hist[threadIdx.x], v);
}

// A full select pass loads its thread's SEL_RR scores of a tile before using any (all the
// loads in flight at once), and looks the tile's cost up once: a tile is one bucket of the
// cost table, so ctab[tile] is the cost of every item when they share a matrix, else -1.
// The keys are recomputed from the scores in each full pass rather than stored (4 bytes
// read per item instead of 8, and no 8-byte write); rejected offsets or costs give every
// item key 0 and cost 0.
__device__ __forceinline__ int64_t sel_load_tile(const float* __restrict__ scores, const CostLookup& cl, int M,
                                                 int64_t base, bool bad, float (&sv)[SEL_PER / 256]) {
#pragma unroll
  for (int i = 0; i < SEL_PER / 256; ++i) {
    const int64_t j = base + i * 256 + threadIdx.x;
    sv[i] = j < M ? scores[j] : 0.f;
  }
  return bad ? 0 : cl.ctab[base >> MB_SHIFT];
}

// key bits and cost of item j from its loaded score (the same as item_key's)
__device__ __forceinline__ void sel_item(float sc, int64_t ct, const CostLookup& cl, int64_t j, bool bad,
                                         uint64_t& u, int64_t& c, bool& nf) {
  nf = false;
  u = 0;
  c = 0;
  if (bad) return;
  c = ct >= 0 ? ct : cl(j);
  u = score_key(sc, c, nf);
}

// zero the level histogram
__global__ __launch_bounds__(256) void sel_init_kernel(unsigned long long* __restrict__ hist) {
  hist[threadIdx.x] = 0;
}

// level 0: the cost of the items of each top digit; flags NaN, infinite or negative scores
__global__ __launch_bounds__(256) void sel_key_kernel(const float* __restrict__ scores, CostLookup cl, int M,
                                                      unsigned long long* __restrict__ hist,
                                                      int32_t* __restrict__ info) {
  __shared__ unsigned long long hc[256];
  hc[threadIdx.x] = 0;
  __syncthreads();
  const bool bad = *info == int32_t(LRC_EINVAL);
  bool any_nf = false;
  uint32_t cd = 0;
  unsigned long long cc = 0;
  for (int64_t base = int64_t(blockIdx.x) * SEL_PER; base < M; base += int64_t(gridDim.x) * SEL_PER) {
    float sv[SEL_RR];
    const int64_t ct = sel_load_tile(scores, cl, M, base, bad, sv);
#pragma unroll
    for (int i = 0; i < SEL_RR; ++i) {
      const int64_t j = base + i * 256 + threadIdx.x;
      if (j < M) {
        uint64_t u;
        int64_t c;
        bool nf;
        sel_item(sv[i], ct, cl, j, bad, u, c, nf);
        any_nf |= nf;
        sel_run_add(hc, cd, cc, uint32_t(u >> 56), c);
      }
    }
  }
  sel_flush(hc, cd, cc, hist);
  if (any_nf) atomicExch(info, int32_t(LRC_ENONFINITE));
}

// level 1: over the items of the chosen top-digit bucket, the cost of each next digit
__global__ __launch_bounds__(256) void sel_hist_kernel(const float* __restrict__ scores, CostLookup cl, int M,
                                                       const int32_t* __restrict__ info,
                                                       const uint64_t* __restrict__ sel,
                                                       unsigned long long* __restrict__ rows) {
  if (sel[2] != 0) return;
  const bool bad = *info == int32_t(LRC_EINVAL);
  __shared__ unsigned long long hc[256];
  const uint64_t pre = sel[0];   // 8 bits
  hc[threadIdx.x] = 0;
  __syncthreads();
  uint32_t cd = 0;
  unsigned long long cc = 0;
  for (int64_t base = int64_t(blockIdx.x) * SEL_PER; base < M; base += int64_t(gridDim.x) * SEL_PER) {
    float sv[SEL_RR];
    const int64_t ct = sel_load_tile(scores, cl, M, base, bad, sv);
#pragma unroll
    for (int i = 0; i < SEL_RR; ++i) {
      const int64_t j = base + i * 256 + threadIdx.x;
      if (j < M) {
        uint64_t u;
        int64_t c;
        bool nf;
        sel_item(sv[i], ct, cl, j, bad, u, c, nf);
        if ((u >> 56) == pre) sel_run_add(hc, cd, cc, uint32_t(u >> 48) & 255u, c);
      }
    }
  }
  sel_flush_row(hc, cd, cc, rows);
}

// level 2 over every item, writing the items of the chosen 16-bit bucket to the candidate
// list: wave w of tile k writes its matches to [k SEL_PER + w SEL_WQ, ...) and their count
// to ccnt[4 k + w]
constexpr int SEL_WQ = SEL_PER / 4;   // items of a tile owned by one wave
__global__ __launch_bounds__(256) void sel_hist_compact_kernel(const float* __restrict__ scores, CostLookup cl,
                                                               int M, const int32_t* __restrict__ info,
                                                               const uint64_t* __restrict__ sel,
                                                               unsigned long long* __restrict__ rows,
                                                               uint64_t* __restrict__ ckeys,
                                                               uint32_t* __restrict__ cids,
                                                               uint32_t* __restrict__ ccnt) {
  if (sel[2] != 0) return;
  __shared__ unsigned long long hc[256];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const uint64_t pre = sel[0];   // 16 bits
  const bool bad = *info == int32_t(LRC_EINVAL);
  const uint64_t below = (uint64_t(1) << lane) - 1;
  hc[t] = 0;
  __syncthreads();
  uint32_t cd = 0;
  unsigned long long cc = 0;
  for (int64_t base = int64_t(blockIdx.x) * SEL_PER; base < M; base += int64_t(gridDim.x) * SEL_PER) {
    const int64_t region = base + wave * SEL_WQ;
    uint32_t filled = 0;   // the same in every lane of the wave
    float sv[SEL_RR];
    const int64_t ct = sel_load_tile(scores, cl, M, base, bad, sv);
#pragma unroll
    for (int i = 0; i < SEL_RR; ++i) {
      const int64_t j = base + i * 256 + t;
      uint64_t u = 0;
      int64_t c = 0;
      bool nf;
      if (j < M) sel_item(sv[i], ct, cl, j, bad, u, c, nf);
      const bool m = j < M && (u >> 48) == pre;
      const uint64_t bal = __ballot(m);
      if (m) {
        const int64_t p = region + filled + __popcll(bal & below);
        ckeys[p] = u;
        cids[p] = uint32_t(j);
        sel_run_add(hc, cd, cc, uint32_t(u >> 40) & 255u, c);
      }
      filled += uint32_t(__popcll(bal));
    }
    if (lane == 0) ccnt[(base / SEL_PER) * 4 + wave] = filled;
  }
  sel_flush_row(hc, cd, cc, rows);
}

// key levels 3 to 7 (idlevel < 0) and id levels 0 to 3 (idlevel >= 0: candidates whose key
// equals the selected key, digits of the id), over the candidate regions only
__global__ __launch_bounds__(256) void sel_hist_cand_kernel(const uint64_t* __restrict__ ckeys,
                                                            const uint32_t* __restrict__ cids,
                                                            const uint32_t* __restrict__ ccnt, int M, CostLookup cl,
                                                            int level, int idlevel, const uint64_t* __restrict__ sel,
                                                            const uint64_t* __restrict__ seli,
                                                            unsigned long long* __restrict__ hist) {
  if (sel[2] != 0) return;
  __shared__ unsigned long long hc[256];
  hc[threadIdx.x] = 0;
  __syncthreads();
  uint32_t cd = 0;
  unsigned long long cc = 0;
  const bool by_id = idlevel >= 0;
  const int shift = by_id ? 24 - 8 * idlevel : 56 - 8 * level;   // ids: 24 .. 0; keys: 32 .. 0
  const uint64_t ks = sel[0];
  const uint64_t pre = by_id ? (idlevel == 0 ? 0 : seli[0]) : ks;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int64_t base = int64_t(blockIdx.x) * SEL_PER; base < M; base += int64_t(gridDim.x) * SEL_PER) {
    // wave w reads the candidates of the tile's quarter w
    const int64_t r0 = base + wave * SEL_WQ;
    const int64_t end = r0 + ccnt[(base / SEL_PER) * 4 + wave];
    for (int64_t p = r0 + lane; p < end; p += 64) {
      const uint64_t u = ckeys[p];
      const uint64_t id = cids[p];
      if (by_id) {
        if (u == ks && (id >> (shift + 8)) == pre) sel_run_add(hc, cd, cc, uint32_t(id >> shift) & 255u, cl(id));
      } else if ((u >> (shift + 8)) == pre) {
        sel_run_add(hc, cd, cc, uint32_t(u >> shift) & 255u, cl(id));
      }
    }
  }
  sel_flush(hc, cd, cc, hist);
}

// One workgroup, thread t owning digit t: fix the digit whose bucket carries the running
// cost past the budget and carry the cost of the buckets below it; the histogram is
// cleared for the next level.  Key levels (idlevel < 0) update sel: at level 0 a pool that
// fits whole sets sel[2].  Id levels update seli, starting from the cost carried below the
// selected key.  Below level 0 a chosen bucket's digits split its cost exactly, so exactly
// one digit crosses.
__global__ __launch_bounds__(256) void sel_step_kernel(unsigned long long* __restrict__ hist, int level, int idlevel,
                                                       int64_t budget, uint64_t* __restrict__ sel,
                                                       uint64_t* __restrict__ seli) {
  __shared__ int64_t wsum[4];
  __shared__ uint64_t cur[3];   // prefix, cost below, pool fits
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (t == 0) {
    if (idlevel < 0) {
      cur[0] = level == 0 ? 0 : sel[0];
      cur[1] = level == 0 ? 0 : sel[1];
      cur[2] = level == 0 ? 0 : sel[2];
    } else {
      cur[0] = idlevel == 0 ? 0 : seli[0];
      cur[1] = idlevel == 0 ? sel[1] : seli[1];
      cur[2] = sel[2];
    }
  }
  const int64_t v = int64_t(hist[t]);
  hist[t] = 0;
  __syncthreads();
  if (cur[2] != 0) return;
  int64_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t x = __shfl_up(inc, o);
    if (lane >= o) inc += x;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int64_t below = int64_t(cur[1]) + inc - v;
  for (int w = 0; w < wave; ++w) below += wsum[w];
  uint64_t* out = idlevel < 0 ? sel : seli;
  if (below <= budget && below + v > budget) {
    out[0] = (cur[0] << 8) | uint64_t(t);
    out[1] = uint64_t(below);
    if (idlevel < 0) out[2] = 0;
  } else if (idlevel < 0 && level == 0 && t == 255 && below + v <= budget) {
    sel[0] = 0;
    sel[1] = uint64_t(below + v);
    sel[2] = 1;
  }
}

// The cut for the mask: the selected key and the first excluded id among its items.
__global__ void sel_cut_kernel(const uint64_t* __restrict__ sel, const uint64_t* __restrict__ seli, int M,
                               const int32_t* __restrict__ info, uint64_t* __restrict__ cutkey) {
  if (*info != 0) {   // rejected inputs: nothing kept
    cutkey[0] = 0;
    cutkey[1] = 0;
  } else if (sel[2] != 0) {   // the whole pool fits
    cutkey[0] = ~uint64_t(0);
    cutkey[1] = uint64_t(M);
  } else {
    cutkey[0] = sel[0];
    cutkey[1] = seli[0];
  }
}

// n_kept = the sum of the mask workgroups' kept counts (one workgroup, fixed order)
__global__ __launch_bounds__(256) void sum_parts_kernel(const int64_t* __restrict__ part, int n,
                                                        int64_t* __restrict__ out) {
  __shared__ int64_t red[4];
  int64_t s = 0;
  for (int i = threadIdx.x; i < n; i += 256) s += part[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) *out = red[0] + red[1] + red[2] + red[3];
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
  uint32_t *va, *vb, *hist, *rowtot;
  int32_t* mtab;
  int64_t* ctab;
  int64_t *bsum, *cut;
  uint64_t* cutkey;
  unsigned long long* sel_hist;   // 256 digit sums of one select level
  uint64_t *sel, *seli;           // select states (key, id)
  uint32_t* ccnt;                 // candidate count per wave of a select tile
  unsigned long long* sel_rows;   // per-workgroup digit sums of a select level
  int64_t* mpart;                 // kept count per mask workgroup
};

// sort geometry: tiles of RT rr items, runs of tpb tiles per sort workgroup
struct SortGeom {
  int64_t ntiles, tpb, nblk;
  int rr;
};
SortGeom sort_geom(int64_t M) {
  SortGeom g;
  g.rr = cdiv(M, int64_t(RT) * RR_BIG) < 512 ? RR_SMALL : RR_BIG;
  g.ntiles = std::max<int64_t>(1, cdiv(M, int64_t(RT) * g.rr));
  g.tpb = cdiv(g.ntiles, MAX_SORT_BLOCKS);
  g.nblk = cdiv(g.ntiles, g.tpb);
  return g;
}

AWs carve_alloc(Carve& cv, int64_t M) {
  const int64_t nblk = sort_geom(M).nblk;
  const int64_t nsb = std::max<int64_t>(1, cdiv(M, STILE));
  AWs w;
  w.ka = cv.take<uint64_t>(size_t(std::max<int64_t>(M, 1)));
  // kb and va also hold the select's candidate list, laid out by tile quarters: rounded
  // up to whole tiles
  const int64_t m_tiles = std::max<int64_t>(1, cdiv(M, SEL_PER)) * SEL_PER;
  w.kb = cv.take<uint64_t>(size_t(m_tiles));
  w.va = cv.take<uint32_t>(size_t(m_tiles));
  w.vb = cv.take<uint32_t>(size_t(std::max<int64_t>(M, 1)));
  w.hist = cv.take<uint32_t>(size_t(256 * nblk));
  w.rowtot = cv.take<uint32_t>(256);
  w.mtab = cv.take<int32_t>(size_t((std::max<int64_t>(M, 1) >> MB_SHIFT) + 2));
  w.ctab = cv.take<int64_t>(size_t((std::max<int64_t>(M, 1) >> MB_SHIFT) + 2));
  w.bsum = cv.take<int64_t>(size_t(nsb));
  w.cut = cv.take<int64_t>(2);
  w.cutkey = cv.take<uint64_t>(2);
  w.sel_hist = cv.take<unsigned long long>(256);
  w.sel = cv.take<uint64_t>(4);
  w.seli = cv.take<uint64_t>(4);
  w.ccnt = cv.take<uint32_t>(size_t(4 * std::max<int64_t>(1, cdiv(M, SEL_PER))));
  w.sel_rows = cv.take<unsigned long long>(size_t(256) * size_t(std::min<int64_t>(
      std::max<int64_t>(1, cdiv(M, SEL_PER)), SEL_MAX_BLOCKS)));
  w.mpart = cv.take<int64_t>(size_t(std::max<int64_t>(1, cdiv(M, MASK_PER))));
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

namespace {

// argument checks shared by both entry points (host only, before any HIP call)
lrc_status alloc_check_args(const float* scores, const int64_t* offsets, const int64_t* cost, int64_t n_mat,
                            int64_t n_items, int64_t budget, int32_t* order, int64_t* n_kept, int32_t* ranks,
                            uint8_t* kept_mask, int32_t* info) {
  if (offsets == nullptr || cost == nullptr || n_kept == nullptr || ranks == nullptr || info == nullptr)
    return LRC_EINVAL;
  if (n_mat <= 0 || n_mat > (int64_t(1) << 30) || n_items < 0 || n_items >= (int64_t(1) << 31) || budget < 0)
    return LRC_EINVAL;
  if (n_items > 0 && (scores == nullptr || kept_mask == nullptr)) return LRC_EINVAL;   // order may be null
  return LRC_OK;
}

// the whole allocation on `st`, scratch at ws (laid out by carve_alloc for n_items)
lrc_status allocate_impl(const float* scores, const int64_t* offsets, const int64_t* cost, int64_t n_mat,
                         int64_t n_items, int64_t budget, int32_t* order, int64_t* n_kept, int32_t* ranks,
                         uint8_t* kept_mask, int32_t* info, void* ws, hipStream_t st) {
  Carve cv(ws);
  AWs w = carve_alloc(cv, n_items);
  const int M = int(n_items);
  const int nm = int(n_mat);

  alloc_check_ends_kernel<<<1, 1, 0, st>>>(offsets, nm, n_items, info);
  LRC_LAUNCHED();
  alloc_check_kernel<<<unsigned(cdiv(int64_t(nm), 256)), 256, 0, st>>>(offsets, cost, nm, info);
  LRC_LAUNCHED();
  if (M > 0) {
    const int nbk = int((int64_t(M) - 1) >> MB_SHIFT) + 1;
    mtab_kernel<<<unsigned(cdiv(nbk + 1, 256)), 256, 0, st>>>(offsets, cost, nm, M, nbk, w.mtab, w.ctab);
    LRC_LAUNCHED();
    const CostLookup cl{offsets, w.mtab, w.ctab, cost};
    const int nsb = int(cdiv(M, STILE));
    if (order == nullptr) {   // no order wanted: select the cut instead of sorting
      const unsigned nsel = unsigned(std::min<int64_t>(cdiv(M, SEL_PER), SEL_MAX_BLOCKS));
      sel_init_kernel<<<1, 256, 0, st>>>(w.sel_hist);
      LRC_LAUNCHED();
      zero_i32_kernel<<<unsigned(cdiv(int64_t(nm), 256)), 256, 0, st>>>(ranks, nm);   // counted by the mask pass
      LRC_LAUNCHED();
      sel_key_kernel<<<nsel, 256, 0, st>>>(scores, cl, M, w.sel_hist, info);
      LRC_LAUNCHED();
      // key levels, then the id levels among the items of the selected key; candidates:
      // keys in kb, ids in va
      for (int level = 0; level < 12; ++level) {
        const int kl = level < 8 ? level : -1, il = level < 8 ? -1 : level - 8;
        if (level == 1)
          sel_hist_kernel<<<nsel, 256, 0, st>>>(scores, cl, M, info, w.sel, w.sel_rows);
        else if (level == 2)
          sel_hist_compact_kernel<<<nsel, 256, 0, st>>>(scores, cl, M, info, w.sel, w.sel_rows, w.kb, w.va, w.ccnt);
        if (level == 1 || level == 2) {
          LRC_LAUNCHED();
          sel_reduce_kernel<<<SEL_REDUCE_BLOCKS, 256, 0, st>>>(w.sel_rows, int(nsel), w.sel, w.sel_hist);
        }
        else if (level > 2)
          sel_hist_cand_kernel<<<nsel, 256, 0, st>>>(w.kb, w.va, w.ccnt, M, cl, kl, il, w.sel, w.seli,
                                                     w.sel_hist);
        if (level > 0) LRC_LAUNCHED();
        sel_step_kernel<<<1, 256, 0, st>>>(w.sel_hist, kl, il, budget, w.sel, w.seli);
        LRC_LAUNCHED();
      }
      sel_cut_kernel<<<1, 1, 0, st>>>(w.sel, w.seli, M, info, w.cutkey);
      LRC_LAUNCHED();
      const int nmask = int(cdiv(M, MASK_PER));
      mask_kernel<<<unsigned(nmask), 256, 0, st>>>(scores, cl, M, w.cutkey, info, kept_mask, w.mpart, ranks);
      LRC_LAUNCHED();
      sum_parts_kernel<<<1, 256, 0, st>>>(w.mpart, nmask, n_kept);
      LRC_LAUNCHED();
      return LRC_OK;
    }
    key_kernel<<<unsigned(cdiv(M, KEY_PER)), 256, 0, st>>>(scores, cl, M, w.ka, w.va, info);
    LRC_LAUNCHED();
    const SortGeom sg = sort_geom(M);
    const int nblk = int(sg.nblk), tpb = int(sg.tpb);
    uint64_t *kin = w.ka, *kout = w.kb;
    uint32_t *vin = w.va, *vout = w.vb;
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = pass * 8;
      // the last pass writes the sorted ids straight into the order output
      uint32_t* vdst = pass == 7 ? reinterpret_cast<uint32_t*>(order) : vout;
      if (sg.rr == RR_SMALL)
        radix_hist_kernel<RR_SMALL><<<unsigned(nblk), RT, 0, st>>>(kin, M, shift, tpb, w.hist, nblk);
      else
        radix_hist_kernel<RR_BIG><<<unsigned(nblk), RT, 0, st>>>(kin, M, shift, tpb, w.hist, nblk);
      LRC_LAUNCHED();
      radix_rowscan_kernel<<<256, 256, 0, st>>>(w.hist, nblk, w.rowtot);
      LRC_LAUNCHED();
      if (sg.rr == RR_SMALL)
        radix_scatter_kernel<RR_SMALL><<<unsigned(nblk), RT, 0, st>>>(kin, vin, kout, vdst, M, shift, tpb, w.hist,
                                                                      w.rowtot, nblk);
      else
        radix_scatter_kernel<RR_BIG><<<unsigned(nblk), RT, 0, st>>>(kin, vin, kout, vdst, M, shift, tpb, w.hist,
                                                                    w.rowtot, nblk);
      LRC_LAUNCHED();
      std::swap(kin, kout);
      std::swap(vin, vout);
    }
    cost_bsum_kernel<<<unsigned(nsb), 256, 0, st>>>(order, cl, M, w.bsum);
    LRC_LAUNCHED();
    cost_cut_block_kernel<<<1, 1024, 0, st>>>(w.bsum, nsb, M, budget, w.cut, n_kept);
    LRC_LAUNCHED();
    cost_cut_kernel<<<1, 256, 0, st>>>(order, cl, M, budget, w.cut, n_kept);
    LRC_LAUNCHED();
    cut_key_kernel<<<1, 1, 0, st>>>(scores, cl, order, M, n_kept, info, w.cutkey);
    LRC_LAUNCHED();
    mask_kernel<<<unsigned(cdiv(M, MASK_PER)), 256, 0, st>>>(scores, cl, M, w.cutkey, info, kept_mask, nullptr,
                                                             nullptr);
    LRC_LAUNCHED();
  } else {
    set_i64_kernel<<<1, 1, 0, st>>>(n_kept, 0);
    LRC_LAUNCHED();
  }
  ranks_kernel<<<unsigned(nm), 256, 0, st>>>(kept_mask, offsets, n_items, info, ranks);
  LRC_LAUNCHED();
  return LRC_OK;
}

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// the device address of `scratch` on the current device, looked up once per device (the
// array's host-side name is only a stand-in and must never reach a kernel)
lrc_status scratch_for_current_device(void** out) {
  int dev = -1;
  LRC_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= MAX_DEVICES) return LRC_EINVAL;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    LRC_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (p == nullptr) return LRC_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LRC_OK;
}

}  // namespace

extern "C" lrc_status lrc_allocate_ranks(const float* scores, const int64_t* offsets, const int64_t* cost,
                                         int64_t n_mat, int64_t n_items, int64_t budget, int32_t* order,
                                         int64_t* n_kept, int32_t* ranks, uint8_t* kept_mask, int32_t* info,
                                         void* ws, size_t ws_bytes, void* stream) {
  LRC_TRY(alloc_check_args(scores, offsets, cost, n_mat, n_items, budget, order, n_kept, ranks, kept_mask, info));
  const size_t need = lrc_allocate_ranks_workspace(n_mat, n_items);
  if (ws == nullptr || ws_bytes < need) return LRC_EWORKSPACE;
  return allocate_impl(scores, offsets, cost, n_mat, n_items, budget, order, n_kept, ranks, kept_mask, info, ws,
                       static_cast<hipStream_t>(stream));
}

extern "C" int64_t lrc_allocate_ranks_noalloc_max_items(void) { return NOALLOC_MAX_ITEMS; }

extern "C" lrc_status lrc_allocate_ranks_noalloc(const float* scores, const int64_t* offsets, const int64_t* cost,
                                                 int64_t n_mat, int64_t n_items, int64_t budget, int32_t* order,
                                                 int64_t* n_kept, int32_t* ranks, uint8_t* kept_mask, int32_t* info,
                                                 void* stream) {
  LRC_TRY(alloc_check_args(scores, offsets, cost, n_mat, n_items, budget, order, n_kept, ranks, kept_mask, info));
  if (n_items > NOALLOC_MAX_ITEMS) return LRC_EWORKSPACE;
  if (lrc_allocate_ranks_workspace(n_mat, n_items) > NOALLOC_SCRATCH_BYTES) return LRC_EWORKSPACE;
  void* ws = nullptr;
  LRC_TRY(scratch_for_current_device(&ws));
  return allocate_impl(scores, offsets, cost, n_mat, n_items, budget, order, n_kept, ranks, kept_mask, info, ws,
                       static_cast<hipStream_t>(stream));
}
