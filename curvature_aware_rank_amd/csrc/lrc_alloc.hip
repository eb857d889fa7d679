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
// is then written in item order by comparing each item's (key, id) with the last kept
// item's.  Matrix costs are looked up per 4096-item bucket.
#include "lrc_internal.h"

namespace lrc {
namespace {

constexpr int RT = 256;        // threads per sort workgroup (4 waves)
constexpr int RR = 16;         // items per thread (each wave: RR rounds of 64 consecutive items)
constexpr int RTILE = RT * RR; // items per workgroup tile
constexpr int MAX_SORT_BLOCKS = 1024;   // sort workgroups per pass; each takes a run of tiles
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

// sort key of item j: ~bits(fp64(score) / fp64(cost)); 0 (first in the order) for a
// rejected item, whose call reports an error
__device__ __forceinline__ uint64_t item_key(const float* __restrict__ scores, const CostLookup& cl, int64_t j,
                                             bool inputs_bad, bool& nonfinite) {
  nonfinite = false;
  if (inputs_bad) return 0;
  const float sc = scores[j];
  if (!isfinite(sc) || sc < 0.f) {
    nonfinite = true;
    return 0;
  }
  const double key = (double(sc) + 0.0) / double(cl(j));   // +0.0: -0 -> +0
  return ~uint64_t(__double_as_longlong(key));
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
__global__ __launch_bounds__(RT) void radix_hist_kernel(const uint64_t* __restrict__ keys, int M, int shift,
                                                        int tpb, uint32_t* __restrict__ cnt, int nblk) {
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
__global__ __launch_bounds__(RT) void radix_scatter_kernel(const uint64_t* __restrict__ kin,
                                                           const uint32_t* __restrict__ vin,
                                                           uint64_t* __restrict__ kout, uint32_t* __restrict__ vout,
                                                           int M, int shift, int tpb, const uint32_t* __restrict__ cnt,
                                                           const uint32_t* __restrict__ rowtot, int nblk) {
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

// key and id of the last kept position (or an empty marker) for the mask
__global__ void cut_key_kernel(const float* __restrict__ scores, CostLookup cl,
                               const int32_t* __restrict__ order, int M, const int64_t* __restrict__ n_kept,
                               const int32_t* __restrict__ info, uint64_t* __restrict__ cutkey) {
  const int64_t nk = *n_kept;
  if (nk <= 0) {
    cutkey[1] = ~uint64_t(0);   // no id is <= this as a signed int64: nothing kept
    return;
  }
  bool nf;
  const int32_t id = order_id(order, nk - 1, M);
  cutkey[0] = item_key(scores, cl, id, *info == int32_t(LRC_EINVAL), nf);
  cutkey[1] = uint64_t(id);
}

// kept_mask in item order: the kept items are the sorted prefix, i.e. exactly those whose
// (key bits, id) pair is at most that of the last kept item.  The key is recomputed here
// so that the mask is written in item order rather than scattered through the order.
// MASK_PER items per workgroup, consecutive lanes on consecutive items.
constexpr int MASK_PER = 256 * 16;
__global__ __launch_bounds__(256) void mask_kernel(const float* __restrict__ scores, CostLookup cl, int M,
                                                   const uint64_t* __restrict__ cutkey,
                                                   const int32_t* __restrict__ info, uint8_t* __restrict__ kept) {
  const uint64_t ck = cutkey[0];
  const int64_t cid = int64_t(cutkey[1]);
  const bool bad = *info == int32_t(LRC_EINVAL);
  const int64_t base = int64_t(blockIdx.x) * MASK_PER;
#pragma unroll 4
  for (int i = 0; i < MASK_PER / 256; ++i) {
    const int64_t j = base + i * 256 + threadIdx.x;
    if (j < M) {
      bool nf;
      const uint64_t key = item_key(scores, cl, j, bad, nf);
      kept[j] = (cid >= 0 && (key < ck || (key == ck && j <= cid))) ? 1 : 0;
    }
  }
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
};

// sort geometry: tiles of RTILE items, runs of tpb tiles per sort workgroup
struct SortGeom {
  int64_t ntiles, tpb, nblk;
};
SortGeom sort_geom(int64_t M) {
  SortGeom g;
  g.ntiles = std::max<int64_t>(1, cdiv(M, RTILE));
  g.tpb = cdiv(g.ntiles, MAX_SORT_BLOCKS);
  g.nblk = cdiv(g.ntiles, g.tpb);
  return g;
}

AWs carve_alloc(Carve& cv, int64_t M) {
  const int64_t nblk = sort_geom(M).nblk;
  const int64_t nsb = std::max<int64_t>(1, cdiv(M, STILE));
  AWs w;
  w.ka = cv.take<uint64_t>(size_t(std::max<int64_t>(M, 1)));
  w.kb = cv.take<uint64_t>(size_t(std::max<int64_t>(M, 1)));
  w.va = cv.take<uint32_t>(size_t(std::max<int64_t>(M, 1)));
  w.vb = cv.take<uint32_t>(size_t(std::max<int64_t>(M, 1)));
  w.hist = cv.take<uint32_t>(size_t(256 * nblk));
  w.rowtot = cv.take<uint32_t>(256);
  w.mtab = cv.take<int32_t>(size_t((std::max<int64_t>(M, 1) >> MB_SHIFT) + 2));
  w.ctab = cv.take<int64_t>(size_t((std::max<int64_t>(M, 1) >> MB_SHIFT) + 2));
  w.bsum = cv.take<int64_t>(size_t(nsb));
  w.cut = cv.take<int64_t>(2);
  w.cutkey = cv.take<uint64_t>(2);
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
    const int nbk = int((int64_t(M) - 1) >> MB_SHIFT) + 1;
    mtab_kernel<<<unsigned(cdiv(nbk + 1, 256)), 256, 0, st>>>(offsets, cost, nm, M, nbk, w.mtab, w.ctab);
    LRC_LAUNCHED();
    const CostLookup cl{offsets, w.mtab, w.ctab, cost};
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
      radix_hist_kernel<<<unsigned(nblk), RT, 0, st>>>(kin, M, shift, tpb, w.hist, nblk);
      LRC_LAUNCHED();
      radix_rowscan_kernel<<<256, 256, 0, st>>>(w.hist, nblk, w.rowtot);
      LRC_LAUNCHED();
      radix_scatter_kernel<<<unsigned(nblk), RT, 0, st>>>(kin, vin, kout, vdst, M, shift, tpb, w.hist,
                                                          w.rowtot, nblk);
      LRC_LAUNCHED();
      std::swap(kin, kout);
      std::swap(vin, vout);
    }
    const int nsb = int(cdiv(M, STILE));
    cost_bsum_kernel<<<unsigned(nsb), 256, 0, st>>>(order, cl, M, w.bsum);
    LRC_LAUNCHED();
    cost_cut_block_kernel<<<1, 1024, 0, st>>>(w.bsum, nsb, M, budget, w.cut, n_kept);
    LRC_LAUNCHED();
    cost_cut_kernel<<<1, 256, 0, st>>>(order, cl, M, budget, w.cut, n_kept);
    LRC_LAUNCHED();
    cut_key_kernel<<<1, 1, 0, st>>>(scores, cl, order, M, n_kept, info, w.cutkey);
    LRC_LAUNCHED();
    mask_kernel<<<unsigned(cdiv(M, MASK_PER)), 256, 0, st>>>(scores, cl, M, w.cutkey, info, kept_mask);
    LRC_LAUNCHED();
  } else {
    set_i64_kernel<<<1, 1, 0, st>>>(n_kept, 0);
    LRC_LAUNCHED();
  }
  ranks_kernel<<<unsigned(nm), 256, 0, st>>>(kept_mask, offsets, n_items, info, ranks);
  LRC_LAUNCHED();
  return LRC_OK;
}
