// Covariance streaming: C[lower] += A^T A  (bf16 MFMA SYRK, fp32 SYRK, int8 QAW pre-pass).
//
// LASER technical summary, Methodology 1 (K-FAC surrogate: activation / gradient
// covariances estimated on a calibration set; QAW: estimated from quantised
// activations) and Swift-SVD technical summary 2A (incremental, one-pass aggregation of
// a covariance over batches of tokens).
//
// bf16 path (the hot one).  The reduction axis is the token axis, which is the strided
// axis of the token-major input, while an MFMA operand wants 8 consecutive reduction
// elements per lane.  Token rows are therefore copied unchanged (16-byte chunks) into
// LDS, and each lane reads its fragment with two LDS transpose reads
// (ds_read_b64_tr_b16), which hand every lane 4 consecutive tokens of one channel.
// Tiles are 256 x 256 of the lower triangle; 4 waves each own a 128 x 128 block computed
// with v_mfma_f32_32x32x16_bf16 (fp32 accumulation of exact bf16 products; the
// accumulators fill the waves' accumulation registers).  Global loads run one stage ahead
// in registers from clamped addresses (range masking happens at the LDS store, so the
// loads stay unpredicated and in flight together).  Tokens are split S ways so that the
// launch fills the chip; every split writes its partial tile and a second kernel adds the
// partials to C in split order, so results are bit-reproducible.
#include "lrc_internal.h"

namespace lrc {
namespace {

constexpr int TB = 256;              // tile edge in channels
constexpr int KS = 64;               // tokens per LDS stage
constexpr int RP = TB + 32;          // bf16 per token row in LDS: 576 B (rows shift by 16 banks)
constexpr int NTH = 256;             // threads per workgroup (4 waves, 2 x 2 blocks of 128 x 128)
constexpr int OPER = KS * RP;        // bf16 per operand per stage
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

// One 16-byte chunk (8 channels of one token) per load, always from a clamped in-range
// address.  Out-of-range tokens and channels are zeroed when the chunk is stored to LDS,
// one pipeline stage later: zeroing next to the load would make the compiler predicate
// the load and wait for it (and for every earlier load) right there.
template <bool VEC>
__device__ __forceinline__ uint4 load_chunk(const uint16_t* __restrict__ X, int64_t ldx, int64_t t, int64_t t_end,
                                            int c, int d) {
  const int64_t tc = t < t_end ? t : t_end - 1;
  if (VEC) {
    const int cc = c < d ? c : d - 8;
    return *reinterpret_cast<const uint4*>(X + tc * ldx + cc);
  }
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = X[tc * ldx + (c + e < d ? c + e : d - 1)];
  return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
}

// zero the halves of a chunk whose token or channel is out of range
__device__ __forceinline__ uint4 mask_chunk(uint4 v, bool ok_t, int c, int d) {
  if (!ok_t || c >= d) return make_uint4(0u, 0u, 0u, 0u);
  if (c + 8 <= d) return v;
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (c + e >= d) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
  return make_uint4(w[0], w[1], w[2], w[3]);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// MFMA operand fragment from token-major LDS rows (row pitch RP bf16): lane l of the wave
// receives channel ch0 + l % 32, tokens k0 + 8 (l / 32) .. + 7, via two LDS transpose
// reads.  Within each 16-lane group, lane s addresses token (s / 4) and channels
// 4 (s % 4) .. + 3 of its 16 channels; lane i of the group then holds 4 tokens of channel i.
__device__ __forceinline__ bf16x8 frag_tr(const uint16_t* base, int ch0, int k0, int lane) {
  const int g = lane >> 4, sl = lane & 15;
  const int ch = ch0 + 16 * (g & 1) + 4 * (sl & 3);
  const int tk = k0 + 8 * (g >> 1) + (sl >> 2);
  const uint16_t* p = base + tk * RP + ch;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 4 * RP));
  const short tmp[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  bf16x8 f;
  __builtin_memcpy(&f, tmp, sizeof(f));
  return f;
}

// Epilogue of one wave's NI x 4 blocks of 32 x 32 (lane l, element e -> row
// 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32 of a block).  With several splits the
// split's partial tile is stored for syrk_reduce_kernel.  With one split there is nothing
// to order, so the wave adds its blocks to C itself, with the masks and the diagonal check
// of the reduction kernel: the result is the reduction's C + (0 + p) bit for bit, since an
// accumulator that starts at +0 never holds -0.
template <int NI>
__device__ __forceinline__ void syrk_store_tile(const f32x16 (&acc)[NI][4], int r_base, int c_base, int lane,
                                                int split, int splits, int tile, int n_tiles, int ti, int tj,
                                                int d, float* __restrict__ partial, float* __restrict__ C,
                                                int64_t ldc, int32_t* __restrict__ info) {
  if (splits > 1) {
    float* part = partial + (int64_t(split) * n_tiles + tile) * (TB * TB);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int lr = r_base + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          const int lc = c_base + j * 32 + (lane & 31);
          part[lr * TB + lc] = acc[i][j][e];
        }
    return;
  }
  bool bad = false;
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = ti * TB + r_base + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int col = tj * TB + c_base + j * 32 + (lane & 31);
        if (row < d && col < d && col <= row) {
          float* c = C + int64_t(row) * ldc + col;
          const float v = *c + acc[i][j][e];
          *c = v;
          bad |= col == row && !isfinite(v);
        }
      }
  if (info && bad) *info = LRC_ENONFINITE;
}

// C[lower] += X^T Y over tokens [0, n) (X, Y: n x d bf16 bits, leading dim ldx).
// Workgroup -> (split, tile): consecutive workgroups land on consecutive XCDs, and XCD x
// takes one compact group of tiles for every split (grid.x = NXCD * tiles_per_xcd *
// splits), so the operand panels its tiles share are read through its own L2.
template <bool VEC>
__global__ __launch_bounds__(NTH, 1) void syrk_bf16_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Y, int64_t ldx, int64_t n, int d,
    int n1, int n_tiles, int tiles_per_xcd, int splits, int steps_per_split, float* __restrict__ partial,
    float* __restrict__ C, int64_t ldc, int32_t* __restrict__ info) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 2 * OPER];

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int wr = wave >> 1, wc = wave & 1;
  // on a diagonal tile the wave owning rows 0..127 x columns 128..255 lies entirely above
  // the diagonal and skips its MFMAs; every other block is computed (products above the
  // diagonal are valid and ignored by the reduction), so the MFMA stream has no branches
  const bool wave_dead = (ti == tj) && (wr < wc);

  // loader role: operand, 16-byte channel chunk, first token (tokens tok0 + 4 i, i < 16)
  const int op = tid >> 7;
  const int u = tid & 127;
  const int chunk = u & 31, tok0 = u >> 5;
  const uint16_t* src = op ? Y : X;
  const int chan = (op ? tj : ti) * TB + chunk * 8;

  const int64_t tok_begin = int64_t(split) * steps_per_split * KS;
  const int64_t tok_end = min<int64_t>(n, tok_begin + int64_t(steps_per_split) * KS);
  const int nsteps = tok_end > tok_begin ? int((tok_end - tok_begin + KS - 1) / KS) : 0;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // two stages of token rows in flight in registers, two in LDS
  uint4 pa[16], pb[16];
  auto load_stage = [&](uint4 (&r)[16], int64_t t0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = load_chunk<VEC>(src, ldx, t0 + tok0 + 4 * i, tok_end, chan, d);
  };
  auto store_stage = [&](const uint4 (&r)[16], int buf, int64_t t0) {
    uint16_t* dst = lds + (buf * 2 + op) * OPER + tok0 * RP + chunk * 8;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      *reinterpret_cast<uint4*>(dst + 4 * i * RP) = mask_chunk(r[i], t0 + tok0 + 4 * i < tok_end, chan, d);
  };
  auto compute = [&](int buf) {
    if (wave_dead) return;
    const uint16_t* xa = lds + (buf * 2 + 0) * OPER;
    const uint16_t* yb = lds + (buf * 2 + 1) * OPER;
#pragma unroll
    for (int kk = 0; kk < KS / 16; ++kk) {
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = frag_tr(xa, wr * 128 + i * 32, kk * 16, lane);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = frag_tr(yb, wc * 128 + j * 32, kk * 16, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };

  // Stage s computes from LDS buffer s & 1.  At its end the registers holding stage s + 1
  // (loaded two stages earlier, the oldest loads in flight) go to the other buffer and are
  // refilled with stage s + 3, so the loads of stage s + 2 stay in flight throughout.
  if (nsteps > 0) load_stage(pa, tok_begin);
  if (nsteps > 1) load_stage(pb, tok_begin + KS);
  if (nsteps > 0) store_stage(pa, 0, tok_begin);
  if (nsteps > 2) load_stage(pa, tok_begin + 2 * KS);
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {
    compute(0);
    if (s + 1 < nsteps) store_stage(pb, 1, tok_begin + int64_t(s + 1) * KS);
    if (s + 3 < nsteps) load_stage(pb, tok_begin + int64_t(s + 3) * KS);
    __syncthreads();
    if (s + 1 >= nsteps) break;
    compute(1);
    if (s + 2 < nsteps) store_stage(pa, 0, tok_begin + int64_t(s + 2) * KS);
    if (s + 4 < nsteps) load_stage(pa, tok_begin + int64_t(s + 4) * KS);
    __syncthreads();
  }

  // ---- epilogue: this split's partial tile, or the tile added to C (one split)
  syrk_store_tile<4>(acc, wr * 128, wc * 128, lane, split, splits, tile, n_tiles, ti, tj, d, partial, C, ldc, info);
}


// ---- bf16 SYRK with direct global -> LDS loads (channel count a multiple of 8, 16-byte
// aligned rows).  The same tiles, waves and MFMAs as above; the operands travel as
// buffer loads straight into LDS (16 bytes per lane, no staging registers), four LDS
// stages of 32 tokens, three of them in flight while one is computed.  A buffer resource
// per operand spans exactly the split's tokens, so rows past the split (and channels
// past d, by an out-of-range offset) read as zeros without any masking code.  Token rows
// sit unpadded (512 bytes) with their 16-byte granules XOR-swizzled by the token index
// (granule g of token t at slot g ^ 4 (t % 4)), so the transposing fragment reads of four
// consecutive tokens fall on four different bank groups.
constexpr int KS2 = 32;                  // tokens per stage
constexpr int NSTG = 4;                  // LDS stages
constexpr int ROWB = TB * 2;             // bytes per token row of one operand
constexpr int OPB = KS2 * ROWB;          // 16 KB: one operand, one stage
constexpr int STB = 2 * OPB;             // 32 KB: one stage

typedef __attribute__((address_space(3))) void lds_void_t;

// Stage barrier: wait until at most N vector memory operations of this wave are
// outstanding and all its LDS reads have returned (a buffer may be refilled by any wave
// once everyone has passed the barrier), then synchronise the workgroup.  Written out
// because the fence of __syncthreads would also wait for the direct loads still in flight.
#define LRC_VMCNT_BARRIER(N) asm volatile("s_waitcnt vmcnt(" #N ") lgkmcnt(0)\n\ts_barrier" ::: "memory")

__device__ __forceinline__ bf16x8 frag_sw(const uint8_t* base, int off) {
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + off));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + off + 4 * ROWB));
  const short tmp[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  bf16x8 f;
  __builtin_memcpy(&f, tmp, sizeof(f));
  return f;
}

// byte offset in a stage operand of lane `lane`'s first transposed read for the 32-channel
// block starting at channel ch0 (token 0 of the stage; later 16-token steps add 16 rows)
__device__ __forceinline__ int frag_off(int ch0, int lane) {
  const int g = lane >> 4, sl = lane & 15;
  const int ch = ch0 + 16 * (g & 1) + 4 * (sl & 3);
  const int tk = 8 * (g >> 1) + (sl >> 2);
  return tk * ROWB + (((ch >> 3) ^ (4 * (tk & 3))) << 4) + (ch & 7) * 2;
}

// DL_NW waves per workgroup (4 or 8): wave (wr, wc) owns rows wr RB .. + RB of the tile
// (RB = 512 / DL_NW) and columns wc 128 .. + 128, i.e. (RB / 32) x 4 blocks of 32 x 32.
// Eight waves measured faster (1.044 against 1.086 ms for 65536 tokens x 4096): four
// waves read half the fragments per MFMA but leave one wave per SIMD to hide latency.
constexpr int DL_NW = 8;
__global__ __launch_bounds__(64 * DL_NW, 1) void syrk_bf16_dl_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Y, int64_t ldx, int64_t n, int d, int n1,
    int n_tiles, int tiles_per_xcd, int splits, int64_t tok_per_split, float* __restrict__ partial,
    float* __restrict__ C, int64_t ldc, int32_t* __restrict__ info) {
  constexpr int LDPW = OPB / 1024 / DL_NW;  // 1 KB loads per wave per operand per stage
  constexpr int RB = TB / (DL_NW / 2);      // rows of a wave's block
  constexpr int NI = RB / 32;
  // one LDS object per stage: the compiler tracks the direct loads per object, so a read
  // of one stage waits only for that stage's loads (with a shared array it would wait for
  // all of them)
  __shared__ __attribute__((aligned(1024))) uint8_t sb0[STB], sb1[STB], sb2[STB], sb3[STB];
  static_assert(NSTG == 4, "one LDS object per stage: sb0 .. sb3");

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  // on a diagonal tile a block wholly above the diagonal is skipped
  const bool wave_dead = (ti == tj) && (wr * RB + RB - 1 < wc * 128);

  const int64_t tok_begin = int64_t(split) * tok_per_split;
  const int64_t tok_end = min<int64_t>(n, tok_begin + tok_per_split);
  const int nsteps = tok_end > tok_begin ? int((tok_end - tok_begin + KS2 - 1) / KS2) : 0;
  // buffer resources over the split's token rows (the launch keeps them below 2^31 bytes);
  // every field is workgroup-uniform, which readfirstlane makes explicit (scalar registers)
  const int nrec = __builtin_amdgcn_readfirstlane(int((tok_end - tok_begin) * ldx * 2));
  auto uniform_ptr = [](const uint16_t* p) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
    return reinterpret_cast<void*>((uint64_t(hi) << 32) | lo);
  };
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(X + tok_begin * ldx), 0, nrec, 0x00020000);
  const __amdgpu_buffer_rsrc_t ry =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(Y + tok_begin * ldx), 0, nrec, 0x00020000);

  // lane byte offsets of its loads: operand op, load j covers token rows 2 q, 2 q + 1
  // (q = LDPW wave + j) of the stage, lane -> row 2 q + lane / 32, LDS slot lane % 32
  unsigned voff[2][LDPW];
#pragma unroll
  for (int op = 0; op < 2; ++op)
#pragma unroll
    for (int j = 0; j < LDPW; ++j) {
      const int q = LDPW * wave + j;
      const int t = 2 * q + (lane >> 5);
      const int gch = (lane & 31) ^ (4 * (t & 3));
      const int chan = (op ? tj : ti) * TB + 8 * gch;
      voff[op][j] = chan < d ? unsigned((int64_t(t) * ldx + chan) * 2) : 0x80000000u;
    }
  auto issue = [&](uint8_t* dst, int st) {
    const int soff = int(int64_t(st) * KS2 * ldx * 2);
#pragma unroll
    for (int j = 0; j < LDPW; ++j) {
      const int q = LDPW * wave + j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(dst + q * 1024), 16, voff[0][j], soff, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ry, (lds_void_t*)(dst + OPB + q * 1024), 16, voff[1][j], soff, 0,
                                               0);
    }
  };

  int offa[NI], offb[4];
#pragma unroll
  for (int i = 0; i < NI; ++i) offa[i] = frag_off(wr * RB + i * 32, lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) offb[j] = frag_off(wc * 128 + j * 32, lane);

  f32x16 acc[NI][4];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // A stage is two 16-token halves.  Fragment sets: F0 holds a stage's first half, F1
  // its second half.
  static_assert(KS2 == 32, "two 16-token halves per stage");
  bf16x8 fa0[NI], fb0[4], fa1[NI], fb1[4];
  auto read_half = [&](const uint8_t* xa, int half, bf16x8* fa, bf16x8* fb) {
    const uint8_t* yb = xa + OPB;
#pragma unroll
    for (int i = 0; i < NI; ++i) fa[i] = frag_sw(xa + half * 16 * ROWB, offa[i]);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = frag_sw(yb + half * 16 * ROWB, offb[j]);
  };
  auto mma = [&](const bf16x8* fa, const bf16x8* fb) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };

  // Schedule (four stage buffers, stage s in buffer s mod 4).  Iteration s: read the
  // second half of stage s, run the MFMAs of its first half, then a barrier that waits
  // for stage s + 1.  At that barrier this wave's loads of s + 1 are the oldest of three
  // stages outstanding (2 LDPW loads each), so vmcnt(4 LDPW) leaves the two newer ones in
  // flight; afterwards stage s + 1 is in LDS and every wave has read all of stage s
  // (lgkmcnt(0) before the barrier), so buffer s mod 4 takes stage s + 4.  Then read the
  // first half of stage s + 1 and run the MFMAs of the second half of stage s: the MFMA
  // pipe never waits on a fragment read across the barrier.  The steady loop is unrolled
  // over the four buffers so that every access names its buffer; the last stages select
  // buffers at run time and wait for everything.  A wave whose block lies above the
  // diagonal of a diagonal tile only loads and synchronises.
  auto stage_barrier = [&]() {
    static_assert(LDPW == 2 || LDPW == 4, "four or eight waves");
    if constexpr (LDPW == 4) {
      LRC_VMCNT_BARRIER(16);
    } else {
      LRC_VMCNT_BARRIER(8);
    }
  };
  auto first_barrier = [&]() {  // stage 0 of four outstanding
    if constexpr (LDPW == 4) {
      LRC_VMCNT_BARRIER(24);
    } else {
      LRC_VMCNT_BARRIER(12);
    }
  };
  auto buf = [&](int st) -> uint8_t* {
    const int k = st & 3;
    return k == 0 ? sb0 : k == 1 ? sb1 : k == 2 ? sb2 : sb3;
  };
  // the first four stages unconditionally (every split has at least one): stages past
  // the split read zeros
  issue(sb0, 0);
  issue(sb1, 1);
  issue(sb2, 2);
  issue(sb3, 3);
  first_barrier();
  int s = 0;
  if (!wave_dead) {
    read_half(sb0, 0, fa0, fb0);
#define LRC_DL_STEP(CUR, NXT, NEXT_ISSUE) \
  read_half(CUR, 1, fa1, fb1);            \
  mma(fa0, fb0);                          \
  stage_barrier();                        \
  issue(CUR, NEXT_ISSUE);                 \
  __builtin_amdgcn_sched_barrier(0);      \
  read_half(NXT, 0, fa0, fb0);            \
  mma(fa1, fb1);
    for (; s + 7 < nsteps; s += 4) {
      LRC_DL_STEP(sb0, sb1, s + 4)
      LRC_DL_STEP(sb1, sb2, s + 5)
      LRC_DL_STEP(sb2, sb3, s + 6)
      LRC_DL_STEP(sb3, sb0, s + 7)
    }
#undef LRC_DL_STEP
    for (; s < nsteps; ++s) {
      read_half(buf(s), 1, fa1, fb1);
      mma(fa0, fb0);
      if (s + 1 < nsteps) {
        if (s + 4 < nsteps) {  // stages s + 2 and s + 3 are outstanding
          stage_barrier();
          issue(buf(s), s + 4);
        } else {
          LRC_VMCNT_BARRIER(0);
        }
        read_half(buf(s + 1), 0, fa0, fb0);
      }
      mma(fa1, fb1);
    }
  } else {
    for (; s + 1 < nsteps; ++s) {
      if (s + 4 < nsteps) {
        stage_barrier();
        issue(buf(s), s + 4);
      } else {
        LRC_VMCNT_BARRIER(0);
      }
    }
  }
  // prologue loads of stages past a short split may still be in flight
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  syrk_store_tile<NI>(acc, wr * RB, wc * 128, lane, split, splits, tile, n_tiles, ti, tj, d, partial, C, ldc, info);
}

// C[lower] += sum over splits of the partial tiles, in split order (bit-reproducible).
// Block (tile, q) handles 256 consecutive float4 of the tile; loads are batched 8 splits
// at a time from clamped addresses, then masked.  A diagonal entry of C is a sum of
// squares, so a NaN or Inf anywhere in column i of the tokens (or an overflow) makes
// C[i][i] non-finite; the thread holding it then sets *info (when given).
__global__ __launch_bounds__(256) void syrk_reduce_kernel(const float* __restrict__ partial, int splits, int n_tiles,
                                                          int n1, int d, float* __restrict__ C, int64_t ldc,
                                                          int vec4, int32_t* __restrict__ info) {
  const int tile = blockIdx.x;
  const TileRC tc = tile_of(tile, n1);
  const int idx = blockIdx.y * 256 + threadIdx.x;   // float4 index within the tile
  const int lr = (idx * 4) / TB, lc = (idx * 4) % TB;
  const int row = tc.ti * TB + lr, col0 = tc.tj * TB + lc;
  if (row >= d || col0 >= d) return;
  if (tc.ti == tc.tj && col0 > row) return;   // entirely above the diagonal
  const int64_t pstride = int64_t(n_tiles) * TB * TB;
  const float* pb = partial + int64_t(tile) * TB * TB + idx * 4;
  f32x4 sum = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const f32x4*>(pb + int64_t(min(s0 + u, splits - 1)) * pstride);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      sum += (s0 + u < splits) ? v[u] : z;
    }
  }
  float* c = C + int64_t(row) * ldc + col0;
  if (vec4 && col0 + 3 < d && (tc.ti != tc.tj || col0 + 3 <= row)) {
    f32x4 cv = *reinterpret_cast<const f32x4*>(c);
    cv += sum;
    *reinterpret_cast<f32x4*>(c) = cv;
    if (info && row == col0 + 3 && !isfinite(cv[3])) *info = LRC_ENONFINITE;
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int col = col0 + e;
    if (col < d && (tc.ti != tc.tj || col <= row)) {
      const float v = c[e] + sum[e];
      c[e] = v;
      if (info && col == row && !isfinite(v)) *info = LRC_ENONFINITE;
    }
  }
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

// The same pre-pass for bf16 rows of at most QAW_VROW elements (a multiple of 8, rows
// 16-byte aligned): each thread holds its 16-byte pieces of the row in registers, so the
// row is read from memory once, and the three outputs are written as 16-byte pieces.  The
// arithmetic per element is that of qaw_prepass_kernel, so the outputs are the same bits.
constexpr int QAW_VPT = 8;                       // 16-byte pieces per thread
constexpr int QAW_VROW = 256 * 8 * QAW_VPT;      // 16384 elements
typedef uint32_t qaw_u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void qaw_prepass_vec_kernel(const uint16_t* __restrict__ A, int64_t lda, int d,
                                                              uint16_t* __restrict__ Q, uint16_t* __restrict__ H,
                                                              uint16_t* __restrict__ L, int64_t ldq) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const qaw_u32x4* row = reinterpret_cast<const qaw_u32x4*>(A + t * lda);
  const int nv = d / 8;
  qaw_u32x4 v[QAW_VPT];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < QAW_VPT; ++i) {
    const int j = threadIdx.x + 256 * i;
    v[i] = j < nv ? row[j] : qaw_u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m = fmaxf(m, fabsf(__uint_as_float(v[i][e] << 16)));
      m = fmaxf(m, fabsf(__uint_as_float(v[i][e] & 0xffff0000u)));
    }
  }
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = __fdiv_rn(m, 127.0f);
  const float s2 = s * s;
  qaw_u32x4* q4 = reinterpret_cast<qaw_u32x4*>(Q + t * ldq);
  qaw_u32x4* h4 = reinterpret_cast<qaw_u32x4*>(H + t * ldq);
  qaw_u32x4* l4 = reinterpret_cast<qaw_u32x4*>(L + t * ldq);
#pragma unroll
  for (int i = 0; i < QAW_VPT; ++i) {
    const int j = threadIdx.x + 256 * i;
    if (j >= nv) continue;
    qaw_u32x4 qo, ho, lo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t qw = 0u, hw = 0u, lw = 0u;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const float a = __uint_as_float(half ? (v[i][e] & 0xffff0000u) : (v[i][e] << 16));
        float q = 0.f;
        if (s > 0.f) q = fminf(fmaxf(rintf(__fdiv_rn(a, s)), -127.f), 127.f);
        const float w = s2 * q;
        const uint16_t hb = f32_to_bf16_bits(w);
        const uint16_t lb = f32_to_bf16_bits(w - bf16_bits_to_f32(hb));
        qw |= uint32_t(f32_to_bf16_bits(q)) << (16 * half);
        hw |= uint32_t(hb) << (16 * half);
        lw |= uint32_t(lb) << (16 * half);
      }
      qo[e] = qw;
      ho[e] = hw;
      lo[e] = lw;
    }
    q4[j] = qo;
    h4[j] = ho;
    l4[j] = lo;
  }
}

// ---- fp32 input: plain LDS-tiled SYRK, 64 x 64 lower tiles, no split (deterministic)
__global__ __launch_bounds__(256) void syrk_f32_kernel(const float* __restrict__ A, int64_t lda, int64_t n,
                                                       int d, float* __restrict__ C, int64_t ldc,
                                                       int32_t* __restrict__ info) {
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
      if (row < d && col < d && row >= col) {
        const float v = C[int64_t(row) * ldc + col] + acc[i][j];
        C[int64_t(row) * ldc + col] = v;
        // a diagonal entry is a sum of squares: non-finite iff a token entry of this
        // column is (or the sum overflowed)
        if (info && row == col && !isfinite(v)) *info = LRC_ENONFINITE;
      }
    }
}

struct SyrkPlan {
  int n1, n_tiles, tiles_per_xcd, splits, steps_per_split;
  int64_t grid;
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
  // cost model: workgroup rounds x (steps per workgroup + partial write overhead; a
  // split's 256 KB partial tile costs about as much time as 16 steps of MFMA work)
  int best = 1;
  double best_cost = 1e300;
  const int smax = int(std::min<int64_t>(std::max(1, max_splits), std::max<int64_t>(1, nsteps)));
  for (int s = 1; s <= smax; ++s) {
    const double rounds = double(cdiv(int64_t(NXCD) * p.tiles_per_xcd * s, cus));
    const double cost = rounds * (double(cdiv(nsteps, s)) + 16.0);
    if (cost < best_cost - 1e-9) { best_cost = cost; best = s; }
  }
  p.steps_per_split = int(cdiv(nsteps, best));
  p.splits = int(cdiv(nsteps, p.steps_per_split));  // drop empty splits
  if (p.splits < 1) p.splits = 1;
  p.grid = int64_t(NXCD) * p.tiles_per_xcd * p.splits;
  return p;
}

size_t syrk_partial_floats(const SyrkPlan& p) { return size_t(p.splits) * p.n_tiles * TB * TB; }

// bf16 SYRK launch over a token block, partial/counter space from the carve
lrc_status launch_syrk_bf16(hipStream_t st, const uint16_t* X, const uint16_t* Y, int64_t ldx, int64_t n,
                            int64_t d, float* C, int64_t ldc, float* partial, int split_cap, int32_t* info) {
  if (n <= 0) return LRC_OK;
  const SyrkPlan p = plan_syrk(n, d, split_cap);  // never more splits than the partial buffer holds
  const bool vec = (d % 8 == 0) && (ldx % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(Y) & 15) == 0);
  const dim3 grid(unsigned(p.grid));
  // algorithmic work: n d (d + 1) / 2 products and adds for the lower triangle incl. the
  // diagonal; bytes: the token block once (twice when the two operands differ) plus one
  // read and one write of the fp32 lower triangle
  const double tri = double(d) * double(d + 1) / 2;
  ProfScope scope("syrk_bf16_kernel", st, 2.0 * double(n) * tri,
                  double(n) * double(d) * 2.0 * (X == Y ? 1 : 2) + 8.0 * tri);
  const int64_t tok_per_split = int64_t(p.steps_per_split) * KS;
  // direct-load kernel: buffer offsets of a split (rows of ldx bf16, plus the four
  // stages the pipeline may fetch past its end) must stay below 2^31
  if (vec && (tok_per_split + 4 * KS2) * ldx * 2 < (int64_t(1) << 31))
    syrk_bf16_dl_kernel<<<grid, 64 * DL_NW, 0, st>>>(X, Y, ldx, n, int(d), p.n1, p.n_tiles, p.tiles_per_xcd, p.splits,
                                                 tok_per_split, partial, C, ldc, info);
  else if (vec)
    syrk_bf16_kernel<true><<<grid, NTH, 0, st>>>(X, Y, ldx, n, int(d), p.n1, p.n_tiles, p.tiles_per_xcd,
                                                 p.splits, p.steps_per_split, partial, C, ldc, info);
  else
    syrk_bf16_kernel<false><<<grid, NTH, 0, st>>>(X, Y, ldx, n, int(d), p.n1, p.n_tiles, p.tiles_per_xcd,
                                                  p.splits, p.steps_per_split, partial, C, ldc, info);
  LRC_LAUNCHED();
  if (p.splits == 1) return LRC_OK;   // the kernel added its tiles to C
  const int vec4 = (ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(C) & 15) == 0);
  syrk_reduce_kernel<<<dim3(unsigned(p.n_tiles), unsigned(TB * TB / 4 / 256)), 256, 0, st>>>(
      partial, p.splits, p.n_tiles, p.n1, int(d), C, ldc, vec4, info);
  LRC_LAUNCHED();
  return LRC_OK;
}

size_t cov_workspace(lrc_dtype dt, int64_t n, int64_t d, uint32_t flags, void* base, float** partial,
                     uint16_t** q, uint16_t** h, uint16_t** l, int64_t* chunk, int* split_cap) {
  Carve cv(base);
  const bool quant = flags & LRC_COV_QUANT_INT8_TOKEN;
  int64_t nb = n;
  if (quant) nb = std::min<int64_t>(n, QAW_CHUNK);
  size_t pf = 0;
  int cap = 1;
  if (dt == LRC_BF16 || quant) {
    // launches see token blocks of nb tokens and, for QAW, one final block of n % nb
    SyrkPlan p = plan_syrk(std::max<int64_t>(nb, 1), d);
    cap = p.splits;
    if (quant && n % nb) cap = std::max(cap, plan_syrk(n % nb, d).splits);
    p.splits = cap;
    // one split everywhere: the SYRK adds its tiles to C itself, no partial tiles
    pf = cap > 1 ? syrk_partial_floats(p) : 0;
  }
  float* pp = cv.take<float>(pf);
  uint16_t *qq = nullptr, *hh = nullptr, *ll = nullptr;
  if (quant) {
    qq = cv.take<uint16_t>(size_t(nb) * d);
    hh = cv.take<uint16_t>(size_t(nb) * d);
    ll = cv.take<uint16_t>(size_t(nb) * d);
  }
  if (partial) *partial = pp;
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
  return cov_workspace(dt, n_tokens, d, flags, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
}

extern "C" lrc_status lrc_accumulate_cov(const void* A, lrc_dtype dt, int64_t n_tokens, int64_t d, int64_t lda,
                                         float* C, int64_t ldc, uint32_t flags, int32_t* info, void* ws,
                                         size_t ws_bytes, void* stream) {
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
  uint16_t *q = nullptr, *h = nullptr, *l = nullptr;
  int64_t chunk = 0;
  int cap = 1;
  cov_workspace(dt, n_tokens, d, flags, ws, &partial, &q, &h, &l, &chunk, &cap);
  const bool quant = flags & LRC_COV_QUANT_INT8_TOKEN;

  if (!quant && dt == LRC_F32) {
    const int tiles = int(cdiv(d, 64) * (cdiv(d, 64) + 1) / 2);
    const double tri = double(d) * double(d + 1) / 2;
    ProfScope scope("syrk_f32_kernel", st, 2.0 * double(n_tokens) * tri, double(n_tokens) * double(d) * 4.0 + 8.0 * tri);
    syrk_f32_kernel<<<tiles, 256, 0, st>>>(static_cast<const float*>(A), lda, n_tokens, int(d), C, ldc, info);
    LRC_LAUNCHED();
    return LRC_OK;
  }
  if (!quant) {
    const uint16_t* a = static_cast<const uint16_t*>(A);
    return launch_syrk_bf16(st, a, a, lda, n_tokens, d, C, ldc, partial, cap, info);
  }
  // 16-byte pieces: rows of a multiple of 8 elements, every buffer 16-byte aligned
  const bool qaw_vec = dt == LRC_BF16 && d % 8 == 0 && d <= QAW_VROW && lda % 8 == 0 &&
                       reinterpret_cast<uintptr_t>(A) % 16 == 0 && reinterpret_cast<uintptr_t>(q) % 16 == 0 &&
                       reinterpret_cast<uintptr_t>(h) % 16 == 0 && reinterpret_cast<uintptr_t>(l) % 16 == 0;
  for (int64_t t0 = 0; t0 < n_tokens; t0 += chunk) {
    const int64_t nb = std::min(chunk, n_tokens - t0);
    {
    ProfScope scope("qaw_prepass_kernel", st, 0.0, double(nb) * double(d) * ((dt == LRC_BF16 ? 2 : 4) + 6));
    if (qaw_vec)
      qaw_prepass_vec_kernel<<<unsigned(nb), 256, 0, st>>>(static_cast<const uint16_t*>(A) + t0 * lda, lda, int(d), q,
                                                           h, l, d);
    else if (dt == LRC_BF16)
      qaw_prepass_kernel<uint16_t><<<unsigned(nb), 256, 0, st>>>(static_cast<const uint16_t*>(A) + t0 * lda, lda,
                                                                 int(d), q, h, l, d);
    else
      qaw_prepass_kernel<float><<<unsigned(nb), 256, 0, st>>>(static_cast<const float*>(A) + t0 * lda, lda,
                                                              int(d), q, h, l, d);
    LRC_LAUNCHED();
    }
    LRC_TRY(launch_syrk_bf16(st, q, h, d, nb, d, C, ldc, partial, cap, info));
    LRC_TRY(launch_syrk_bf16(st, q, l, d, nb, d, C, ldc, partial, cap, info));
  }
  return LRC_OK;
}
