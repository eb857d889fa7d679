// Decode-time low-rank SwiGLU FFN with int8 factors.
//
// LASER technical summary, 4 (System Implementation): the low-rank FFN runs as fused
// kernels covering the input projection, the latent activations, SwiGLU and the
// quantisation/dequantisation steps, to cut memory movement and launches.  Reading:
// y = W_down (SiLU(W_gate x) * (W_up x)) with every W replaced by its factors L R, each an
// int8 matrix with one fp32 scale per row (as lrc_rotate_quantize writes them; a rotation
// between the factors leaves the product unchanged).  Activations and sums are fp32.
//
// Four launches per call, each reading its int8 factors once, in 16-byte rows pieces:
//   1. latent_g = R_gate x, latent_u = R_up x         (one wave per latent row)
//   2. for a chunk of hidden channels: expand both latents (rows of L_gate, L_up),
//      h = SiLU(gate) * up in LDS, and its share of R_down h (rows of R_down^T), written
//      as per-chunk partial latents
//   3. latent_d = sum of the partials in a fixed order, times R_down's row scales
//   4. y = L_down latent_d                              (one wave per output row)
// Tokens are handled TG at a time so every weight piece is dequantised once per group.
#include "lrc_internal.h"

namespace lrc {
namespace {

constexpr int FT = 256;      // threads per workgroup
constexpr int TG = 4;        // tokens per group
// hidden-channel chunks (workgroups of the expansion kernel): two workgroups of 8 waves per
// CU keep enough weight loads in flight, while each chunk's n_tok x r_down partial stays a
// small share of the traffic
constexpr int HC = 512;

__device__ __forceinline__ float wave_sumf(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ void unpack16(uint4 w, float (&f)[16]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 16; ++i) f[i] = float(int8_t(uint8_t(u[i >> 2] >> (8 * (i & 3)))));
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// out[t][row] = scale[row] * (q[row] . v[t]) for the rows of one or two int8 matrices
// (rows0 rows of q0, then rows1 rows of q1; each row n int8, n % 16 == 0).  One wave per
// row, GW / 64 rows per workgroup; the activations of a token group pass through LDS in
// XC-column chunks, so each is read from L2 once per workgroup rather than once per row.
// A lane takes 4-byte weight pieces 256 columns apart, eight in flight, and the matching
// float4 of each token from LDS (consecutive lanes, consecutive 16 bytes: no bank conflicts).
constexpr int GW = 1024;
constexpr int XC = 2048;
__global__ __launch_bounds__(GW) void rows_gemv_kernel(const int8_t* __restrict__ q0, const float* __restrict__ s0,
                                                       int rows0, const int8_t* __restrict__ q1,
                                                       const float* __restrict__ s1, int rows1, int n,
                                                       const float* __restrict__ v, int n_tok,
                                                       float* __restrict__ out0, float* __restrict__ out1,
                                                       int accumulate = 0) {
  __shared__ float4 xs[TG][XC / 4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int row = blockIdx.x * (GW / 64) + (tid >> 6);
  const bool live = row < rows0 + rows1;   // waves past the last row still join the staging
  const int rw = live ? row : rows0 + rows1 - 1;
  const bool first = rw < rows0;
  const int r = first ? rw : rw - rows0;
  const int8_t* q = (first ? q0 : q1) + int64_t(r) * n;
  const float sc = first ? s0[r] : s1[r];
  float* out = first ? out0 : out1;
  const int ld_out = first ? rows0 : rows1;
  for (int t0 = 0; t0 < n_tok; t0 += TG) {
    float acc[TG] = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < n; c0 += XC) {
      const int nc4 = min(XC, n - c0) / 4;
      __syncthreads();
      for (int i = tid; i < TG * nc4; i += GW) {
        const int t = i / nc4, k4 = i % nc4;
        xs[t][k4] = t0 + t < n_tok ? reinterpret_cast<const float4*>(v + int64_t(t0 + t) * n + c0)[k4]
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      __syncthreads();
      if (live) {
        uint32_t wq[8];
#pragma unroll
        for (int p = 0; p < 8; ++p)
          wq[p] = *reinterpret_cast<const uint32_t*>(q + c0 + 4 * min(lane + 64 * p, nc4 - 1));
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const int k4 = lane + 64 * p;
          if (k4 < nc4) {
            float w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = float(int8_t(uint8_t(wq[p] >> (8 * e))));
#pragma unroll
            for (int t = 0; t < TG; ++t) {
              const float4 xv = xs[t][k4];
              acc[t] += w[0] * xv.x + w[1] * xv.y + w[2] * xv.z + w[3] * xv.w;
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const float a = wave_sumf(acc[t]);
      if (live && lane == 0 && t0 + t < n_tok) {
        float* o = out + int64_t(t0 + t) * ld_out + r;
        *o = accumulate ? *o + sc * a : sc * a;
      }
    }
  }
}

// The same product for a single token: one wave per row, a lane's four 16-byte weight
// pieces in flight together and the activation read straight from L2 (at one token the
// re-reads cost less than the loads in flight that LDS staging gives up)
__global__ __launch_bounds__(FT) void rows_gemv1_kernel(const int8_t* __restrict__ q0, const float* __restrict__ s0,
                                                       int rows0, const int8_t* __restrict__ q1,
                                                       const float* __restrict__ s1, int rows1, int n,
                                                       const float* __restrict__ v, int n_tok,
                                                       float* __restrict__ out0, float* __restrict__ out1,
                                                       int accumulate = 0) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (FT / 64) + (threadIdx.x >> 6);
  if (row >= rows0 + rows1) return;
  const bool first = row < rows0;
  const int r = first ? row : row - rows0;
  const int8_t* q = (first ? q0 : q1) + int64_t(r) * n;
  const float sc = first ? s0[r] : s1[r];
  float* out = first ? out0 : out1;
  const int ld_out = first ? rows0 : rows1;
  for (int t0 = 0; t0 < n_tok; t0 += TG) {
    float acc[TG] = {0.f, 0.f, 0.f, 0.f};
    for (int jb = lane * 16; jb < n; jb += 4 * 64 * 16) {
      uint4 wq[4];   // the lane's next four 16-byte pieces, all in flight before any use
#pragma unroll
      for (int p = 0; p < 4; ++p) wq[p] = *reinterpret_cast<const uint4*>(q + min(jb + p * 1024, n - 16));
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int j0 = jb + p * 1024;
        if (j0 < n) {
          float w[16];
          unpack16(wq[p], w);
#pragma unroll
          for (int t = 0; t < TG; ++t) {
            if (t0 + t < n_tok) {
              const float4* x = reinterpret_cast<const float4*>(v + int64_t(t0 + t) * n + j0);
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const float4 xv = x[c];
                acc[t] += w[4 * c] * xv.x + w[4 * c + 1] * xv.y + w[4 * c + 2] * xv.z + w[4 * c + 3] * xv.w;
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const float a = wave_sumf(acc[t]);
      if (lane == 0 && t0 + t < n_tok) {
        float* o = out + int64_t(t0 + t) * ld_out + r;
        *o = accumulate ? *o + sc * a : sc * a;
      }
    }
  }
}


// row GEMV launch: the single-token kernel at n_tok == 1, the LDS-staged one otherwise
void launch_rows_gemv(hipStream_t st, const int8_t* q0, const float* s0, int rows0, const int8_t* q1, const float* s1,
                      int rows1, int n, const float* v, int n_tok, float* out0, float* out1, int accumulate) {
  const int rows = rows0 + rows1;
  if (n_tok == 1)
    rows_gemv1_kernel<<<unsigned(cdiv(rows, FT / 64)), FT, 0, st>>>(q0, s0, rows0, q1, s1, rows1, n, v, n_tok, out0,
                                                                     out1, accumulate);
  else
    rows_gemv_kernel<<<unsigned(cdiv(rows, GW / 64)), GW, 0, st>>>(q0, s0, rows0, q1, s1, rows1, n, v, n_tok, out0,
                                                                    out1, accumulate);
}

// LDS slot of latent index k: one spare slot after every 16, so the 16 lanes of a row,
// which start 16 indices apart, fall in distinct banks (unpadded, the four-token layout
// puts all 16 on one bank group)
__host__ __device__ __forceinline__ int64_t pslot(int64_t k) { return k + (k >> 4); }

// Hidden channels [b J, b J + J): gate/up expansion, SwiGLU, and the chunk's partial of
// R_down h: pd[b][t][k] = sum_j q_rdt[j][k] h[t][j] (R_down's row scales come later).
// NG tokens per group (1 or TG); with TG the latents sit in LDS token-interleaved
// ([k][t]), so one 16-byte read serves the four tokens of a weight element.
constexpr int FE = 512;      // threads per workgroup of the expansion kernel
constexpr int DK = FE / 2 * 8;   // down-projection outputs per pass (8 per thread of a half)

template <int NG>
__global__ __launch_bounds__(FE) void swiglu_down_kernel(const int8_t* __restrict__ qlg, const float* __restrict__ slg,
                                                         const int8_t* __restrict__ qlu, const float* __restrict__ slu,
                                                         int rg, int ru, const float* __restrict__ latg,
                                                         const float* __restrict__ latu,
                                                         const int8_t* __restrict__ qrdt, int rd, int d_ff, int J,
                                                         int n_tok, float* __restrict__ pd) {
  extern __shared__ float sh[];
  // one latent at a time in LDS ([slot(k)][NG]): the gate pass, then the up pass over the
  // same region, so the footprint is one latent and several workgroups fit on a CU
  float* lat = sh;                             // also the down pass's exchange buffer [NG][DK]
  float* gg = lat + NG * max(int(pslot(max(rg, ru))), DK);   // [NG][J] scaled gate pre-activations
  float* hh = gg + NG * J;                     // [NG][J]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j0 = blockIdx.x * J;
  const int jn = min(J, d_ff - j0);
  const int sub = lane >> 4, sl = lane & 15;
  // one expansion pass: for the chunk's rows j, out(j, t) = row j of q (r int8) . latent t,
  // a wave taking four rows at a time with 16 lanes per row (lanes split the latent index),
  // every weight load of the four rows issued before any use; fin(jj, t, sum) stores it
  auto expand = [&](const int8_t* __restrict__ q, int r, const float* __restrict__ src, int nt, int t0,
                    auto fin) {
    __syncthreads();
    for (int i = tid; i < NG * r; i += FE) {
      const int t = i / r, k = i % r;
      lat[pslot(k) * NG + t] = t < nt ? src[int64_t(t0 + t) * r + k] : 0.f;
    }
    __syncthreads();
    for (int jb = wave * 4; jb < jn; jb += FE / 16) {
      const int jj = jb + sub;
      const int j = j0 + min(jj, jn - 1);
      float a[TG] = {0.f, 0.f, 0.f, 0.f};
      for (int k0 = sl * 16; k0 < r; k0 += 16 * 16 * 4) {
        uint4 wq[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int k = min(k0 + c * 256, r - 16);
          wq[c] = *reinterpret_cast<const uint4*>(q + int64_t(j) * r + k);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int k = k0 + c * 256;
          if (k < r) {
            float w[16];
            unpack16(wq[c], w);
            if constexpr (NG == 1) {
#pragma unroll
              for (int e = 0; e < 16; ++e) a[0] += w[e] * lat[pslot(k) + e];
            } else {
#pragma unroll
              for (int e = 0; e < 16; ++e) {
                const float4 lv = *reinterpret_cast<const float4*>(lat + (pslot(k) + e) * NG);
                a[0] += w[e] * lv.x;
                a[1] += w[e] * lv.y;
                a[2] += w[e] * lv.z;
                a[3] += w[e] * lv.w;
              }
            }
          }
        }
      }
#pragma unroll
      for (int t = 0; t < NG; ++t) {
        float s = a[t];
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) s += __shfl_xor(s, o);   // sum over the row's 16 lanes
        if (sl == 0 && jj < jn) fin(jj, j, t, s);
      }
    }
  };
  for (int t0 = 0; t0 < n_tok; t0 += NG) {
    const int nt = min(NG, n_tok - t0);
    expand(qlg, rg, latg, nt, t0, [&](int jj, int j, int t, float s) { gg[t * J + jj] = slg[j] * s; });
    expand(qlu, ru, latu, nt, t0,
           [&](int jj, int j, int t, float s) { hh[t * J + jj] = silu(gg[t * J + jj]) * (slu[j] * s); });
    __syncthreads();
    // R_down's share: the two halves of the workgroup take the two halves of the chunk's
    // channels for the same 8 outputs per thread; the upper half's sums pass through LDS
    // and are added to the lower half's
    const int half = tid / (FE / 2), ht = tid % (FE / 2);
    const int jh = (jn + 1) / 2, r0 = half ? jh : 0, r1 = half ? jn : jh;
    for (int kp = 0; kp < rd; kp += DK) {
      const int kb = kp + ht * 8;
      const bool act = kb < rd;
      float acc[NG][8];
#pragma unroll
      for (int t = 0; t < NG; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[t][e] = 0.f;
      for (int jb = r0; act && jb < r1; jb += 8) {
        uint2 w8[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
          w8[c] = *reinterpret_cast<const uint2*>(qrdt + int64_t(j0 + min(jb + c, r1 - 1)) * rd + kb);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          if (jb + c < r1) {
            const uint32_t wu[2] = {w8[c].x, w8[c].y};
            float w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = float(int8_t(uint8_t(wu[e >> 2] >> (8 * (e & 3)))));
#pragma unroll
            for (int t = 0; t < NG; ++t) {
              if (t < nt) {
                const float hv = hh[t * J + jb + c];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[t][e] += w[e] * hv;
              }
            }
          }
        }
      }
      if (half == 1 && act) {
#pragma unroll
        for (int t = 0; t < NG; ++t)
#pragma unroll
          for (int e = 0; e < 8; ++e) lat[t * DK + ht * 8 + e] = acc[t][e];
      }
      __syncthreads();
      if (half == 0 && act) {
#pragma unroll
        for (int t = 0; t < NG; ++t) {
          if (t < nt) {
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = acc[t][e] + lat[t * DK + ht * 8 + e];
            float4* dst = reinterpret_cast<float4*>(pd + (int64_t(blockIdx.x) * n_tok + t0 + t) * rd + kb);
            dst[0] = make_float4(o[0], o[1], o[2], o[3]);
            dst[1] = make_float4(o[4], o[5], o[6], o[7]);
          }
        }
      }
      __syncthreads();
    }
  }
}

// dense hidden channels: g[i] <- SiLU(g[i]) * u[i] (n_tok x n_dense, in place)
__global__ __launch_bounds__(FT) void swiglu_dense_kernel(float* __restrict__ g, const float* __restrict__ u,
                                                          int64_t cnt) {
  const int64_t i = int64_t(blockIdx.x) * FT + threadIdx.x;
  if (i < cnt) g[i] = silu(g[i]) * u[i];
}

// latent_d[t][k] = s_rd[k] * sum over chunks b of pd[b][t][k]: a workgroup takes RO
// consecutive outputs and RS slices of the chunks, each thread summing its slice in chunk
// order (16 loads in flight), the slices then added in slice order
constexpr int RO = 16, RS = FT / RO;
__global__ __launch_bounds__(FT) void latent_reduce_kernel(const float* __restrict__ pd, int nb, int n_tok, int rd,
                                                           const float* __restrict__ srd, float* __restrict__ latd) {
  __shared__ float part[RS][RO];
  const int sl = threadIdx.x / RO, o = threadIdx.x % RO;
  const int64_t i = int64_t(blockIdx.x) * RO + o;
  const int64_t tot = int64_t(n_tok) * rd;
  const int64_t ic = min(i, tot - 1);
  const int per = (nb + RS - 1) / RS, b0 = min(nb, sl * per), b1 = min(nb, b0 + per);
  float s = 0.f;
  for (int b = b0; b < b1; b += 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = pd[int64_t(min(b + u, b1 - 1)) * tot + ic];
#pragma unroll
    for (int u = 0; u < 16; ++u) s += b + u < b1 ? v[u] : 0.f;
  }
  part[sl][o] = s;
  __syncthreads();
  if (sl == 0 && i < tot) {
    float t = part[0][o];
    for (int q = 1; q < RS; ++q) t += part[q][o];
    latd[i] = srd[int(i % rd)] * t;
  }
}

}  // namespace
}  // namespace lrc

using namespace lrc;

namespace {
struct FfnWs {
  float *latg, *latu, *pd, *latd;
};
FfnWs carve_ffn(Carve& cv, int64_t n_tok, int64_t rg, int64_t ru, int64_t rd, int64_t nb) {
  FfnWs w;
  w.latg = cv.take<float>(size_t(n_tok * rg));
  w.latu = cv.take<float>(size_t(n_tok * ru));
  w.pd = cv.take<float>(size_t(nb * n_tok * rd));
  w.latd = cv.take<float>(size_t(n_tok * rd));
  return w;
}
int64_t ffn_chunk(int64_t d_ff) { return cdiv(d_ff, HC); }
}  // namespace

extern "C" size_t lrc_lowrank_ffn_workspace(int64_t n_tok, int64_t d_ff, int64_t rg, int64_t ru, int64_t rd) {
  if (n_tok <= 0 || d_ff <= 0 || rg <= 0 || ru <= 0 || rd <= 0) return 0;
  Carve cv(nullptr);
  carve_ffn(cv, n_tok, rg, ru, rd, cdiv(d_ff, ffn_chunk(d_ff)));
  return cv.bytes();
}

extern "C" lrc_status lrc_lowrank_ffn(const float* x, int64_t n_tok, int64_t d, int64_t d_ff, const int8_t* q_rg,
                                      const float* s_rg, const int8_t* q_lg, const float* s_lg, int64_t rg,
                                      const int8_t* q_ru, const float* s_ru, const int8_t* q_lu, const float* s_lu,
                                      int64_t ru, const int8_t* q_rdt, const float* s_rd, const int8_t* q_ld,
                                      const float* s_ld, int64_t rd, float* y, void* ws, size_t ws_bytes,
                                      void* stream) {
  const void* ptrs[] = {x, q_rg, s_rg, q_lg, s_lg, q_ru, s_ru, q_lu, s_lu, q_rdt, s_rd, q_ld, s_ld, y};
  for (const void* p : ptrs)
    if (p == nullptr) return LRC_EINVAL;
  // 16-byte pieces of every int8 row and of the activations
  for (const void* p : {(const void*)x, (const void*)q_rg, (const void*)q_lg, (const void*)q_ru, (const void*)q_lu,
                        (const void*)q_ld})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return LRC_EINVAL;
  if (reinterpret_cast<uintptr_t>(q_rdt) % 8 != 0) return LRC_EINVAL;
  if (n_tok <= 0 || d <= 0 || d_ff <= 0 || rg <= 0 || ru <= 0 || rd <= 0) return LRC_EINVAL;
  if (d % 16 || rg % 16 || ru % 16 || rd % 16) return LRC_EINVAL;
  if (n_tok > (int64_t(1) << 20) || d > (int64_t(1) << 24) || d_ff > (int64_t(1) << 24)) return LRC_EINVAL;
  const int64_t J = ffn_chunk(d_ff), nb = cdiv(d_ff, J);
  const size_t lds = sizeof(float) * size_t(TG * std::max(pslot(std::max(rg, ru)), int64_t(DK)) + 2 * TG * J);
  if (lds > 160 * 1024) return LRC_EINVAL;   // the larger latent of a token group must fit in LDS
  const size_t need = lrc_lowrank_ffn_workspace(n_tok, d_ff, rg, ru, rd);
  if (ws == nullptr || ws_bytes < need) return LRC_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the expansion kernel's LDS (one latent of a token group at a time) may exceed the default cap
  const int ng = n_tok == 1 ? 1 : TG;
  const size_t lds_used = sizeof(float) * size_t(ng * std::max(pslot(std::max(rg, ru)), int64_t(DK)) + 2 * ng * J);
  if (lds_used > 64 * 1024)
    LRC_HIP(hipFuncSetAttribute(ng == 1 ? reinterpret_cast<const void*>(&swiglu_down_kernel<1>)
                                        : reinterpret_cast<const void*>(&swiglu_down_kernel<TG>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds_used)));
  Carve cv(ws);
  const FfnWs w = carve_ffn(cv, n_tok, rg, ru, rd, nb);
  // bytes: every int8 factor once, the activations, the outputs
  const double fb = double(rg + ru) * d + double(d_ff) * (rg + ru) + double(d_ff) * rd + double(d) * rd;
  ProfScope scope("lowrank_ffn", st, 0.0, fb + 4.0 * double(n_tok) * 2 * d);
  launch_rows_gemv(st, q_rg, s_rg, int(rg), q_ru, s_ru, int(ru), int(d), x, int(n_tok), w.latg, w.latu, 0);
  LRC_LAUNCHED();
  if (ng == 1)
    swiglu_down_kernel<1><<<unsigned(nb), FE, lds_used, st>>>(q_lg, s_lg, q_lu, s_lu, int(rg), int(ru), w.latg, w.latu,
                                                              q_rdt, int(rd), int(d_ff), int(J), int(n_tok), w.pd);
  else
    swiglu_down_kernel<TG><<<unsigned(nb), FE, lds_used, st>>>(q_lg, s_lg, q_lu, s_lu, int(rg), int(ru), w.latg,
                                                               w.latu, q_rdt, int(rd), int(d_ff), int(J), int(n_tok),
                                                               w.pd);
  LRC_LAUNCHED();
  latent_reduce_kernel<<<unsigned(cdiv(n_tok * rd, RO)), FT, 0, st>>>(w.pd, int(nb), int(n_tok), int(rd), s_rd,
                                                                          w.latd);
  LRC_LAUNCHED();
  launch_rows_gemv(st, q_ld, s_ld, int(d), nullptr, nullptr, 0, int(rd), w.latd, int(n_tok), y, nullptr, 0);
  LRC_LAUNCHED();
  return LRC_OK;
}

// Hybrid FFN (LASER 3, item Hybrid architecture): hidden channels [0, n_lr) take the
// low-rank branch (the kernels above), channels [n_lr, n_lr + n_dense) stay dense (int8
// rows with per-row scales): their gate and up pre-activations are one row GEMV each, the
// SwiGLU runs in place, and W_down's dense columns (passed as d rows of n_dense int8) add
// their share to y.
namespace {
struct HybWs {
  FfnWs lr;
  float *gd, *ud;
};
HybWs carve_hyb(Carve& cv, int64_t n_tok, int64_t n_lr, int64_t rg, int64_t ru, int64_t rd, int64_t n_dense) {
  HybWs w{};
  if (n_lr > 0) w.lr = carve_ffn(cv, n_tok, rg, ru, rd, cdiv(n_lr, ffn_chunk(n_lr)));
  if (n_dense > 0) {
    w.gd = cv.take<float>(size_t(n_tok * n_dense));
    w.ud = cv.take<float>(size_t(n_tok * n_dense));
  }
  return w;
}
}  // namespace

extern "C" size_t lrc_hybrid_ffn_workspace(int64_t n_tok, int64_t n_lr, int64_t rg, int64_t ru, int64_t rd,
                                           int64_t n_dense) {
  if (n_tok <= 0 || n_lr < 0 || n_dense < 0 || n_lr + n_dense <= 0) return 0;
  if (n_lr > 0 && (rg <= 0 || ru <= 0 || rd <= 0)) return 0;
  Carve cv(nullptr);
  carve_hyb(cv, n_tok, n_lr, rg, ru, rd, n_dense);
  return cv.bytes();
}

extern "C" lrc_status lrc_hybrid_ffn(const float* x, int64_t n_tok, int64_t d, int64_t n_lr, const int8_t* q_rg,
                                     const float* s_rg, const int8_t* q_lg, const float* s_lg, int64_t rg,
                                     const int8_t* q_ru, const float* s_ru, const int8_t* q_lu, const float* s_lu,
                                     int64_t ru, const int8_t* q_rdt, const float* s_rd, const int8_t* q_ld,
                                     const float* s_ld, int64_t rd, int64_t n_dense, const int8_t* q_gd,
                                     const float* s_gd, const int8_t* q_ud, const float* s_ud, const int8_t* q_dd,
                                     const float* s_dd, float* y, void* ws, size_t ws_bytes, void* stream) {
  if (x == nullptr || y == nullptr || n_tok <= 0 || d <= 0 || n_lr < 0 || n_dense < 0 || n_lr + n_dense <= 0)
    return LRC_EINVAL;
  if (d % 16 || n_dense % 16 || reinterpret_cast<uintptr_t>(x) % 16 != 0) return LRC_EINVAL;
  if (n_dense > 0) {
    const void* ptrs[] = {q_gd, s_gd, q_ud, s_ud, q_dd, s_dd};
    for (const void* p : ptrs)
      if (p == nullptr) return LRC_EINVAL;
    for (const void* p : {(const void*)q_gd, (const void*)q_ud, (const void*)q_dd})
      if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return LRC_EINVAL;
    if (n_tok > (int64_t(1) << 20) || n_dense > (int64_t(1) << 24) || d > (int64_t(1) << 24) ||
        n_tok * n_dense > (int64_t(1) << 31))
      return LRC_EINVAL;
  }
  const size_t need = lrc_hybrid_ffn_workspace(n_tok, n_lr, rg, ru, rd, n_dense);
  if (n_lr > 0 && need == 0) return LRC_EINVAL;
  if (ws == nullptr || ws_bytes < need) return LRC_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Carve cv(ws);
  const HybWs w = carve_hyb(cv, n_tok, n_lr, rg, ru, rd, n_dense);
  if (n_lr > 0) {
    // the low-rank channels write y; the dense ones add to it
    const lrc_status s2 = lrc_lowrank_ffn(x, n_tok, d, n_lr, q_rg, s_rg, q_lg, s_lg, rg, q_ru, s_ru, q_lu, s_lu, ru,
                                          q_rdt, s_rd, q_ld, s_ld, rd, y, static_cast<void*>(w.lr.latg),
                                          lrc_lowrank_ffn_workspace(n_tok, n_lr, rg, ru, rd), stream);
    if (s2 != LRC_OK) return s2;
  }
  if (n_dense > 0) {
    ProfScope scope("hybrid_ffn_dense", st, 0.0, 3.0 * double(n_dense) * double(d) + 4.0 * double(n_tok) * 2 * d);
    launch_rows_gemv(st, q_gd, s_gd, int(n_dense), q_ud, s_ud, int(n_dense), int(d), x, int(n_tok), w.gd, w.ud, 0);
    LRC_LAUNCHED();
    swiglu_dense_kernel<<<unsigned(cdiv(n_tok * n_dense, FT)), FT, 0, st>>>(w.gd, w.ud, n_tok * n_dense);
    LRC_LAUNCHED();
    launch_rows_gemv(st, q_dd, s_dd, int(d), nullptr, nullptr, 0, int(n_dense), w.gd, int(n_tok), y, nullptr,
                     n_lr > 0 ? 1 : 0);
    LRC_LAUNCHED();
  }
  return LRC_OK;
}
