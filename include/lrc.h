/*
 * lrc.h -- C ABI of liblrc: whitened truncated decomposition of linear-layer weights
 * and global rank allocation, on AMD Instinct MI355X (gfx950).
 *
 * The method (pages: gist.science explainers of three papers):
 *   LASER: Loss-Aware Singular-value Decomposition and Rank Allocation for Efficient
 *     Low-Precision Vision-Language Models -- technical summary, Methodology 1
 *     (K-FAC surrogate, Transformation, QAW) and Methodology 2 (empirical-Fisher
 *     importance score, global optimisation);
 *   Swift-SVD: Theoretical Optimality Meets Practical Efficiency in Low-Rank LLM
 *     Compression -- technical summary, section 2A (closed-form optimum from one
 *     eigendecomposition of the incrementally aggregated output covariance);
 *   UniRank: Unified Rank Allocation for Low-Rank LLM Compression -- technical summary,
 *     section 2.1 (Sorting-and-Truncation: pooled sort, m+n parameters per component,
 *     accumulate until the budget is reached).
 *
 * Conventions shared by every entry point
 *   - Matrices are row-major with an explicit leading dimension (elements).
 *   - A weight W is d_out x d_in (y = W x).  Calibration activations A are
 *     n_tokens x d_in and output gradients B are n_tokens x d_out, token-major.
 *   - Every pointer except the host scalars is DEVICE memory owned by the caller.  The
 *     library allocates nothing and keeps no state between calls; scratch space comes
 *     from the caller's workspace `ws` of at least the size the matching *_workspace
 *     query returns (256-byte aligned, contents need not be initialised).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Kernels are enqueued on
 *     it and no entry point waits for them: every call returns as soon as its work is
 *     enqueued (only lrc_profile_stop, a measurement call, waits for its events).
 *   - Return value: LRC_OK, or an error found before or while enqueueing work.
 *     Argument errors are detected on the host before any HIP call is made.
 *   - Failures found by the kernels themselves (a covariance that is not positive
 *     definite, an eigensolver that hit its sweep cap, a NaN or Inf in the data) are
 *     written to a device `info` argument; the caller reads it after its own
 *     synchronisation.  The outputs of a call whose info reports a failure are undefined
 *     unless the entry point says otherwise.
 */
#ifndef LRC_H
#define LRC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LRC_OK = 0,
  LRC_EINVAL = 1,       /* null pointer, negative or inconsistent size, bad leading dim */
  LRC_EDTYPE = 2,       /* dtype or flag combination not supported */
  LRC_EWORKSPACE = 3,   /* workspace missing or smaller than the query says */
  LRC_EHIP = 4,         /* a HIP runtime call or launch failed (lrc_last_hip_error) */
  LRC_ENOTPD = 5,       /* a covariance is not positive definite (Cholesky pivot <= 0) */
  LRC_ENOCONV = 6,      /* the eigensolver did not converge within its sweep cap */
  LRC_ENONFINITE = 7    /* a NaN or Inf was met */
} lrc_status;

typedef enum { LRC_F32 = 0, LRC_BF16 = 1 } lrc_dtype;

/* lrc_accumulate_cov flags */
#define LRC_COV_QUANT_INT8_TOKEN 0x1u  /* fake-quantise each token to int8 first (QAW) */

/* lrc_score_components flags (exactly one) */
#define LRC_SCORE_FISHER 0x1u          /* empirical-Fisher score, needs A and B */
#define LRC_SCORE_KFAC 0x2u            /* 1/2 sigma^2, needs sigma only */

/* lrc_rank_scores modes (exactly one) */
#define LRC_RANKSCORE_UNIRANK 0x1u     /* I_l sigma^2 / ||Sigma_l||_F^2 per component */
#define LRC_RANKSCORE_SWIFT 0x2u       /* beta_l^alpha log(e + eps*_k)^(1-alpha) per rank k */

/*
 * lrc_accumulate_cov -- covariance streaming.
 * LASER Methodology 1 (K-FAC surrogate): X and G are the activation and gradient
 * covariances estimated on a calibration set; Swift-SVD 2A aggregates such a
 * covariance incrementally, one batch of tokens at a time.
 *
 *   C[i][j] += sum_t a_t[i] * a_t[j]   for 0 <= j <= i < d   (lower triangle incl. diag)
 *
 * A: n_tokens x d, leading dim lda >= d, dtype `dt` (LRC_BF16 or LRC_F32).
 * C: d x d fp32, leading dim ldc >= d; only the lower triangle is read and written
 *    (the strict upper triangle is left untouched).  C holds a RAW sum: the caller
 *    keeps the token count N and passes it to lrc_whiten_decompose, so a stream of
 *    chunks is accumulated by calling this once per chunk.
 * flags: 0 or LRC_COV_QUANT_INT8_TOKEN.  With the flag each token a_t is replaced by
 *    its per-token symmetric int8 fake quantisation (LASER Methodology 1, QAW):
 *    s_t = fl32(max_j |a_tj| / 127), q = clamp(round_half_even(fl32(a_tj / s_t)), -127,
 *    127), a_hat = q * s_t (an all-zero token stays zero).  On the GPU the products are
 *    formed as q_i * (s_t^2 q_j) with s_t^2 q_j split into two bf16 terms (error ~2^-17).
 * Accumulation is fp32 with bf16 x bf16 products exact; the split of the token range
 * over workgroups and its reduction order are fixed, so equal inputs give equal bits.
 * info: device int32, or NULL for no check.  Set to LRC_ENONFINITE when a diagonal entry
 *    of C comes out NaN or Inf after this call (a diagonal entry is a sum of squares, so
 *    that happens exactly when a token entry of its column is NaN/Inf, when the sum
 *    overflows, or when C held a non-finite diagonal already); never cleared, so a stream
 *    of chunks can share one flag initialised to 0 by the caller.
 * n_tokens == 0 is a no-op (A may be NULL).
 */
lrc_status lrc_accumulate_cov(const void* A, lrc_dtype dt, int64_t n_tokens, int64_t d,
                              int64_t lda, float* C, int64_t ldc, uint32_t flags,
                              int32_t* info, void* ws, size_t ws_bytes, void* stream);
size_t lrc_accumulate_cov_workspace(lrc_dtype dt, int64_t n_tokens, int64_t d, uint32_t flags);

/*
 * lrc_whiten_decompose -- whitened truncated decomposition of one weight or a batch of
 * weight slices sharing the same covariances.
 * LASER Methodology 1 (Transformation): W is moved into the curvature-weighted space
 * with the Cholesky factors of X and G, decomposed there, truncated, and the low-rank
 * factors are mapped back; Swift-SVD 2A: the decomposition is one symmetric
 * eigendecomposition of the aggregated covariance of the whitened outputs.
 *
 * With X = Xsum/n_x + damping*I = L_x L_x^T and G = Gsum/n_g + damping*I = L_g L_g^T
 * (lower Cholesky; an absent sum means identity), the whitened weight is
 *      W~ = L_g^T W L_x  = U~ S~ V~^T  (S~ descending, k = min(d_out, d_in))
 * and the outputs are
 *      sigma = diag(S~)                       (all k values)
 *      Left  = L_g^-T U~_r S~_r^{1/2}         (d_out x r)
 *      Right = S~_r^{1/2} V~_r^T L_x^-1       (r x d_in),   Left @ Right = W_r
 * W_r minimises the K-FAC loss 1/2 tr((W - W_r) X (W - W_r)^T G) over rank r.
 * The eigendecomposed Gram is the one of the smaller side (W~ W~^T if d_out <= d_in,
 * else W~^T W~), formed and solved in fp64 from the fp32 whitened weight; each pair is
 * signed so that the largest-magnitude entry of that side's singular vector is positive.
 *
 * W: batch slices, slice b at W + b*stride_w, each d_out x d_in fp32 with leading dim
 *    ldw >= d_in.  Xsum: d_in x d_in fp32 (lower triangle read), leading dim ldx, or
 *    NULL.  Gsum: d_out x d_out (lower read), leading dim ldg, or NULL.  n_x, n_g > 0
 *    when the matching sum is given.  rank: 0 <= r <= k.  damping >= 0.
 * Outputs (packed, fp32): sigma[batch][k], left[batch][d_out][r], right[batch][r][d_in].
 * info (device int32[batch], written by the call): 0 ok; p in 1..d_in: pivot p of X not
 *    positive (LRC_ENOTPD condition; every slice reports it); d_in + p: pivot p of G not
 *    positive; -1: the Jacobi solver still rotated after its last sweep (LRC_ENOCONV
 *    condition).  Solver: the tridiagonal one (Householder reduction, bisection, inverse
 *    iteration) for a single slice and for batches with k >= 384 (the slices' reductions
 *    run together, one launch per step for the whole batch); the
 *    batched block-Jacobi one for batches of smaller slices; the environment variable
 *    LRC_EIGENSOLVER=jacobi or =tridiag forces one.  The outputs of a slice with nonzero info are
 *    undefined.  These conditions are found on the device: the call itself returns LRC_OK
 *    once everything is enqueued (the solver's work is fixed in advance, so nothing is
 *    read back to the host).
 */
lrc_status lrc_whiten_decompose(const float* W, int64_t d_out, int64_t d_in, int64_t ldw,
                                int64_t batch, int64_t stride_w,
                                const float* Xsum, int64_t ldx, int64_t n_x,
                                const float* Gsum, int64_t ldg, int64_t n_g,
                                int64_t rank, float damping,
                                float* sigma, float* left, float* right, int32_t* info,
                                void* ws, size_t ws_bytes, void* stream);
size_t lrc_whiten_decompose_workspace(int64_t d_out, int64_t d_in, int64_t batch, int64_t rank,
                                      int has_x, int has_g);

/*
 * lrc_whiten_decompose_strided -- lrc_whiten_decompose for a batch of slices that may
 * each have their own covariances (independent layers, each calibrated on its own
 * activations and gradients; LASER Methodology 1 applied layer by layer, as the global
 * allocation of Methodology 2 then pools them).  Slice b is whitened with
 * Xsum + b*stride_x and Gsum + b*stride_g; a stride of 0 shares one sum over the batch
 * (stride_x = stride_g = 0 is exactly lrc_whiten_decompose).  A per-slice sum needs
 * stride_x >= d_in*ldx (stride_g >= d_out*ldg); n_x and n_g are common to the slices.
 * Outputs, info codes and asynchrony as lrc_whiten_decompose; a covariance that is not
 * positive definite is reported in the info of the slices it belongs to.  Every slice
 * gives the same bits as a call of its own.  Workspace: x_slices / g_slices are 0 (no
 * such sum), 1 (shared) or batch (one per slice); 0 is returned for other values.
 */
lrc_status lrc_whiten_decompose_strided(const float* W, int64_t d_out, int64_t d_in, int64_t ldw,
                                        int64_t batch, int64_t stride_w,
                                        const float* Xsum, int64_t ldx, int64_t stride_x, int64_t n_x,
                                        const float* Gsum, int64_t ldg, int64_t stride_g, int64_t n_g,
                                        int64_t rank, float damping,
                                        float* sigma, float* left, float* right, int32_t* info,
                                        void* ws, size_t ws_bytes, void* stream);
size_t lrc_whiten_decompose_strided_workspace(int64_t d_out, int64_t d_in, int64_t batch, int64_t rank,
                                              int64_t x_slices, int64_t g_slices);

/*
 * lrc_score_components -- importance score of every singular component.
 * LASER Methodology 2 (empirical-Fisher importance score): a component's contribution
 * to the empirical-Fisher quadratic loss, combining its size with its alignment to the
 * calibration gradients in the original parameter space.  With per-token gradient
 * samples b_t a_t^T and the component left_i right_i^T:
 *   FISHER: scores[i] = 1/(2 n_total) * sum_t (b_t . left_i)^2 (a_t . right_i)^2
 *   KFAC:   scores[i] = 1/2 sigma_i^2   (its K-FAC loss alone; no data needed)
 * A: n_tokens x d_in (lda = d_in), B: n_tokens x d_out (ldb = d_out), dtype `dt`.
 * left: d_out x k (leading dim k), right: k x d_in (leading dim d_in), fp32, as written
 * by lrc_whiten_decompose with rank k.  sigma: k floats (KFAC only).
 * FISHER streams the tokens in chunks: the first call of a stream passes accumulate=0
 * (scores are overwritten by this chunk's sum), later calls accumulate=1; the call with
 * finalize=1 scales the running sum by 1/(2*n_total).  KFAC ignores A, B, accumulate.
 * The per-token products are formed on fp32 values; the reduction order is fixed.
 * info: device int32, or NULL for no check.  Set to LRC_ENONFINITE when a score written
 *    by this call is NaN or Inf (each is a sum of non-negative terms, so a NaN/Inf in A,
 *    B or the factors, or an overflow, shows up there); never cleared by the library.
 */
lrc_status lrc_score_components(const void* A, const void* B, lrc_dtype dt, int64_t n_tokens,
                                int64_t d_in, int64_t d_out, const float* left,
                                const float* right, const float* sigma, int64_t k,
                                uint32_t flags, int accumulate, int finalize, int64_t n_total,
                                float* scores, int32_t* info, void* ws, size_t ws_bytes,
                                void* stream);
size_t lrc_score_components_workspace(int64_t n_tokens, int64_t d_in, int64_t d_out, int64_t k,
                                      uint32_t flags);

/*
 * lrc_allocate_ranks -- global sort-and-truncate under a parameter budget.
 * LASER Methodology 2 (global optimisation: greedy by importance per parameter cost
 * until the target parameter budget is reached) and UniRank 2.1 (pool all components,
 * sort descending, accumulate while the total stays within the budget; a component of
 * an m x n matrix costs m + n parameters).
 *
 * scores: M = offsets[n_mat] fp32 values, matrix m owning scores[offsets[m] ..
 *   offsets[m+1]) in component order.  offsets: int64[n_mat + 1] (device, offsets[0]=0,
 *   non-decreasing).  cost: int64[n_mat] (device, > 0; normally d_out + d_in).
 * key_j = fp64(score_j) / fp64(cost of j's matrix), IEEE round-to-nearest.  Items are
 * sorted by key descending, equal keys keeping the input order (matrix id, then
 * component index).  The kept set is the longest prefix of that order whose int64
 * cumulative cost is <= budget.
 * Outputs (device): order[M] (int32 item ids in sorted order), n_kept (one int64),
 *   ranks[n_mat] (int32 kept count per matrix), kept_mask[M] (uint8 0/1),
 *   info (one int32: 0 ok, LRC_ENONFINITE if a score is NaN/Inf or negative,
 *   LRC_EINVAL if a cost is <= 0 or offsets are inconsistent).  A call with nonzero info
 *   keeps nothing: n_kept = 0, kept_mask and ranks all zero (order is still a
 *   permutation, with no meaning).
 * order may be NULL (here and in lrc_allocate_ranks_noalloc): the library then finds the
 *   first excluded item by a radix select weighted by cost instead of sorting the pool,
 *   and writes the same n_kept, ranks, kept_mask and info bit for bit, with the same
 *   workspace.  The kept set depends only on that item, so no order is needed for it.
 * Identical inputs give identical outputs bit for bit.  M must be < 2^31.
 */
lrc_status lrc_allocate_ranks(const float* scores, const int64_t* offsets, const int64_t* cost,
                              int64_t n_mat, int64_t n_items, int64_t budget, int32_t* order,
                              int64_t* n_kept, int32_t* ranks, uint8_t* kept_mask, int32_t* info,
                              void* ws, size_t ws_bytes, void* stream);
size_t lrc_allocate_ranks_workspace(int64_t n_mat, int64_t n_items);

/*
 * lrc_allocate_ranks_noalloc -- lrc_allocate_ranks for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, outputs and kernels, minus the workspace.  Its scratch
 * is a device array inside the library (about 52 MB, one per GPU the library runs on,
 * held until the process ends), so no memory is allocated by the call.
 * n_items may be at most lrc_allocate_ranks_noalloc_max_items() (2^21 = 2,097,152);
 * larger pools get LRC_EWORKSPACE (use lrc_allocate_ranks).  Every call on one GPU uses
 * that GPU's single array: calls that overlap on one GPU (two streams, two host threads)
 * race and must be serialised by the caller.  The array needs no initialisation; it
 * keeps the last call's contents.
 */
lrc_status lrc_allocate_ranks_noalloc(const float* scores, const int64_t* offsets, const int64_t* cost,
                                      int64_t n_mat, int64_t n_items, int64_t budget, int32_t* order,
                                      int64_t* n_kept, int32_t* ranks, uint8_t* kept_mask, int32_t* info,
                                      void* stream);
int64_t lrc_allocate_ranks_noalloc_max_items(void);

/*
 * lrc_rank_scores -- alternative scores over the same component layout as
 * lrc_allocate_ranks, from the singular values alone.
 *   UNIRANK (UniRank 2.1, "Aggregation and Truncation"): scores[j] = weight[m] *
 *     sigma_j^2 / sum over matrix m of sigma^2 -- the layer's global functional
 *     importance I_l (weight, >= 0, supplied by the caller) times the component's share
 *     of the singular-value energy; an all-zero spectrum scores 0.  These feed
 *     lrc_allocate_ranks directly.
 *   SWIFT (Swift-SVD section B, "Hybrid Scoring"): for the component at position p of
 *     matrix m, scores[j] = weight[m]^alpha * log(e + eps)^(1 - alpha) with eps = the sum
 *     of sigma^2 over positions > p: the layer's compressibility score if its rank were
 *     p + 1 (weight = the layer importance beta_l > 0, 0 <= alpha <= 1).  The pages choose
 *     ranks from these by a search on validation data, which is not part of the library.
 * sigma: M = offsets[n_mat] fp32 singular values, matrix m owning sigma[offsets[m] ..
 *   offsets[m+1]) in descending order (as lrc_whiten_decompose writes them).
 * offsets: int64[n_mat + 1] (device, offsets[0] = 0, non-decreasing, offsets[n_mat] =
 *   n_items).  weight: float[n_mat] (device).  scores: float[M] (device, output).
 * info (device int32): 0 ok, LRC_EINVAL for inconsistent offsets or a weight out of range,
 *   LRC_ENONFINITE for a NaN/Inf sigma or weight (the offending matrices' scores are not
 *   written).  Sums are fp64 in a fixed order; identical inputs give identical bits.
 */
lrc_status lrc_rank_scores(const float* sigma, const int64_t* offsets, int64_t n_mat, int64_t n_items,
                           const float* weight, float alpha, uint32_t mode, float* scores, int32_t* info,
                           void* stream);

/*
 * lrc_rotate_quantize -- factor codec after the back-map.
 * LASER section 3 (Hybrid SVD-Quantization for FFNs), item Quantization: an orthogonal
 * rotation between the low-rank factors smooths outliers, then both factors are quantised
 * round-to-nearest.  With R = H_r diag(signs) / sqrt(r) (H_r the Sylvester Hadamard
 * matrix; r a power of two, r <= 8192; signs: r floats, each +1 or -1, chosen by the
 * caller), left' = left R (d_out x r) and right' = R^T right (r x d_in), so their product
 * is unchanged.  The rotation runs in fp64 and is rounded once to fp32; each row of left'
 * and of right' is then quantised with its own scale:
 *   scale = fl32(max|row| / 127), q = clamp(round_half_even(fl32(x / scale)), -127, 127)
 *   (an all-zero row gives codes 0 and scale 0).
 * left: d_out x r (leading dim r), right: r x d_in (leading dim d_in), fp32 (as written by
 *   lrc_whiten_decompose).  Outputs (device): q_left int8 d_out x r, s_left float[d_out],
 *   q_right int8 r x d_in, s_right float[r]; left_rot / right_rot (fp32, same shapes) may be
 *   NULL or receive the rotated factors.
 */
lrc_status lrc_rotate_quantize(const float* left, const float* right, int64_t d_out, int64_t r, int64_t d_in,
                               const float* signs, int8_t* q_left, float* s_left, int8_t* q_right,
                               float* s_right, float* left_rot, float* right_rot, void* ws, size_t ws_bytes,
                               void* stream);
size_t lrc_rotate_quantize_workspace(int64_t d_out, int64_t r, int64_t d_in);

/*
 * lrc_quantize_rows -- the same per-row int8 RTN for a dense branch (LASER section 3: the
 * channels kept dense are quantised as well).  X: rows x cols fp32 (leading dim ldx);
 * q: int8 rows x cols (leading dim cols); scale: float[rows].
 */
lrc_status lrc_quantize_rows(const float* X, int64_t rows, int64_t cols, int64_t ldx, int8_t* q, float* scale,
                             void* stream);

/*
 * lrc_ffn_select_channels -- which hidden channels of an FFN take the low-rank branch.
 * LASER section 3 (Hybrid SVD-Quantization for FFNs), items Channel selection and Hybrid
 * architecture: a temporary SVD of the gate and up projections finds the hidden channels
 * the low-rank form reconstructs well ("SVD-friendly"); those are compressed, the rest stay
 * dense.  A channel's error is the expected squared error of its two pre-activations under
 * the calibration distribution:
 *   err[h] = sum over P in {gate, up} of dW_P[h] X dW_P[h]^T,  dW_P = W_P - left_P right_P,
 * X = Xsum/n_x + damping*I, evaluated as the squared row norm of dW_P L_x (X = L_x L_x^T,
 * fp32 products, fp64 row sums in a fixed order).
 * w_gate, w_up: d_ff x d fp32, leading dim ldw >= d.  left_*: d_ff x r (leading dim r),
 *   right_*: r x d (leading dim d): the factors lrc_whiten_decompose wrote for gate and up
 *   with this Xsum, no Gsum and rank r (0 <= r <= min(d_ff, d); r = 0 needs no factors).
 * Xsum: d x d fp32 (lower triangle read), leading dim ldx >= d; n_x > 0; damping >= 0.
 * Outputs (device): err double[d_ff]; order int32[d_ff]: the channels by ascending err,
 *   ties by channel index; lowrank uint8[d_ff]: 1 for the first n_lowrank channels of
 *   `order` (0 <= n_lowrank <= d_ff), else 0.
 * info (device int32[1], written by the call): 0, or p when pivot p of X is not positive
 *   (the LRC_ENOTPD condition; order and lowrank are then not written and err holds no
 *   meaningful values).  Found on the device: the call returns LRC_OK once enqueued.
 */
lrc_status lrc_ffn_select_channels(const float* w_gate, const float* w_up, int64_t d_ff, int64_t d, int64_t ldw,
                                   const float* left_gate, const float* right_gate, const float* left_up,
                                   const float* right_up, int64_t r, const float* Xsum, int64_t ldx, int64_t n_x,
                                   float damping, int64_t n_lowrank, double* err, int32_t* order, uint8_t* lowrank,
                                   int32_t* info, void* ws, size_t ws_bytes, void* stream);
size_t lrc_ffn_select_channels_workspace(int64_t d_ff, int64_t d);

/*
 * lrc_lowrank_ffn -- decode-time forward of a SwiGLU FFN whose weights are replaced by
 * int8 low-rank factors.
 * LASER section 4 (System Implementation): the low-rank FFN runs as fused kernels for the
 * input projection, the latent activations, SwiGLU and the dequantisation.  Computes
 *   y = W_down (SiLU(W_gate x) * (W_up x)),  W = (q_L * s_L[:,None]) (q_R * s_R[:,None])
 * for gate, up and down (one fp32 scale per factor row, as lrc_rotate_quantize writes).
 * x: n_tok x d fp32 (16-byte aligned); y: n_tok x d fp32.
 * gate: q_rg (rg x d int8), s_rg[rg], q_lg (d_ff x rg int8), s_lg[d_ff]; up likewise with ru.
 * down: q_rdt = R_down^T (d_ff x rd int8: row j holds hidden channel j's latent weights),
 *   s_rd[rd] (R_down's row scales), q_ld (d x rd int8), s_ld[d].
 * d, rg, ru, rd multiples of 16; the int8 matrices 16-byte aligned (q_rdt 8-byte);
 * the larger latent of a token group must fit in LDS: 4 * (17/16) * max(rg, ru) + 8 * ceil(d_ff / 512)
 * floats within 160 KiB (max(rg, ru) up to about 9500).
 * Activations and sums are fp32; the reduction order is fixed.
 */
lrc_status lrc_lowrank_ffn(const float* x, int64_t n_tok, int64_t d, int64_t d_ff, const int8_t* q_rg,
                           const float* s_rg, const int8_t* q_lg, const float* s_lg, int64_t rg, const int8_t* q_ru,
                           const float* s_ru, const int8_t* q_lu, const float* s_lu, int64_t ru, const int8_t* q_rdt,
                           const float* s_rd, const int8_t* q_ld, const float* s_ld, int64_t rd, float* y, void* ws,
                           size_t ws_bytes, void* stream);
size_t lrc_lowrank_ffn_workspace(int64_t n_tok, int64_t d_ff, int64_t rg, int64_t ru, int64_t rd);

/*
 * lrc_hybrid_ffn -- the same forward for an FFN in LASER's hybrid form (section 3, item
 * Hybrid architecture: the selected hidden channels compressed, the others dense).  The
 * hidden channels are ordered so that [0, n_lr) take the low-rank branch and the next
 * n_dense stay dense (the order lrc_ffn_select_channels returns, applied by the caller to
 * the rows of W_gate, W_up and the columns of W_down; a permutation of the hidden channels
 * leaves the FFN unchanged):
 *   y = sum over low-rank channels (as lrc_lowrank_ffn, with d_ff = n_lr)
 *     + Wd_dense (SiLU(Wg_dense x) * (Wu_dense x)),
 * every dense matrix int8 with one fp32 scale per row: q_gd, q_ud: n_dense x d (scales
 * s_gd, s_ud [n_dense]); q_dd: d x n_dense, W_down's dense columns as rows (scales s_dd[d]).
 * n_lr = 0 (no factors needed) or n_dense = 0 (no dense matrices needed) are allowed,
 * not both.  d and n_dense multiples of 16; x and the dense int8 matrices 16-byte aligned;
 * the low-rank arguments as lrc_lowrank_ffn requires.  Sums fp32, order fixed.
 */
lrc_status lrc_hybrid_ffn(const float* x, int64_t n_tok, int64_t d, int64_t n_lr, const int8_t* q_rg,
                          const float* s_rg, const int8_t* q_lg, const float* s_lg, int64_t rg, const int8_t* q_ru,
                          const float* s_ru, const int8_t* q_lu, const float* s_lu, int64_t ru, const int8_t* q_rdt,
                          const float* s_rd, const int8_t* q_ld, const float* s_ld, int64_t rd, int64_t n_dense,
                          const int8_t* q_gd, const float* s_gd, const int8_t* q_ud, const float* s_ud,
                          const int8_t* q_dd, const float* s_dd, float* y, void* ws, size_t ws_bytes, void* stream);
size_t lrc_hybrid_ffn_workspace(int64_t n_tok, int64_t n_lr, int64_t rg, int64_t ru, int64_t rd, int64_t n_dense);

/*
 * Measurement support (benchmarks and profilers; not needed for results).
 * Between lrc_profile_start and lrc_profile_stop every launch of an instrumented kernel
 * is bracketed by two HIP events recorded on the stream it runs on, and the work it
 * performed is added to its kernel's totals: algorithmic flops and HBM bytes computed
 * from the launch shape, or, for the eigensolver kernels, counted on the device (tile
 * products and rotations actually executed).  lrc_profile_stop waits for the recorded
 * events; then lrc_profile_kernels / lrc_profile_kernel return one entry per kernel
 * name (name is a static string).  Host-side state, one profiling session per process.
 */
lrc_status lrc_profile_start(void);
lrc_status lrc_profile_stop(void);
int lrc_profile_kernels(void);
lrc_status lrc_profile_kernel(int index, const char** name, int64_t* launches, double* total_ms,
                              double* flops, double* bytes);

/* Human-readable name of a status code (static string). */
const char* lrc_status_string(lrc_status s);
/* The hipError_t value of the last LRC_EHIP returned on this thread (0 if none). */
int lrc_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LRC_H */
