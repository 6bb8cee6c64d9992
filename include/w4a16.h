/*
 * w4a16.h -- weight-only int4, group-128 quantized linear layers (W4A16) on
 * AMD CDNA4 (MI355X, gfx950): quantize + pack, decode GEMV, prefill GEMM and the
 * batched fake-quant loss of an AWQ scale-exponent / clip-shrink search.
 *
 * Sources for what is computed (web pages, cited by title and section):
 *   [AWQ-W4 card]  model card "rebuttal_w4g128_awq_w2": details table rows
 *                  "Scheme" (weight-only, 4-bit, group size 128, asymmetric zero
 *                  point) and "Search" (20-point scale-exponent grid + 10-point
 *                  global shrink grid); the scale-rewrite paragraph
 *                  (prev_op /= s, W *= s  ==  Q(W diag(s)) diag(1/s)); the
 *                  "Clipping granularity" paragraph; RTN note under the perplexity table.
 *   [27B card]     model card "Qwen3.6-27B-W4A16": opening paragraph (int4, group
 *                  128, symmetric, weight-only, 16-bit activations, data-free RTN).
 *   [QSRT card]    model card "GLM-5.2-QSRT-Fruit-Instruct", "Reproducible runtime":
 *                  decode-sized batches of at most 16 rows take a separate path
 *                  from prefill; unsupported shapes fail closed.
 *   [AWQ record]   benchmark record "AWQ INT4-g128 WikiText-2 perplexity delta vs
 *                  fp16, Llama-2 7B", "Methodology": group 128, alpha grid of 20.
 *
 * Conventions for every entry point
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - Array pointers are DEVICE pointers owned by the caller unless a parameter
 *     says "host".  The library never frees caller memory and never allocates
 *     device memory: scratch space comes in through a caller workspace (with a
 *     size query), or, for w4a16_gemv_noalloc, from one static array per device
 *     that exists while the library is loaded.  Every kernel is the library's
 *     own; it links nothing beyond the HIP runtime.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously on it; results are ready once the stream is synchronized.
 *     awq_search and awq_search_lookahead are the calls that synchronize (they
 *     read losses on the host).
 *   - Arguments are validated on the host before any HIP call; a failing check
 *     returns a negative w4_status and enqueues nothing.  No call aborts or prints.
 *   - Weight layout: W is [N][K] row-major (output channels x input channels,
 *     input channels contiguous) -- the K x N weight of the linear, stored so that
 *     W diag(s) scales input channels.  K must be a multiple of 128.
 *   - Packed layout: qweight[n][i] (uint32, [N][K/8]) holds in nibble j (bits
 *     4j..4j+3) the code of input channel k = 8i + j.  scales[n][g] (bf16,
 *     [N][K/128]) is the scale of group g = k / 128.  qzeros[n][i] (uint32,
 *     [N][ceil(K/1024)]) holds in nibble j the zero point of group 8i + j; unused
 *     nibbles are 0.  Symmetric weights have no qzeros: the stored nibble is the
 *     signed code + 8.
 *   - Dequantized weight: W_hat[n][k] = (q - z) * scale, z = zero point
 *     (asymmetric) or 8 (symmetric).
 *   - Alignment: every array pointer must be 16-byte aligned (W4_ERR_ALIGN).
 *   - Sizes are int; products are formed in 64-bit.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W4_OK = 0,
  W4_ERR_NULL = -1,         /* a required pointer is NULL (or a forbidden one is not)   */
  W4_ERR_SHAPE = -2,        /* a size is out of range, or K is not a multiple of 128    */
  W4_ERR_ALIGN = -3,        /* an array pointer is not 16-byte aligned                   */
  W4_ERR_UNSUPPORTED = -4,  /* group_size != 128, gemv with M > 16, ...                  */
  W4_ERR_WORKSPACE = -5,    /* workspace missing or smaller than the size query returns  */
  W4_ERR_HIP = -6,          /* a HIP runtime call failed                                 */
  W4_ERR_VALUE = -7,        /* a scalar argument is out of range (clip ratio, grid size) */
  W4_ERR_SCRATCH = -8       /* the problem needs more than the library's static scratch  */
} w4_status;

#define W4_GROUP_SIZE 128
#define W4_GEMV_MAX_M 16
/* Size of the static device scratch array of w4a16_gemv_noalloc (per device). */
#define W4_GEMV_SCRATCH_BYTES (8u << 20)

/* Human-readable name of a status code (static storage; never NULL). */
const char* w4_status_string(int status);

/*
 * awq_quantize_pack -- round-to-nearest group-128 quantization of v = W diag(s),
 * with optional clipping, and nibble packing.  [AWQ-W4 card] "Scheme" and the
 * scale-rewrite paragraph (the candidate weight Q(W diag(s))); "Clipping
 * granularity" (one shrink ratio r for the whole linear); [27B card] opening
 * paragraph (symmetric form).
 *
 * Per row n and group g, in IEEE fp32 with round-half-to-even rint:
 *   v_k  = W[n][k] * s[k]                (s == NULL: v_k = W[n][k])
 *   r<1: t = r * max|v|,  v_k = min(max(v_k, -t), t)
 *   asymmetric: scale = bf16(max(max v - min v, 1e-5) / 15)
 *               z = clamp(rint(-min v / scale), 0, 15)
 *               q_k = clamp(rint(v_k / scale) + z, 0, 15)
 *   symmetric : scale = bf16(max(max|v|, 1e-5) / 7)
 *               q_k = clamp(rint(v_k / scale), -8, 7) + 8
 * bf16() rounds to nearest even; "/" is IEEE division by the stored bf16 scale.
 *
 *   W          [N][K] bf16, device.           s        [K] fp32 or NULL.
 *   clip_ratio in (0, 1]; 1 = no clipping.      symmetric 0 or 1.   group_size == 128.
 *   qweight    [N][K/8] out.   scales [N][K/128] out.
 *   qzeros     [N][ceil(K/1024)] out; must be NULL iff symmetric.
 * Results are bit-identical to the definition above for every finite input.
 */
int awq_quantize_pack(const uint16_t* W, int N, int K, const float* s, float clip_ratio,
                      int symmetric, int group_size, uint32_t* qweight, uint16_t* scales,
                      uint32_t* qzeros, void* stream);

/*
 * w4a16_gemv -- decode contraction Y = X W_hat^T for 1 <= M <= 16 rows, bf16
 * activations, int4 weights unpacked in registers.  The smallest batches take
 * one wavefront dot-product reduction per output; larger ones (from M = 5, or
 * earlier on wide or large weights, by a fixed rule of the shape) take 16x16x32
 * bf16 matrix-core products over all rows at once.  [QSRT card] "Reproducible
 * runtime": decode batches of at most 16 rows take their own path; [27B card]
 * activations stay 16-bit.
 *
 *   X [M][K] bf16.  qweight/scales/qzeros as produced by awq_quantize_pack
 *   (qzeros NULL iff symmetric).  Y [M][N] bf16 out: fp32 accumulation, each
 *   128-group summed with exact integer weights (q - z) and scaled once, rounded
 *   to nearest even at the store.
 *   M > 16 returns W4_ERR_UNSUPPORTED (no silent fallback: use w4a16_gemm).
 *   W4_ERR_SHAPE (from the size query too) when N K / 2 >= 2^31 or 32 K >= 2^31:
 *   the kernels address the packed weights and the activation rows with 32-bit
 *   byte offsets.
 *   workspace / workspace_bytes: fp32 K-split partial sums for long K (the
 *   wavefront form above K = 32768 at M <= 2 and K = 16384 at M = 3, 4; the
 *   matrix-core form above K = 6144); size 0 for shorter K.
 *   Size query: workspace == NULL with workspace_bytes != NULL writes the size
 *   needed and returns W4_OK without enqueuing work.  To run a shape whose size
 *   is 0, pass workspace == NULL and workspace_bytes == NULL.
 */
int w4a16_gemv(const uint16_t* X, int M, int K, int N, const uint32_t* qweight,
               const uint16_t* scales, const uint32_t* qzeros, int symmetric, int group_size,
               uint16_t* Y, void* workspace, size_t* workspace_bytes, void* stream);

/*
 * w4a16_gemv_noalloc -- w4a16_gemv for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments minus the workspace, same kernels, bit-identical
 * results.  The fp32 partial sums of a K split (the workspace of w4a16_gemv) live
 * in a static device array of W4_GEMV_SCRATCH_BYTES (8 MiB), one per device, held
 * until the process ends; its device address is fetched once per device, on the
 * first call there.  Nothing is allocated or freed.
 *   Problems whose split partials exceed the array (w4a16_gemv's size query above
 *   8 MiB, e.g. M = 16 at K = 17408 with N > 43,690) return W4_ERR_SCRATCH and
 *   enqueue nothing; every other argument is checked as in w4a16_gemv.
 *   All calls on one device share its array: calls whose executions overlap on
 *   one device (concurrent streams, or host threads on different streams) race
 *   and must be serialized by the caller.  Calls on one stream never overlap.
 */
int w4a16_gemv_noalloc(const uint16_t* X, int M, int K, int N, const uint32_t* qweight,
                       const uint16_t* scales, const uint32_t* qzeros, int symmetric, int group_size,
                       uint16_t* Y, void* stream);

/*
 * w4a8_quantize_activations -- per-row symmetric int8 quantization of decode
 * activations for w4a8_gemv.  [QSRT card] "What is included" and "Size and
 * memory": a W4A8 decode path over the same stored int4 weights; the pages do
 * not define the 8-bit activation format, the reading used here is per row:
 *   sx[m] = max_k |X[m][k]| / 127 (fp32 IEEE division; 1 for an all-zero row),
 *   Xq[m][k] = clamp(rint(X[m][k] / sx[m]), -127, 127) (IEEE division, ties to even),
 *   xsum[m][g] = sum of Xq[m][k] over group g (exact int32).
 *   X [M][K] bf16 in, 1 <= M <= 16 (M > 16: W4_ERR_UNSUPPORTED; M = 0: no-op).
 *   Xq [M][K] int8, sx [M] fp32, xsum [M][K/128] int32 out (device).
 */
int w4a8_quantize_activations(const uint16_t* X, int M, int K, int8_t* Xq, float* sx, int32_t* xsum,
                              void* stream);

/*
 * w4a8_gemv -- W4A8 decode contraction for 1 <= M <= 16 rows on int8 matrix
 * cores.  [QSRT card] "Reproducible runtime": decode batches of at most 16 rows
 * take the W4A8 path, W4A16 serves everything above.
 *   Y[m][n] = bf16( sx[m] * sum_g scales[n][g] * (sum_{k in g} Xq[m][k] q[n][k]
 *                                                 - z[n][g] xsum[m][g]) )
 *   with q the stored nibble, z the zero point (8 when symmetric); the group
 *   sums are exact int32, the scaling fp32.  Xq, sx, xsum as written by
 *   w4a8_quantize_activations; qweight/scales/qzeros as for w4a16_gemv.
 *   M > 16: W4_ERR_UNSUPPORTED; K above 51,200 channels (400 groups, 25 per
 *   wave of a 16-wave workgroup): W4_ERR_UNSUPPORTED.
 *   workspace / workspace_bytes: as for w4a16_gemv.  When K has at least 64
 *   groups and N is below 8,192 (fewer than two 16-column tiles per CU of
 *   256), the groups are split among several workgroups per tile (ranges of at
 *   least 16 groups, as many as bring the workgroups near two per CU) and the
 *   workspace holds their fp32 partial sums
 *   (splits x M x N x 4 bytes, added in split order by a second kernel before
 *   the sx[m] scaling); otherwise the size is 0 and both may be NULL.  The size
 *   depends only on (M, K, N).
 *   Measured against w4a16_gemv on MI355X (graph-replayed GEMV launches, the
 *   W4A8 activations quantized beforehand as the previous op would emit them):
 *   w4a16_gemv is faster at every M measured -- on the decode-block linears by
 *   1.5x at M = 1, 1.2x at M = 4 and 8, 1.1x at M = 16, and on the 27B-shaped
 *   linears cold (W4A8 at M = 16: 26 / 30 us; W4A16 at M = 8: 14 / 17 us) -- and
 *   keeps 16-bit activations; W4A8 remains for stacks that need the int8
 *   activation path.
 */
int w4a8_gemv(const int8_t* Xq, const float* sx, const int32_t* xsum, int M, int K, int N,
              const uint32_t* qweight, const uint16_t* scales, const uint32_t* qzeros, int symmetric,
              int group_size, uint16_t* Y, void* workspace, size_t* workspace_bytes, void* stream);

/*
 * w4a16_gemm -- prefill contraction Y = X W_hat^T for any M >= 1, on MFMA bf16
 * matrix cores.  [QSRT card] "Reproducible runtime": W4A16 serves prefill row
 * counts.  Same operands and rounding as w4a16_gemv.  Two forms, chosen by shape:
 *   - M <= 16: the kernels of w4a16_gemv (its workspace and size limits); measured
 *     faster than the one-pass form below at every such M.
 *   - 17 <= M <= 48 (with N K / 2 < 2^31 and 2 M K < 2^31): one pass over the packed
 *     weights, each wave holding all M activation rows of one group in
 *     registers; no workspace when K <= 2048 (16 groups, one workgroup's waves),
 *     else the groups are split into ranges of at most 16 whose fp32 partial
 *     outputs (splits x M x N x 4 bytes) a second kernel adds in split order.
 *   - larger M: tiles of 64 x 128 outputs with LDS-staged activations; the
 *     workspace (always > 0 bytes) holds X with every 8-channel run reordered
 *     for the packed-word expansion, the negated group row sums of X (each as
 *     three exact bf16 parts) and, per group and column, the scale with
 *     bf16(128 + z); when the output tiles are too few to fill the chip, the
 *     groups are split among several workgroups per tile and the workspace also
 *     holds their fp32 partial outputs (splits x M x N x 4 bytes, added in split
 *     order by a second kernel); about 2 M K bytes plus the partials.
 *   Size query as in w4a16_gemv (when the size is 0, pass workspace == NULL and
 *   workspace_bytes == NULL).  The size depends only on (M, K, N).
 *   W4_ERR_SHAPE (from the size query too) when (M + 64) K >= 2^31 or
 *   N K >= 2^33 (32-bit byte offsets into the arranged activations and the
 *   packed weights).
 */
int w4a16_gemm(const uint16_t* X, int M, int K, int N, const uint32_t* qweight,
               const uint16_t* scales, const uint32_t* qzeros, int symmetric, int group_size,
               uint16_t* Y, void* workspace, size_t* workspace_bytes, void* stream);

/*
 * w4_bf16_linear -- the unquantized linear Y = bf16(X W^T) (fp32 accumulation,
 * rounded to nearest even), on the library's bf16 matrix-core kernel.
 * [AWQ-W4 card] scale-rewrite paragraph and the paragraph under the details
 * table: the losses of the search compare against the linear in original
 * precision (awq_grid_loss computes its Yref with this kernel; the decoder-block
 * calls run their unquantized projections on it).
 *   X [M][K] bf16, W [N][K] bf16 (K contiguous), Y [M][N] bf16 out (device).
 *   K a positive multiple of 64 (else W4_ERR_SHAPE); 2 M K and 2 N K below 2^32.
 */
int w4_bf16_linear(const uint16_t* X, int M, int K, int N, const uint16_t* W, uint16_t* Y, void* stream);

/*
 * awq_grid_loss -- losses of C fake-quant candidates of one linear.
 * [AWQ-W4 card] scale-rewrite paragraph: a candidate (s, r) is simulated by
 * swapping the weight for Q(W diag(s)) diag(1/s), i.e. by feeding X diag(1/s)
 * (rounded to bf16, the deployed prev_op /= s) to the int4 weight Q(W diag(s));
 * "Search" and "Clipping granularity": s from the scale-exponent grid, one
 * global shrink ratio r.
 *   losses[c] = mean over T x N of (Y_hat_c - Y_ref)^2, Y_hat_c in fp32 and
 *   Y_ref = bf16(X W^T).
 *
 *   X [T][K] bf16 calibration activations.  W [N][K] bf16 unquantized weight.
 *   Yref [T][N] bf16, or NULL: then bf16(X W^T) is computed into the workspace.
 *   S [C][K] fp32 (row c = s_c, every s_c[k] > 0).  ratios [C] fp32 in (0, 1].
 *   losses [C] fp32 out (device).  Workspace size query as in w4a16_gemm; it
 *   depends on (T, K, N, C) and on whether Yref is NULL.
 *   W4_ERR_SHAPE (from the size query too) when (T + 64) K >= 2^31, N K >= 2^31
 *   or C > 65535.  awq_search applies the same limits with C = max(n_alpha,
 *   n_ratio); w4a8_gemv those of w4a16_gemv.
 * The per-tile partial sums are reduced in a fixed order: results are
 * bit-identical from run to run.
 */
int awq_grid_loss(const uint16_t* X, int T, int K, int N, const uint16_t* W,
                  const uint16_t* Yref, const float* S, const float* ratios, int C,
                  int symmetric, int group_size, float* losses, void* workspace,
                  size_t* workspace_bytes, void* stream);

/*
 * awq_clip_search -- stock per-output-channel clipping: a shrink ratio per
 * (output channel, group).  [AWQ-W4 card] "Clipping granularity" and the caveat
 * under the perplexity table: the d = 0 arm searches the clipping threshold per
 * output channel, each channel scored on its own error (the look-ahead arm's one
 * global ratio is awq_grid_loss / awq_search).  For channel n, group g, ratio j:
 *   v = fp32(W[n][k] s[k]) over the 128 channels k of g;
 *   w_hat = the dequantized RTN of v clamped to +-ratios[j] * absmax(v), exactly
 *           as awq_quantize_pack with clip ratios[j];  e = v - w_hat;
 *   losses[g][n][j] = sum_t (sum_{k in g} x'[t][k] e[k])^2,
 *                     x' = bf16(X[t][k] / s[k]) (the deployed activations);
 *   best[n][g] = the first j with the least losses[g][n][j].
 * The loss is formed as e^T H_g e with the Gram matrix H_g = X'_g^T X'_g (fp32
 * accumulation of exact bf16 products) and bf16 hi + lo splits of e and H_g on
 * the matrix cores: relative error of order 2^-16 of e^T |H_g| e, so ratios whose
 * losses differ by less than that may be chosen either way.
 *
 *   X [T][K] bf16 calibration activations, T >= 0 (T = 0: every loss is 0).
 *   W [N][K] bf16 unquantized weight.  s [K] fp32 (every s[k] > 0) or NULL (= 1).
 *   ratios [R] fp32 device, 1 <= R <= 64 (else W4_ERR_VALUE); every ratio must
 *   lie in (0, 1] (a ratio of 1 means no clipping; the values are read on the
 *   device and not checked: others give unspecified losses, never a fault).
 *   losses [G][N][R] fp32 device out, or NULL (not written); G = K / 128.
 *   best [N][G] uint8 device out.
 *   workspace: size query as in w4a16_gemm (workspace == NULL and workspace_bytes
 *   != NULL); the size depends on (T, K) and is about 16 MiB + 64 KiB per group.
 * Deterministic: fixed summation orders, bit-identical from run to run.
 */
int awq_clip_search(const uint16_t* X, int T, int K, int N, const uint16_t* W, const float* s,
                    const float* ratios, int R, int symmetric, int group_size, float* losses,
                    uint8_t* best, void* workspace, size_t* workspace_bytes, void* stream);

/*
 * awq_search -- the two-phase search of [AWQ-W4 card] "Search": every alpha in
 * `alphas` scored at r = 1, keep the first minimum alpha*; then every ratio in
 * `ratios` scored at s(alpha*), keep the first minimum r*.
 *   s(alpha)_k = max(m_k^alpha, 1e-4) / sqrt(max_j p_j * min_j p_j) with
 *   m_k = mean_t |X[t][k]| (device, fp64, fixed order) and the rest in fp64 on
 *   the host, stored fp32.
 *
 *   alphas [n_alpha], ratios [n_ratio]: host fp64 (1 <= n <= 64 each).
 *   losses_out [n_alpha + n_ratio]: host fp32 out (alpha losses, then ratio losses).
 *   alpha_index, ratio_index: host int out.   s_out [K] fp32 device out: s(alpha*).
 *   workspace / workspace_bytes: as awq_grid_loss with C = max(n_alpha, n_ratio) plus
 *   the statistic; workspace == NULL and workspace_bytes != NULL -> size query.
 *   The workspace is required: W4_ERR_WORKSPACE when it is NULL (without a size
 *   query) or smaller than the query's answer.  Synchronizes `stream` (twice).
 */
int awq_search(const uint16_t* X, int T, int K, int N, const uint16_t* W,
               const double* alphas, int n_alpha, const double* ratios, int n_ratio,
               int symmetric, int group_size, float* losses_out, int* alpha_index,
               int* ratio_index, float* s_out, void* workspace, size_t* workspace_bytes,
               void* stream);

/*
 * One decoder block's weights (all bf16, device pointers, [out][in] row-major):
 * the base model's block ([AWQ-W4 card] "Base model": Qwen3-1.7B, hidden 2048;
 * [q326 page] architecture notes: grouped-query attention, head size 128,
 * rotary positions with base 10^6, SiLU-gated feed-forward).
 *   norm1 [H], wq [128 n_q][H], wk [128 n_kv][H], wv [128 n_kv][H], wo [H][128 n_q],
 *   norm2 [H], wgate [I][H], wup [I][H], wdown [H][I].
 */
typedef struct w4_block {
  const uint16_t* norm1;
  const uint16_t* wq;
  const uint16_t* wk;
  const uint16_t* wv;
  const uint16_t* wo;
  const uint16_t* norm2;
  const uint16_t* wgate;
  const uint16_t* wup;
  const uint16_t* wdown;
} w4_block;

/*
 * w4_block_forward -- Y = block(X) for B sequences of L tokens, X and Y [B L][H] bf16.
 *   a = rmsnorm(x) * norm1 (eps 1e-6); q, k, v = a Wq^T, a Wk^T, a Wv^T; rotary
 *   embedding of q and k on the pairs (j, j + 64) of each head at the token's
 *   position in its sequence; o = causal softmax(q k^T / sqrt(128)) v per sequence,
 *   query head h reading key/value head h / (n_q / n_kv); h1 = x + o Wo^T;
 *   b = rmsnorm(h1) * norm2; y = h1 + (silu(b Wg^T) * (b Wu^T)) Wd^T.  No biases,
 *   no per-head q/k norms.  Every op computes in fp32 and stores bf16 (nearest
 *   even); the projections are bf16 GEMMs with fp32 accumulation (w4_bf16_linear's
 *   kernel).
 *   H and I multiples of 128; n_kv >= 1 divides n_q; B, L >= 1.
 *   Workspace: size query as in w4a16_gemm (about 2 B L (5 H + 3 I + 2 128 n_q +
 *   2 128 n_kv) bytes).
 */
int w4_block_forward(const uint16_t* X, int B, int L, int hidden, int n_q, int n_kv, int inter,
                     const w4_block* blk, uint16_t* Y, void* workspace, size_t* workspace_bytes,
                     void* stream);

/*
 * w4_block_forward_quantized -- w4_block_forward with linear `linear` (0..6: q, k,
 * v, o, gate, up, down) in its deployed int4 form.  [AWQ-W4 card] scale-rewrite
 * paragraph: the rewrite prev_op /= s, W *= s runs as the input bf16(a / s) (IEEE
 * fp32 division, rounded to nearest even) against the packed weights of
 * Q(W diag(s)) on the int4 GEMM (w4a16_gemm), exactly as awq_lookahead_loss scores
 * a candidate; every other op as in w4_block_forward.
 *   s [K] fp32 device (K the linear's input size, every s[k] > 0).  qweight,
 *   scales, qzeros: the linear's packed weights [N][K/8], [N][K/128],
 *   [N][ceil(K/1024)] as written by awq_quantize_pack (qzeros NULL iff
 *   symmetric).  X, Y, blk, shapes and the workspace size query as in
 *   w4_block_forward; the size also depends on `linear`.
 */
int w4_block_forward_quantized(const uint16_t* X, int B, int L, int hidden, int n_q, int n_kv, int inter,
                               const w4_block* blk, int linear, const float* s, const uint32_t* qweight,
                               const uint16_t* scales, const uint32_t* qzeros, int symmetric, int group_size,
                               uint16_t* Y, void* workspace, size_t* workspace_bytes, void* stream);

/*
 * awq_lookahead_loss -- look-ahead (d = 1) scoring of C candidates for one linear of
 * block `blk`.  [AWQ-W4 card] "Search" and the paragraph under it: the candidate
 * weights go into this block, the MSE is taken at the output of the next block
 * `next`, which runs unquantized; the reference is the same path with this block
 * unquantized; with next == NULL (the last block) the loss is taken at this
 * block's own output.  Candidate c replaces linear `linear` (0..6: q, k, v, o,
 * gate, up, down) by its deployed form: input bf16(a / S[c]) against the int4
 * codes Q(W diag(S[c]), ratios[c]) (awq_quantize_pack, symmetric or not).
 *   losses[c] = mean over the B L tokens and H outputs of (y_c - y_ref)^2, both
 *   bf16 outputs of the scored block, fp64 sum in a fixed order, stored fp32.
 *   losses_d0[c] (or NULL) = the same at this block's output (d = 0).
 *   X [B L][H] bf16: the input of this block.  S [C][K] fp32 device (K the
 *   linear's input size), ratios [C] fp32 device in (0, 1].  Blocks as in
 *   w4_block_forward.  Workspace: size query; it depends on the shape and on
 *   `linear`.  Candidates run one after another on `stream`.
 */
int awq_lookahead_loss(const uint16_t* X, int B, int L, int hidden, int n_q, int n_kv, int inter,
                       const w4_block* blk, const w4_block* next, int linear, const float* S,
                       const float* ratios, int C, int symmetric, int group_size, float* losses,
                       float* losses_d0, void* workspace, size_t* workspace_bytes, void* stream);

/*
 * awq_search_lookahead -- the two-phase search of [AWQ-W4 card] "Search" scored
 * with the look-ahead loss of awq_lookahead_loss: m_k = mean_t |a[t][k]| of the
 * linear's input a in the reference pass (device, fp64, fixed order), s(alpha) as in
 * awq_search (host fp64, stored fp32); every alpha at r = 1, first minimum alpha*;
 * then every ratio at s(alpha*), first minimum r*.
 *   alphas [n_alpha], ratios [n_ratio]: host fp64 (1 <= n <= 64 each; alphas in
 *   [0, 16], ratios in (0, 1]).  losses_out [n_alpha + n_ratio]: host fp32 out
 *   (d = 1 losses).  alpha_index, ratio_index: host int out.  s_out [K] fp32
 *   device out: s(alpha*).  Workspace as in awq_search (size query, then
 *   required).  Synchronizes `stream` (three times).
 */
int awq_search_lookahead(const uint16_t* X, int B, int L, int hidden, int n_q, int n_kv, int inter,
                         const w4_block* blk, const w4_block* next, int linear, const double* alphas,
                         int n_alpha, const double* ratios, int n_ratio, int symmetric, int group_size,
                         float* losses_out, int* alpha_index, int* ratio_index, float* s_out,
                         void* workspace, size_t* workspace_bytes, void* stream);

/*
 * Measurement helpers (not part of the method): the yardsticks the kernels
 * above are measured against on the same device.
 *
 * w4_probe_stream_read -- read `bytes` (multiple of 16, 16-byte aligned) from
 *   device buffer `buf` with a grid-stride loop of `blocks` x 256 threads, each
 *   thread loading `unroll` (1, 2, 4 or 8) 16-byte chunks per iteration
 *   (non-temporal loads if `nontemporal`), and write one uint32 XOR per thread
 *   to `sink` (blocks * 256 uint32, device).  Its duration gives the bandwidth a
 *   plain read reaches at that size, and its known traffic scales the hardware
 *   fetch counters.
 * w4_probe_empty -- launch a kernel that does nothing (one 64-thread block):
 *   the launch-duration floor.
 */
int w4_probe_stream_read(const void* buf, size_t bytes, int unroll, int nontemporal, int blocks,
                         uint32_t* sink, void* stream);
int w4_probe_empty(void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
