// Internal interfaces between the C-ABI entry points (w4a16_abi.hip) and the
// kernel launchers.  Launchers assume validated arguments.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace w4 {

struct QuantArgs {
  const uint16_t* W;   // [N][K] bf16
  int N, K;
  const float* s;      // [C][s_stride] or NULL
  size_t s_stride;
  float ratio;         // used when ratios == NULL
  const float* ratios; // [C] or NULL
  int symmetric;
  uint32_t* qweight;   // [C][qw_stride]
  size_t qw_stride;
  uint16_t* scales;    // [C][sc_stride]
  size_t sc_stride;
  uint32_t* qzeros;    // [C][qz_stride] (asymmetric only)
  size_t qz_stride;
};

int launch_quantize_pack(const QuantArgs& a, int C, hipStream_t stream);

// ---------------------------------------------------------------- GEMV (M <= 16)
// Whether a decode GEMV of this shape runs on the matrix cores (gemv_mfma.hip)
// instead of the vector ALUs (gemv.hip).
bool gemv_use_mfma(int M, int K, int N);
// W4_ERR_SHAPE when a GEMV or GEMM of this shape would exceed the kernels' 32-bit
// buffer offsets (checked by the entry points before their size queries, too).
int gemv_check_size(int M, int K, int N);
int gemm_check_size(int M, int K, int N);
size_t gemv_workspace_bytes(int M, int K, int N);
int launch_gemv(const uint16_t* X, int M, int K, int N, const uint32_t* qweight,
                const uint16_t* scales, const uint32_t* qzeros, int symmetric, uint16_t* Y,
                void* workspace, hipStream_t stream);
size_t gemv_mfma_workspace_bytes(int M, int K, int N);
int launch_gemv_mfma(const uint16_t* X, int M, int K, int N, const uint32_t* qweight,
                     const uint16_t* scales, const uint32_t* qzeros, int symmetric, uint16_t* Y,
                     void* workspace, hipStream_t stream);
// Y[i] = bf16(sum over k < splits of partial[k * stride + i]) for i < count, in split order.
int launch_split_reduce(const float* partial, int splits, size_t stride, size_t count, uint16_t* Y,
                        hipStream_t stream);
// The same with stride = count = MN.
int launch_gemv_split_reduce(const float* partial, int splits, size_t MN, uint16_t* Y, hipStream_t stream);

// ---------------------------------------------------------------- W4A8 decode (M <= 16)
int launch_w4a8_quantize(const uint16_t* X, int M, int K, int8_t* Xq, float* sx, int32_t* xsum,
                         hipStream_t stream);
int w4a8_plan(int K, int N, int cus, int* ni, int* waves, size_t* lds);   // W4_ERR_UNSUPPORTED when K is too long
int launch_w4a8_gemv(const int8_t* Xq, const float* sx, const int32_t* xsum, int M, int K, int N,
                     const uint32_t* qweight, const uint16_t* scales, const uint32_t* qzeros, int symmetric,
                     uint16_t* Y, void* workspace, hipStream_t stream);
size_t w4a8_workspace_bytes(int M, int K, int N);   // fp32 partials of a K split (0 without one)

// ---------------------------------------------------------------- GEMM (MFMA)
// Which kernels serve w4a16_gemm: up to 16 rows the decode GEMV's (gemm_use_gemv), up
// to kSkinnyMaxM rows the one-pass kernel of gemm_skinny.hip (when the 32-bit buffer
// offsets of either cover the shape), else the tiled core.
bool gemm_use_gemv(int M, int K, int N);
constexpr int kSkinnyMaxM = 48;
bool gemm_use_skinny(int M, int K, int N);
size_t gemm_skinny_workspace_bytes(int M, int K, int N);
int launch_gemm_skinny(const uint16_t* X, int M, int K, int N, const uint32_t* qweight,
                       const uint16_t* scales, const uint32_t* qzeros, int symmetric, uint16_t* Y,
                       void* workspace, hipStream_t stream);
size_t gemm_workspace_bytes(int M, int K, int N);
int launch_gemm(const uint16_t* X, int M, int K, int N, const uint32_t* qweight,
                const uint16_t* scales, const uint32_t* qzeros, int symmetric, uint16_t* Y,
                void* workspace, hipStream_t stream);

// ---------------------------------------------------------------- grid loss
int grid_loss_check_size(int T, int K, int N, int C);
size_t grid_loss_workspace_bytes(int T, int K, int N, int C, bool need_yref);
// shared_s: every row of S is the same (the ratio phase of the search, at s(alpha*)):
// the scaled activations and their row sums are formed once for all candidates.
int launch_grid_loss(const uint16_t* X, int T, int K, int N, const uint16_t* W,
                     const uint16_t* Yref, const float* S, const float* ratios, int C,
                     int symmetric, float* losses, void* workspace, hipStream_t stream,
                     bool shared_s = false);

// ---------------------------------------------------------------- per-channel clipping search
size_t clip_search_workspace_bytes(int T, int K);
int launch_clip_search(const uint16_t* X, int T, int K, int N, const uint16_t* W, const float* s,
                       const float* ratios, int R, int symmetric, float* losses, uint8_t* best,
                       void* workspace, hipStream_t stream);

// ---------------------------------------------------------------- decoder block / look-ahead loss
size_t block_forward_workspace_bytes(int B, int L, int H, int nq, int nkv, int I);
int launch_block_forward(const uint16_t* X, int B, int L, int H, int nq, int nkv, int I, const w4_block& blk,
                         uint16_t* Y, void* workspace, hipStream_t stream);
size_t block_quantized_workspace_bytes(int B, int L, int H, int nq, int nkv, int I, int linear);
int launch_block_forward_quantized(const uint16_t* X, int B, int L, int H, int nq, int nkv, int I,
                                   const w4_block& blk, int linear, const float* s, const uint32_t* qweight,
                                   const uint16_t* scales, const uint32_t* qzeros, int symmetric, uint16_t* Y,
                                   void* workspace, hipStream_t stream);
size_t lookahead_workspace_bytes(int B, int L, int H, int nq, int nkv, int I, int linear);
int launch_lookahead_loss(const uint16_t* X, int B, int L, int H, int nq, int nkv, int I, const w4_block& blk,
                          const w4_block* next, int linear, const float* S, const float* ratios, int C,
                          int symmetric, float* losses, float* losses_d0, void* workspace, hipStream_t stream);
int lookahead_input_size(int H, int nq, int I, int linear);
// With m_host and m_ready set (and m), the statistic is also copied to m_host (K doubles)
// and m_ready recorded right after it, before the next block is enqueued.
int launch_lookahead_reference(const uint16_t* X, int B, int L, int H, int nq, int nkv, int I, const w4_block& blk,
                               const w4_block* next, int linear, double* m, void* workspace, hipStream_t stream,
                               double* m_host = nullptr, hipEvent_t m_ready = nullptr);
int launch_lookahead_candidates(const uint16_t* X, int B, int L, int H, int nq, int nkv, int I, const w4_block& blk,
                                const w4_block* next, int linear, const float* S, const float* ratios, int C,
                                int symmetric, float* losses, float* losses_d0, void* workspace,
                                hipStream_t stream);

// Y = bf16(X W^T) with bf16 weights W [N][K] on the library's bf16 MFMA kernel
// (K a multiple of 64).
int launch_bf16_gemm(const uint16_t* X, int M, int K, int N, const uint16_t* W, uint16_t* Y, hipStream_t stream);
// One launch for up to three weights W[s] [N[s]][K] reading the same X: Y[s] = bf16(X W[s]^T),
// or bf16(R[s] + bf16(X W[s]^T)) with residuals R (NULL: none; R[s] NULL: none for s).
int launch_bf16_gemm_multi(const uint16_t* X, int M, int K, int nseg, const uint16_t* const* W, const int* N,
                           uint16_t* const* Y, hipStream_t stream, const uint16_t* const* R = nullptr);
// As launch_bf16_gemm_multi without residuals; the segments whose bit is set in
// rope_mask (N[s] a multiple of the head size 128) get the rotary embedding of row
// position row % L from the tables cs, sn [L][64], as the standalone rope kernel.
int launch_bf16_gemm_rope(const uint16_t* X, int M, int K, int nseg, const uint16_t* const* W, const int* N,
                          uint16_t* const* Y, int rope_mask, const float* cs, const float* sn, int L,
                          hipStream_t stream);
// Y = bf16(silu(bf16(X Wg^T)) bf16(X Wu^T)) [M][N] in one launch (gate and up [N][K]).
int launch_bf16_glu(const uint16_t* X, int M, int K, int N, const uint16_t* Wg, const uint16_t* Wu, uint16_t* Y,
                    hipStream_t stream);

// Y = bf16(X W^T) with bf16 weights W [N][K] (the unquantized reference output).
int launch_reference_gemm(const uint16_t* X, int M, int K, int N, const uint16_t* W, uint16_t* Y,
                          hipStream_t stream);

// m_k = mean_t |X[t][k]| in fp64, fixed summation order.
// m must hold (1 + ceil(T / 64)) * K doubles: m[0..K) is the result, the rest
// per-chunk partial sums.
int launch_act_mean_abs(const uint16_t* X, int T, int K, double* m, hipStream_t stream);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace w4
