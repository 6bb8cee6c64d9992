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
size_t gemv_workspace_bytes(int M, int K, int N);
int launch_gemv(const uint16_t* X, int M, int K, int N, const uint32_t* qweight,
                const uint16_t* scales, const uint32_t* qzeros, int symmetric, uint16_t* Y,
                void* workspace, hipStream_t stream);

// ---------------------------------------------------------------- W4A8 decode (M <= 16)
int launch_w4a8_quantize(const uint16_t* X, int M, int K, int8_t* Xq, float* sx, int32_t* xsum,
                         hipStream_t stream);
int w4a8_plan(int K, int N, int cus, int* ni, int* waves, size_t* lds);   // W4_ERR_UNSUPPORTED when K is too long
int launch_w4a8_gemv(const int8_t* Xq, const float* sx, const int32_t* xsum, int M, int K, int N,
                     const uint32_t* qweight, const uint16_t* scales, const uint32_t* qzeros, int symmetric,
                     uint16_t* Y, void* workspace, hipStream_t stream);
size_t w4a8_workspace_bytes(int M, int K, int N);   // fp32 partials of a K split (0 without one)

// ---------------------------------------------------------------- GEMM (MFMA)
size_t gemm_workspace_bytes(int M, int K, int N);
int launch_gemm(const uint16_t* X, int M, int K, int N, const uint32_t* qweight,
                const uint16_t* scales, const uint32_t* qzeros, int symmetric, uint16_t* Y,
                void* workspace, hipStream_t stream);

// ---------------------------------------------------------------- grid loss
size_t grid_loss_workspace_bytes(int T, int K, int N, int C, bool need_yref);
int launch_grid_loss(const uint16_t* X, int T, int K, int N, const uint16_t* W,
                     const uint16_t* Yref, const float* S, const float* ratios, int C,
                     int symmetric, float* losses, void* workspace, hipStream_t stream);

// ---------------------------------------------------------------- per-channel clipping search
size_t clip_search_workspace_bytes(int T, int K);
int launch_clip_search(const uint16_t* X, int T, int K, int N, const uint16_t* W, const float* s,
                       const float* ratios, int R, int symmetric, float* losses, uint8_t* best,
                       void* workspace, hipStream_t stream);

// ---------------------------------------------------------------- decoder block / look-ahead loss
size_t block_forward_workspace_bytes(int B, int L, int H, int nq, int nkv, int I);
int launch_block_forward(const uint16_t* X, int B, int L, int H, int nq, int nkv, int I, const w4_block& blk,
                         uint16_t* Y, void* workspace, hipStream_t stream);
size_t lookahead_workspace_bytes(int B, int L, int H, int nq, int nkv, int I, int linear);
int launch_lookahead_loss(const uint16_t* X, int B, int L, int H, int nq, int nkv, int I, const w4_block& blk,
                          const w4_block* next, int linear, const float* S, const float* ratios, int C,
                          int symmetric, float* losses, float* losses_d0, void* workspace, hipStream_t stream);
int lookahead_input_size(int H, int nq, int I, int linear);
int launch_lookahead_reference(const uint16_t* X, int B, int L, int H, int nq, int nkv, int I, const w4_block& blk,
                               const w4_block* next, int linear, double* m, void* workspace, hipStream_t stream);
int launch_lookahead_candidates(const uint16_t* X, int B, int L, int H, int nq, int nkv, int I, const w4_block& blk,
                                const w4_block* next, int linear, const float* S, const float* ratios, int C,
                                int symmetric, float* losses, float* losses_d0, void* workspace,
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
