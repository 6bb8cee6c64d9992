// Prefill contraction Y = X W_hat^T on MFMA (model card
// "GLM-5.2-QSRT-Fruit-Instruct", "Reproducible runtime": W4A16 serves prefill row
// counts; model card "Qwen3.6-27B-W4A16": int4 weights, 16-bit activations).
#include "gemm_core.hpp"

namespace w4 {

// rs[z][g][m] = sum of the 128 bf16 values X[z][m][128 g .. 128 g + 127] in fp32,
// fixed order; rows m >= M (up to mpad) are written as 0.
// One wave per (row, 4-group slab): lane -> 8 channels, 16 lanes per group.
__global__ __launch_bounds__(256) void group_rowsum_kernel(const uint16_t* X, size_t x_stride, int M,
                                                           int K, int mpad, float* rs, size_t rs_stride) {
  const int lane = threadIdx.x & 63;
  const int G = K >> 7;
  const int slabs = (G + 3) >> 2;
  const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (long long)mpad * slabs) return;
  const int m = (int)(item / slabs);
  const int slab = (int)(item % slabs);
  const int g = slab * 4 + (lane >> 4);
  const int z = blockIdx.z;
  float s = 0.0f;
  if (m < M && g < G) {
    const uint4 v = *reinterpret_cast<const uint4*>(X + (size_t)z * x_stride + (size_t)m * K + (size_t)g * kGroup + (lane & 15) * 8);
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) s += __uint_as_float(d[q] << 16) + __uint_as_float(d[q] & 0xFFFF0000u);
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) s += __shfl_xor(s, off, kWave);
  if ((lane & 15) == 0 && g < G) rs[(size_t)z * rs_stride + (size_t)g * mpad + m] = s;
}

int launch_group_rowsum(const uint16_t* X, size_t x_stride, int M, int K, int mpad, float* rs,
                               size_t rs_stride, int C, hipStream_t stream) {
  const long long items = (long long)mpad * (((K >> 7) + 3) >> 2);
  const long long blocks = (items + 3) / 4;
  if (blocks == 0) return W4_OK;
  hipLaunchKernelGGL(group_rowsum_kernel, dim3((unsigned)blocks, 1, (unsigned)C), dim3(256), 0, stream, X,
                     x_stride, M, K, mpad, rs, rs_stride);
  W4_CHECK_LAUNCH();
  return W4_OK;
}


size_t gemm_workspace_bytes(int M, int K, int N) {
  (void)N;
  if (M <= 0 || K <= 0) return 0;
  const size_t mpad = align_up((size_t)M, kBM);
  return align_up((size_t)(K / kGroup) * mpad * sizeof(float), 256);
}

int launch_gemm(const uint16_t* X, int M, int K, int N, const uint32_t* qweight,
                const uint16_t* scales, const uint32_t* qzeros, int symmetric, uint16_t* Y,
                void* workspace, hipStream_t stream) {
  if (M == 0 || N == 0) return W4_OK;
  const int mpad = (int)align_up((size_t)M, kBM);
  float* rs = static_cast<float*>(workspace);
  int st = launch_group_rowsum(X, 0, M, K, mpad, rs, 0, 1, stream);
  if (st != W4_OK) return st;
  GemmCoreArgs a{};
  a.X = X;
  a.M = M;
  a.K = K;
  a.N = N;
  a.qweight = qweight;
  a.scales = scales;
  a.qzeros = symmetric ? nullptr : qzeros;
  a.symmetric = symmetric;
  a.rs = rs;
  a.mpad = mpad;
  a.Y = Y;
  dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM), 1);
  if (grid.y > 65535) return W4_ERR_SHAPE;
  hipLaunchKernelGGL((gemm_core_kernel<true, EPI_STORE>), grid, dim3(256), 0, stream, a);
  W4_CHECK_LAUNCH();
  return W4_OK;
}

}  // namespace w4
