// Prefill contraction Y = X W_hat^T on MFMA (model card
// "GLM-5.2-QSRT-Fruit-Instruct", "Reproducible runtime": W4A16 serves prefill row
// counts; model card "Qwen3.6-27B-W4A16": int4 weights, 16-bit activations).
#include "gemm_core.hpp"

namespace w4 {

// Exact splits into bf16 parts (round to nearest even each time; every residual
// is exact in fp32).
__device__ __forceinline__ void split3(float v, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = f32_to_bf16_bits(v);
  const float r1 = v - bf16_bits_to_f32(hi);
  mid = f32_to_bf16_bits(r1);
  const float r2 = r1 - bf16_bits_to_f32(mid);
  lo = f32_to_bf16_bits(r2);
}

// One launch, two jobs (grid.z = problem c):
//  * blocks [0, rs_blocks): one wave per (row m < mpad, triple of groups t):
//    lanes 0..47 each sum 8 consecutive bf16 of the triple's 384 channels (fp32,
//    fixed order), 16-lane xor trees give the three group sums; lane 0 writes
//    rsq[g][m] = the negated sum split into three bf16 parts (exact) and a zero
//    (rows >= M: zeros), and, when xp is set, every lane writes its 8 channels
//    of X pair-arranged into xp (rows >= M: zeros);
//  * the remaining blocks: one thread per (triple t, column n < npad) writes
//    szq[g][n] = scale bits | bf16(128 + z) << 16 (0 for n >= N).
__global__ __launch_bounds__(256) void gemm_prep_kernel(const uint16_t* X, size_t x_stride, int M, int K, int mpad,
                                                        const uint16_t* scales, size_t sc_stride,
                                                        const uint32_t* qzeros, size_t qz_stride, int symmetric,
                                                        int N, uint16_t* rsq, size_t rsq_stride, uint32_t* szq,
                                                        size_t szq_stride, uint16_t* xp, int rs_blocks) {
#pragma clang fp contract(off)
  const int G = K >> 7;
  const int T3 = (G + 2) / 3;
  const int c = blockIdx.z;
  if ((int)blockIdx.x < rs_blocks) {
    const int lane = threadIdx.x & 63;
    const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= (long long)mpad * T3) return;            // uniform per wave
    const int m = (int)(item / T3);
    const int t = (int)(item % T3);
    const int j = lane >> 4;
    const int g = 3 * t + j;
    float s = 0.0f;
    if (j < 3 && g < G) {
      const size_t off = (size_t)c * x_stride + (size_t)m * K + (size_t)g * kGroup + (lane & 15) * 8;
      if (m < M) {
        const uint4 v = *reinterpret_cast<const uint4*>(X + off);
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) s += __uint_as_float(d[q] << 16) + __uint_as_float(d[q] & 0xFFFF0000u);
        if (xp) {
          uint32_t e[4];
          pair_activations(d, e);
          *reinterpret_cast<uint4*>(xp + off) = make_uint4(e[0], e[1], e[2], e[3]);
        }
      } else if (xp) {
        *reinterpret_cast<uint4*>(xp + off) = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) s += __shfl_xor(s, off, kWave);
    const float r0 = __shfl(s, 0, kWave), r1 = __shfl(s, 16, kWave), r2 = __shfl(s, 32, kWave);
    if (lane == 0) {
      const float rr[3] = {r0, r1, r2};
#pragma unroll
      for (int jj = 0; jj < 3; ++jj) {
        const int gg = 3 * t + jj;
        if (gg >= G) break;
        uint32_t hi, mid, lo;
        split3(-rr[jj], hi, mid, lo);
        *reinterpret_cast<uint2*>(rsq + (size_t)c * rsq_stride + ((size_t)gg * mpad + m) * 4) =
            make_uint2(hi | (mid << 16), lo);
      }
    }
  } else {
    const int npad = gemm_npad(N);
    const long long item = (long long)(blockIdx.x - rs_blocks) * 256 + threadIdx.x;
    if (item >= (long long)npad * T3) return;
    const int t = (int)(item / npad);
    const int n = (int)(item % npad);
    const int GW = (G + 7) >> 3;
    for (int jj = 0; jj < 3; ++jj) {
      const int g = 3 * t + jj;
      if (g >= G) break;
      uint32_t v = 0;
      if (n < N) {
        const uint32_t scb = scales[(size_t)c * sc_stride + (size_t)n * G + g];
        uint32_t z = 8;
        if (!symmetric) z = (qzeros[(size_t)c * qz_stride + (size_t)n * GW + (g >> 3)] >> (4 * (g & 7))) & 0xFu;
        v = scb | ((0x4300u | z) << 16);                      // bf16 0x4300 | z = 128 + z exactly
      }
      szq[(size_t)c * szq_stride + (size_t)g * npad + n] = v;
    }
  }
}

int launch_gemm_prep(const uint16_t* X, size_t x_stride, int M, int K, int mpad, const uint16_t* scales,
                     size_t sc_stride, const uint32_t* qzeros, size_t qz_stride, int symmetric, int N,
                     uint16_t* rsq, size_t rsq_stride, uint32_t* szq, size_t szq_stride, uint16_t* xp, int C,
                     hipStream_t stream) {
  const int T3 = ((K >> 7) + 2) / 3;
  const long long rs_blocks = ((long long)mpad * T3 + 3) / 4;
  const long long sz_blocks = ((long long)gemm_npad(N) * T3 + 255) / 256;
  if (rs_blocks + sz_blocks == 0) return W4_OK;
  if (rs_blocks + sz_blocks > 0x7FFFFFFFLL || C > 65535) return W4_ERR_SHAPE;
  hipLaunchKernelGGL(gemm_prep_kernel, dim3((unsigned)(rs_blocks + sz_blocks), 1, (unsigned)C), dim3(256), 0,
                     stream, X, x_stride, M, K, mpad, scales, sc_stride, symmetric ? nullptr : qzeros, qz_stride,
                     symmetric, N, rsq, rsq_stride, szq, szq_stride, xp, (int)rs_blocks);
  W4_CHECK_LAUNCH();
  return W4_OK;
}


// workspace: pair-arranged X [mpad][K] bf16 (rows >= M zero), rsq [G][mpad][4] bf16,
// szq [G][npad] u32
size_t gemm_workspace_bytes(int M, int K, int N) {
  if (M <= 0 || K <= 0 || N <= 0) return 0;
  const size_t mpad = align_up((size_t)M, kBM);
  const size_t G = (size_t)(K / kGroup);
  return align_up(mpad * K * 2, 256) + align_up(G * mpad * 8, 256) + align_up(G * gemm_npad(N) * 4, 256);
}

int launch_gemm(const uint16_t* X, int M, int K, int N, const uint32_t* qweight,
                const uint16_t* scales, const uint32_t* qzeros, int symmetric, uint16_t* Y,
                void* workspace, hipStream_t stream) {
  if (M == 0 || N == 0) return W4_OK;
  // 32-bit per-lane byte offsets in the kernel: 2 mpad K and N K / 2 below 2^32
  if (((long long)M + kBM) * K >= (1LL << 31) || (long long)N * K >= (1LL << 33)) return W4_ERR_SHAPE;
  const int mpad = (int)align_up((size_t)M, kBM);
  const int G = K / kGroup;
  char* ws = static_cast<char*>(workspace);
  uint16_t* xp = reinterpret_cast<uint16_t*>(ws);
  ws += align_up((size_t)mpad * K * 2, 256);
  uint16_t* rsq = reinterpret_cast<uint16_t*>(ws);
  ws += align_up((size_t)G * mpad * 8, 256);
  uint32_t* szq = reinterpret_cast<uint32_t*>(ws);
  int st = launch_gemm_prep(X, 0, M, K, mpad, scales, 0, qzeros, 0, symmetric, N, rsq, 0, szq, 0, xp, 1, stream);
  if (st != W4_OK) return st;
  GemmCoreArgs a{};
  a.X = xp;
  a.M = M;
  a.K = K;
  a.N = N;
  a.qweight = qweight;
  a.rsq = rsq;
  a.szq = szq;
  a.mpad = mpad;
  a.npad = gemm_npad(N);
  a.Y = Y;
  const long long tiles = (long long)((N + kBN - 1) / kBN) * ((M + kBM - 1) / kBM);
  if (tiles > 0x7FFFFFFFLL) return W4_ERR_SHAPE;
  const dim3 grid((unsigned)tiles, 1, 1);
  hipLaunchKernelGGL((gemm_core_kernel<true, EPI_STORE>), grid, dim3(kGemmWaves * 64), 0, stream, a);
  W4_CHECK_LAUNCH();
  return W4_OK;
}

}  // namespace w4
