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
//  * blocks [0, rsx_blocks): one wave per (row m < mpad, triple t): lanes 0..47
//    each sum 8 consecutive bf16 of the triple's 384 channels (fp32, fixed order),
//    16-lane xor trees give the three group sums, lane 0 writes the 16 slots;
//  * the remaining blocks: one thread per (triple t, column n < npad) writes the
//    16 slots of -sc (128 + z) and the triple's scales group-major (0 past N).
__global__ __launch_bounds__(256) void zterm_prep_kernel(const uint16_t* X, size_t x_stride, int M, int K,
                                                         int mpad, const uint16_t* scales, size_t sc_stride,
                                                         const uint32_t* qzeros, size_t qz_stride, int symmetric,
                                                         int N, uint16_t* rsx, size_t rsx_stride, uint16_t* cz,
                                                         size_t cz_stride, uint16_t* sct, size_t sct_stride,
                                                         uint16_t* xp, int rsx_blocks) {
#pragma clang fp contract(off)
  const int G = K >> 7;
  const int T3 = (G + 2) / 3;
  const int kz = 16 * T3;
  const int c = blockIdx.z;
  if ((int)blockIdx.x < rsx_blocks) {
    const int lane = threadIdx.x & 63;
    const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= (long long)mpad * T3) return;            // uniform per wave
    const int m = (int)(item / T3);
    const int t = (int)(item % T3);
    const int j = lane >> 4;
    const int g = 3 * t + j;
    float s = 0.0f;
    if (m < M && j < 3 && g < G) {
      const size_t off = (size_t)c * x_stride + (size_t)m * K + (size_t)g * kGroup + (lane & 15) * 8;
      const uint4 v = *reinterpret_cast<const uint4*>(X + off);
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) s += __uint_as_float(d[q] << 16) + __uint_as_float(d[q] & 0xFFFF0000u);
      if (xp) {
        uint32_t e[4];
        pair_activations(d, e);
        *reinterpret_cast<uint4*>(xp + off) = make_uint4(e[0], e[1], e[2], e[3]);
      }
    } else if (xp && m >= M && j < 3 && g < G) {      // padding rows of xp
      const size_t off = (size_t)c * x_stride + (size_t)m * K + (size_t)g * kGroup + (lane & 15) * 8;
      *reinterpret_cast<uint4*>(xp + off) = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) s += __shfl_xor(s, off, kWave);
    const float r0 = __shfl(s, 0, kWave), r1 = __shfl(s, 16, kWave), r2 = __shfl(s, 32, kWave);
    if (lane == 0) {
      uint32_t sl[16];
      const float rr[3] = {r0, r1, r2};
#pragma unroll
      for (int jj = 0; jj < 3; ++jj) {
        uint32_t hi, mid, lo;
        split3(rr[jj], hi, mid, lo);
        sl[5 * jj + 0] = hi;
        sl[5 * jj + 1] = hi;
        sl[5 * jj + 2] = mid;
        sl[5 * jj + 3] = mid;
        sl[5 * jj + 4] = lo;
      }
      sl[15] = 0;
      uint4* dst = reinterpret_cast<uint4*>(rsx + (size_t)c * rsx_stride + (size_t)m * kz + 16 * t);
      dst[0] = make_uint4(sl[0] | sl[1] << 16, sl[2] | sl[3] << 16, sl[4] | sl[5] << 16, sl[6] | sl[7] << 16);
      dst[1] = make_uint4(sl[8] | sl[9] << 16, sl[10] | sl[11] << 16, sl[12] | sl[13] << 16, sl[14] | sl[15] << 16);
    }
  } else {
    const int npad = (N + 127) & ~127;
    const long long item = (long long)(blockIdx.x - rsx_blocks) * 256 + threadIdx.x;
    if (item >= (long long)npad * T3) return;
    const int t = (int)(item / npad);
    const int n = (int)(item % npad);
    uint16_t* sct_c = sct + (size_t)c * sct_stride;
    if (n >= N) {                                          // padding columns: scale 0
      for (int jj = 0; jj < 3; ++jj)
        if (3 * t + jj < G) sct_c[(size_t)(3 * t + jj) * npad + n] = 0;
      return;
    }
    const int GW = (G + 7) >> 3;
    uint32_t sl[16];
#pragma unroll
    for (int jj = 0; jj < 3; ++jj) {
      const int g = 3 * t + jj;
      uint32_t hi = 0, lo = 0;
      if (g < G) {
        const uint16_t scb = scales[(size_t)c * sc_stride + (size_t)n * G + g];
        sct_c[(size_t)g * npad + n] = scb;
        const float sc = bf16_bits_to_f32(scb);
        uint32_t z = 8;
        if (!symmetric) z = (qzeros[(size_t)c * qz_stride + (size_t)n * GW + (g >> 3)] >> (4 * (g & 7))) & 0xFu;
        const float cv = -(sc * (float)(128u + z));          // exact: at most 16 significant bits
        hi = f32_to_bf16_bits(cv);
        lo = f32_to_bf16_bits(cv - bf16_bits_to_f32(hi));   // exact residual
      }
      sl[5 * jj + 0] = hi;
      sl[5 * jj + 1] = lo;
      sl[5 * jj + 2] = hi;
      sl[5 * jj + 3] = lo;
      sl[5 * jj + 4] = hi;
    }
    sl[15] = 0;
    uint4* dst = reinterpret_cast<uint4*>(cz + (size_t)c * cz_stride + (size_t)n * kz + 16 * t);
    dst[0] = make_uint4(sl[0] | sl[1] << 16, sl[2] | sl[3] << 16, sl[4] | sl[5] << 16, sl[6] | sl[7] << 16);
    dst[1] = make_uint4(sl[8] | sl[9] << 16, sl[10] | sl[11] << 16, sl[12] | sl[13] << 16, sl[14] | sl[15] << 16);
  }
}

int launch_zterm_prep(const uint16_t* X, size_t x_stride, int M, int K, int mpad, const uint16_t* scales,
                      size_t sc_stride, const uint32_t* qzeros, size_t qz_stride, int symmetric, int N,
                      uint16_t* rsx, size_t rsx_stride, uint16_t* cz, size_t cz_stride, uint16_t* sct,
                      size_t sct_stride, uint16_t* xp, int C, hipStream_t stream) {
  const int T3 = ((K >> 7) + 2) / 3;
  const long long rsx_blocks = ((long long)mpad * T3 + 3) / 4;
  const long long cz_blocks = ((long long)gemm_npad(N) * T3 + 255) / 256;
  if (rsx_blocks + cz_blocks == 0) return W4_OK;
  if (rsx_blocks + cz_blocks > 0x7FFFFFFFLL || C > 65535) return W4_ERR_SHAPE;
  hipLaunchKernelGGL(zterm_prep_kernel, dim3((unsigned)(rsx_blocks + cz_blocks), 1, (unsigned)C), dim3(256), 0,
                     stream, X, x_stride, M, K, mpad, scales, sc_stride, symmetric ? nullptr : qzeros, qz_stride,
                     symmetric, N, rsx, rsx_stride, cz, cz_stride, sct, sct_stride, xp, (int)rsx_blocks);
  W4_CHECK_LAUNCH();
  return W4_OK;
}


// workspace: pair-arranged X [mpad][K] bf16 (rows >= M zero), rsx [mpad][kz] bf16,
// cz [N][kz] bf16, sct [K/128][npad] bf16
size_t gemm_workspace_bytes(int M, int K, int N) {
  if (M <= 0 || K <= 0 || N <= 0) return 0;
  const size_t mpad = align_up((size_t)M, kBM);
  const size_t kz = (size_t)zterm_kz(K);
  return align_up(mpad * K * 2, 256) + align_up(mpad * kz * 2, 256) + align_up((size_t)N * kz * 2, 256) +
         align_up((size_t)(K / kGroup) * gemm_npad(N) * 2, 256);
}

int launch_gemm(const uint16_t* X, int M, int K, int N, const uint32_t* qweight,
                const uint16_t* scales, const uint32_t* qzeros, int symmetric, uint16_t* Y,
                void* workspace, hipStream_t stream) {
  if (M == 0 || N == 0) return W4_OK;
  // 32-bit per-lane byte offsets in the kernel: 2 mpad K and N K / 2 below 2^32
  if (((long long)M + kBM) * K >= (1LL << 31) || (long long)N * K >= (1LL << 33)) return W4_ERR_SHAPE;
  const int mpad = (int)align_up((size_t)M, kBM);
  const int kz = zterm_kz(K);
  char* ws = static_cast<char*>(workspace);
  uint16_t* xp = reinterpret_cast<uint16_t*>(ws);
  ws += align_up((size_t)mpad * K * 2, 256);
  uint16_t* rsx = reinterpret_cast<uint16_t*>(ws);
  ws += align_up((size_t)mpad * kz * 2, 256);
  uint16_t* cz = reinterpret_cast<uint16_t*>(ws);
  ws += align_up((size_t)N * kz * 2, 256);
  uint16_t* sct = reinterpret_cast<uint16_t*>(ws);
  int st = launch_zterm_prep(X, 0, M, K, mpad, scales, 0, qzeros, 0, symmetric, N, rsx, 0, cz, 0, sct, 0, xp, 1,
                             stream);
  if (st != W4_OK) return st;
  GemmCoreArgs a{};
  a.X = xp;
  a.M = M;
  a.K = K;
  a.N = N;
  a.qweight = qweight;
  a.sct = sct;
  a.npad = gemm_npad(N);
  a.rsx = rsx;
  a.cz = cz;
  a.kz = kz;
  a.Y = Y;
  const long long tiles = (long long)((N + kBN - 1) / kBN) * ((M + kBM - 1) / kBM);
  if (tiles > 0x7FFFFFFFLL) return W4_ERR_SHAPE;
  const dim3 grid((unsigned)tiles, 1, 1);
  hipLaunchKernelGGL((gemm_core_kernel<true, EPI_STORE>), grid, dim3(256), 0, stream, a);
  W4_CHECK_LAUNCH();
  return W4_OK;
}

}  // namespace w4
