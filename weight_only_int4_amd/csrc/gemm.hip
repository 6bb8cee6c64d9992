// Prefill contraction Y = X W_hat^T on MFMA (model card
// "GLM-5.2-QSRT-Fruit-Instruct", "Reproducible runtime": W4A16 serves prefill row
// counts; model card "Qwen3.6-27B-W4A16": int4 weights, 16-bit activations).
#include <type_traits>

#include <algorithm>

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

// Sum over the 16 lanes of each 16-lane row of the wave (DPP: mirror inside the
// row, mirror inside each half, then the quad permutations), in every lane.
__device__ __forceinline__ float row16_sum(float v) {
  auto step = [](float x, auto ctrl) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xF, 0xF, true));
  };
  v = step(v, std::integral_constant<int, 0x140>{});   // row_mirror
  v = step(v, std::integral_constant<int, 0x141>{});   // row_half_mirror
  v = step(v, std::integral_constant<int, 0x4E>{});    // quad_perm [2,3,0,1]
  v = step(v, std::integral_constant<int, 0xB1>{});    // quad_perm [1,0,3,2]
  return v;
}

// One launch, two jobs (grid.z = problem c):
//  * blocks [0, rs_blocks): one wave per (row m < mpad, chunk of CH passes).
//    Pass i covers channels 512 i .. 512 i + 511: lane l loads 8 consecutive bf16
//    (16 bytes) at 512 i + 8 l, so the 16 lanes of row r of the wave hold group
//    4 i + r; each lane sums its 8 values in fp32 (fixed order), the row adds its 16
//    lanes, and lane 16 r writes rsq[g][m] = the negated group sum split into three
//    bf16 parts (exact) and a zero (rows >= M: zeros).  When xp is set every lane
//    also writes its 8 channels pair-arranged into xp (rows >= M: zeros).  The
//    chunk's loads are issued before its first sum.
//  * the remaining blocks: one thread per (column n < npad, block of 8 groups)
//    writes szq[g][n] = scale bits | bf16(128 + z) << 16 (0 for n >= N); the 8
//    zero points of the block are one packed word.
// Passes (512 channels each) per wave: CH = 8 (4096 channels), or CH = 2 when that
// would leave fewer than four waves per CU (few rows; see launch_gemm_prep).
template <int CH>
__global__ __launch_bounds__(256) void gemm_prep_kernel(const uint16_t* X, size_t x_stride, int M, int K, int mpad,
                                                        const uint16_t* scales, size_t sc_stride,
                                                        const uint32_t* qzeros, size_t qz_stride, int symmetric,
                                                        int N, uint16_t* rsq, size_t rsq_stride, uint32_t* szq,
                                                        size_t szq_stride, uint16_t* xp, int rs_blocks, int rs_c) {
#pragma clang fp contract(off)
  const int G = K >> 7;
  const int c = blockIdx.z;
  if ((int)blockIdx.x < rs_blocks) {
    if (c >= rs_c) return;                                // problems that share the first one's X
    const int lane = threadIdx.x & 63;
    const int passes = (K + 511) >> 9;
    const int chunks = (passes + CH - 1) / CH;
    const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int m = (int)(w / chunks);
    if (m >= mpad) return;                                // uniform per wave
    const int i0 = (int)(w % chunks) * CH;
    const uint16_t* xrow = X + (size_t)c * x_stride + (size_t)m * K;
    uint16_t* prow = xp ? xp + (size_t)c * x_stride + (size_t)m * K : nullptr;
    uint4 v[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int k = (i0 + j) * 512 + lane * 8;
      v[j] = (i0 + j < passes && k < K && m < M) ? *reinterpret_cast<const uint4*>(xrow + k)
                                                   : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int i = i0 + j;
      if (i >= passes) break;                             // uniform
      const int k = i * 512 + lane * 8;
      const uint32_t d[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
      float s = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) s += __uint_as_float(d[q] << 16) + __uint_as_float(d[q] & 0xFFFF0000u);
      if (prow && k < K) {
        uint32_t e[4];
        pair_activations(d, e);
        // non-temporal: the arranged rows are read back only by the next kernel, and
        // stores that do not stay dirty in L2 spare the write-back at the end of
        // this one (measured: 10.2 -> 7.0 us for 2048 x 2048 activations)
        const u32x4 ev = {e[0], e[1], e[2], e[3]};
        __builtin_nontemporal_store(ev, reinterpret_cast<u32x4*>(prow + k));
      }
      s = row16_sum(s);
      const int g = 4 * i + (lane >> 4);
      if ((lane & 15) == 0 && g < G) {
        uint32_t hi, mid, lo;
        split3(-s, hi, mid, lo);
        *reinterpret_cast<uint2*>(rsq + (size_t)c * rsq_stride + ((size_t)g * mpad + m) * 4) =
            make_uint2(hi | (mid << 16), lo);
      }
    }
  } else {
    const int GW = (G + 7) >> 3;
    const int npad = gemm_npad(N);
    const long long item = (long long)(blockIdx.x - rs_blocks) * 256 + threadIdx.x;
    if (item >= (long long)npad * GW) return;
    const int gw = (int)(item / npad);
    const int n = (int)(item % npad);
    uint32_t zw = 0x88888888u;                            // symmetric: z = 8 for every group
    if (!symmetric && n < N) zw = qzeros[(size_t)c * qz_stride + (size_t)n * GW + gw];
    const uint16_t* srow = scales + (size_t)c * sc_stride + (size_t)n * G;
    // all eight scale loads are issued before the first store (one memory round
    // trip per thread, not eight); a full block of 8 groups in a 16-byte aligned
    // row is one 16-byte load
    uint32_t sv[8];
    const uint16_t* sblk = srow + 8 * gw;
    if (n < N && 8 * gw + 8 <= G && (reinterpret_cast<uintptr_t>(sblk) & 15) == 0) {
      const uint4 v = *reinterpret_cast<const uint4*>(sblk);
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        sv[2 * jj] = d[jj] & 0xFFFFu;
        sv[2 * jj + 1] = d[jj] >> 16;
      }
    } else {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int g = 8 * gw + jj;
        sv[jj] = (n < N && g < G) ? (uint32_t)srow[g] : 0u;
      }
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int g = 8 * gw + jj;
      if (g < G) {
        const uint32_t v = n < N ? sv[jj] | ((0x4300u | ((zw >> (4 * jj)) & 0xFu)) << 16) : 0u;   // bf16 0x4300 | z = 128 + z
        szq[(size_t)c * szq_stride + (size_t)g * npad + n] = v;
      }
    }
  }
}

int launch_gemm_prep(const uint16_t* X, size_t x_stride, int M, int K, int mpad, const uint16_t* scales,
                     size_t sc_stride, const uint32_t* qzeros, size_t qz_stride, int symmetric, int N,
                     uint16_t* rsq, size_t rsq_stride, uint32_t* szq, size_t szq_stride, uint16_t* xp, int C,
                     hipStream_t stream, int rs_c) {
  const int GW = ((K >> 7) + 7) / 8;
  const int passes = (K + 511) >> 9;
  // short chunks when long ones would leave fewer than four waves per CU (measured on
  // the 27B shapes at M = 64: 30.6 / 29.9 -> 29.4 / 28.9 us per GEMM; at M = 2048,
  // K = 6144 the long chunks stay 0.6 us faster)
  const bool few = (long long)mpad * ((passes + 7) / 8) < 4 * 256;
  const int ch = few ? 2 : 8;
  const int chunks = (passes + ch - 1) / ch;
  const long long rs_blocks = ((long long)mpad * chunks + 3) / 4;
  const long long sz_blocks = ((long long)gemm_npad(N) * GW + 255) / 256;
  if (rs_blocks + sz_blocks == 0) return W4_OK;
  if (rs_blocks + sz_blocks > 0x7FFFFFFFLL || C > 65535) return W4_ERR_SHAPE;
  hipLaunchKernelGGL(few ? gemm_prep_kernel<2> : gemm_prep_kernel<8>, dim3((unsigned)(rs_blocks + sz_blocks), 1,
                     (unsigned)C), dim3(256), 0, stream, X, x_stride, M, K, mpad, scales, sc_stride,
                     symmetric ? nullptr : qzeros, qz_stride, symmetric, N, rsq, rsq_stride, szq, szq_stride, xp,
                     (int)rs_blocks, rs_c < 0 ? C : rs_c);
  W4_CHECK_LAUNCH();
  return W4_OK;
}


namespace {

// K split for grids too small to fill the chip: as many splits as fit the tiles x
// splits workgroups into one round of two resident workgroups on each of 256 CUs
// (at least 2 below a full round), each split at least 4 groups long.  A function
// of the shape only (the workspace size follows it).
constexpr long long kSplitSlots = kCoreSlots;

int gemm_k_splits(int M, int K, int N) {
  const long long tiles = (long long)((N + kBN - 1) / kBN) * ((M + kBM - 1) / kBM);
  const int G = K / kGroup;
  if (tiles >= kSplitSlots || G < 8) return 1;
  int s = (int)std::min<long long>(std::max<long long>(2, kSplitSlots / tiles), G / 4);
  s = std::max(s, 1);
  const int gps = (G + s - 1) / s;
  return (G + gps - 1) / gps;          // every split non-empty
}

}  // namespace

// Up to 16 rows the decode GEMV's kernels serve the GEMM too: measured on MI355X
// (graphs of launches over weight copies larger than the Infinity Cache, M = 4, 8,
// 16 on the decode-block and 27B-shaped linears), they were faster than the
// one-pass form by up to 3.6 us or equal (K = 2048, N = 12288 at M = 16: 8.6 / 8.5 us).
bool gemm_use_gemv(int M, int K, int N) { return M <= W4_GEMV_MAX_M && gemv_check_size(M, K, N) == W4_OK; }

// workspace: pair-arranged X [mpad][K] bf16 (rows >= M zero), rsq [G][mpad][4] bf16,
// szq [G][npad] u32, and with a K split the fp32 partial outputs [splits][M][N]
size_t gemm_workspace_bytes(int M, int K, int N) {
  if (M <= 0 || K <= 0 || N <= 0) return 0;
  if (gemm_use_gemv(M, K, N)) return gemv_workspace_bytes(M, K, N);
  if (gemm_use_skinny(M, K, N)) return gemm_skinny_workspace_bytes(M, K, N);
  const size_t mpad = align_up((size_t)M, kBM);
  const size_t G = (size_t)(K / kGroup);
  const int splits = gemm_k_splits(M, K, N);
  return align_up(mpad * K * 2, 256) + align_up(G * mpad * 8, 256) + align_up(G * gemm_npad(N) * 4, 256) +
         (splits > 1 ? (size_t)splits * align_up((size_t)M * N, 64) * 4 : 0);
}

// 32-bit per-lane byte offsets in the core: the arranged activations (2 x (M + 64) x K
// bytes) and the packed weights (N K / 2 bytes) below 2^32.
int gemm_check_size(int M, int K, int N) {
  if (((long long)M + kBM) * K >= (1LL << 31) || (long long)N * K >= (1LL << 33)) return W4_ERR_SHAPE;
  return W4_OK;
}

int launch_gemm(const uint16_t* X, int M, int K, int N, const uint32_t* qweight,
                const uint16_t* scales, const uint32_t* qzeros, int symmetric, uint16_t* Y,
                void* workspace, hipStream_t stream) {
  if (M == 0 || N == 0) return W4_OK;
  if (int st = gemm_check_size(M, K, N)) return st;
  if (gemm_use_gemv(M, K, N)) return launch_gemv(X, M, K, N, qweight, scales, qzeros, symmetric, Y, workspace, stream);
  if (gemm_use_skinny(M, K, N))
    return launch_gemm_skinny(X, M, K, N, qweight, scales, qzeros, symmetric, Y, workspace, stream);
  const int mpad = (int)align_up((size_t)M, kBM);
  const int G = K / kGroup;
  const int splits = gemm_k_splits(M, K, N);
  char* ws = static_cast<char*>(workspace);
  uint16_t* xp = reinterpret_cast<uint16_t*>(ws);
  ws += align_up((size_t)mpad * K * 2, 256);
  uint16_t* rsq = reinterpret_cast<uint16_t*>(ws);
  ws += align_up((size_t)G * mpad * 8, 256);
  uint32_t* szq = reinterpret_cast<uint32_t*>(ws);
  ws += align_up((size_t)G * gemm_npad(N) * 4, 256);
  float* ypart = splits > 1 ? reinterpret_cast<float*>(ws) : nullptr;
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
  a.ypart = ypart;
  a.ypart_stride = align_up((size_t)M * N, 64);
  a.gsplit = splits > 1 ? (G + splits - 1) / splits : 0;
  const long long tiles = (long long)((N + kBN - 1) / kBN) * ((M + kBM - 1) / kBM);
  if (tiles > 0x7FFFFFFFLL) return W4_ERR_SHAPE;
  const dim3 grid((unsigned)tiles, (unsigned)splits, 1);
  if (gemm_core_wide(tiles * splits))
    hipLaunchKernelGGL((gemm_core_kernel<EPI_STORE, true>), grid, dim3(kGemmWaves * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_core_kernel<EPI_STORE>), grid, dim3(kGemmWaves * 64), 0, stream, a);
  W4_CHECK_LAUNCH();
  if (splits > 1) return launch_split_reduce(ypart, splits, a.ypart_stride, (size_t)M * N, Y, stream);
  return W4_OK;
}

}  // namespace w4
