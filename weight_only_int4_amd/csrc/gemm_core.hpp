// MFMA core of the W4A16 prefill contraction, shared by w4a16_gemm and the AWQ
// grid loss.  Y = X W_hat^T with X bf16 [M][K] and W_hat given either as packed
// int4 groups (q - z) * sc or, for the unquantized reference, as bf16 [N][K].
//
// Workgroup tile 128 x 128, 4 waves in a 2 x 2 grid, wave tile 64 x 64 made of
// 2 x 2 v_mfma_f32_32x32x16_bf16 blocks.  One main-loop step covers one
// 128-channel quantization group:
//   * the activation tile (128 rows x 128 channels bf16) is staged in LDS,
//     double buffered, with a 16-byte pad per row (conflict-free 16-byte reads);
//     for int4 weights each 8-channel run is stored as the pairs
//     (x0,x4)(x1,x5)(x2,x6)(x3,x7) so it lines up with the packed nibbles;
//   * each lane's weight operand for one MFMA is exactly one packed uint32 word
//     (8 consecutive channels of its output column), read straight from global
//     memory one group ahead and expanded in registers to bf16 integers 128 + q;
//   * the 8 MFMAs of a group accumulate exact integer-weight products into a
//     per-group fp32 tile, which is folded into the output accumulator with the
//     group's scale and zero point:
//       acc += sc * (tmp - (128 + z) * rowsum_g(X))
//     rowsum_g(X) (fp32, per row and group) comes from a prologue kernel.
// The k-slots of the MFMA are assigned so that lane half h, step j covers
// channels 64h + 8j .. 64h + 8j + 7 of the group: each lane's 8 words of a group
// are contiguous (two 16-byte loads).
#pragma once

#include "internal.hpp"

namespace w4 {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kLDA = 136;  // bf16 per LDS activation row (128 + 8 pad)

enum { EPI_STORE = 0, EPI_SQDIFF = 1 };

struct GemmCoreArgs {
  const uint16_t* X;       // [M][K] bf16 (+ z * x_stride)
  size_t x_stride;
  int M, K, N;
  // int4 weights
  const uint32_t* qweight; // [N][K/8] (+ z * qw_stride)
  size_t qw_stride;
  const uint16_t* scales;  // [N][K/128]
  size_t sc_stride;
  const uint32_t* qzeros;  // [N][ceil(K/1024)] or NULL (symmetric)
  size_t qz_stride;
  int symmetric;
  const float* rs;         // [G][mpad] group row sums of X (+ z * rs_stride)
  size_t rs_stride;
  int mpad;
  // bf16 weights (reference path)
  const uint16_t* W;       // [N][K]
  // epilogue
  uint16_t* Y;             // EPI_STORE: [M][N] bf16
  const uint16_t* Yref;    // EPI_SQDIFF: [M][N] bf16
  float* partials;         // EPI_SQDIFF: [z][tiles]
};

template <bool INT4, int EPI>
__global__ __launch_bounds__(256, 2) void gemm_core_kernel(GemmCoreArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kBM * kLDA];
  __shared__ __attribute__((aligned(16))) float sRS[2][kBM];
  __shared__ float sRed[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, l32 = lane & 31;
  const int m0 = blockIdx.y * kBM, n0 = blockIdx.x * kBN;
  const int zc_idx = blockIdx.z;
  const int G = a.K >> 7;
  const int GW = (G + 7) >> 3;
  const int words = a.K >> 3;

  const uint16_t* X = a.X + (size_t)zc_idx * a.x_stride;

  // activation staging: thread -> (row ar, 64-channel half ah)
  const int ar = tid >> 1, ah = tid & 1;
  const bool arow_ok = (m0 + ar) < a.M;
  const uint16_t* aptr = X + (size_t)(arow_ok ? m0 + ar : 0) * a.K + ah * 64;

  // weight rows of this lane
  int ncol[2];
  bool nok[2];
#pragma unroll
  for (int bn = 0; bn < 2; ++bn) {
    ncol[bn] = n0 + wn * 64 + bn * 32 + l32;
    nok[bn] = ncol[bn] < a.N;
  }

  const uint32_t* qw = nullptr;
  const uint16_t* scl = nullptr;
  const uint32_t* qz = nullptr;
  const float* rs = nullptr;
  if constexpr (INT4) {
    qw = a.qweight + (size_t)zc_idx * a.qw_stride;
    scl = a.scales + (size_t)zc_idx * a.sc_stride;
    qz = a.qzeros ? a.qzeros + (size_t)zc_idx * a.qz_stride : nullptr;
    rs = a.rs + (size_t)zc_idx * a.rs_stride;
  }

  uint4 areg[8];
  float4 rsreg = make_float4(0.f, 0.f, 0.f, 0.f);

  auto load_a = [&](int g) {
#pragma unroll
    for (int i = 0; i < 8; ++i) areg[i] = make_uint4(0u, 0u, 0u, 0u);
    if (arow_ok) {
      const uint4* p = reinterpret_cast<const uint4*>(aptr + (size_t)g * kGroup);
#pragma unroll
      for (int i = 0; i < 8; ++i) areg[i] = p[i];
    }
    if constexpr (INT4) {
      if (tid < kBM / 4) rsreg = *reinterpret_cast<const float4*>(rs + (size_t)g * a.mpad + m0 + tid * 4);
    }
  };
  auto store_a = [&](int buf) {
    uint16_t* dst = &sA[buf][ar * kLDA + ah * 64];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint4 v = areg[i];
      if constexpr (INT4) {
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
        uint32_t e[4];
        pair_activations(d, e);
        v = make_uint4(e[0], e[1], e[2], e[3]);
      }
      *reinterpret_cast<uint4*>(dst + i * 8) = v;
    }
    if constexpr (INT4) {
      if (tid < kBM / 4) *reinterpret_cast<float4*>(&sRS[buf][tid * 4]) = rsreg;
    }
  };

  // weight operand registers: INT4 -> 8 words per column block (2 x uint4);
  // bf16 -> 64 channels per column block (8 x uint4)
  constexpr int BREGS = INT4 ? 2 : 8;
  uint4 bcur[2][BREGS], bnext[2][BREGS];
  float sc_cur[2] = {0.f, 0.f}, zf_cur[2] = {0.f, 0.f};
  float sc_next[2] = {0.f, 0.f}, zf_next[2] = {0.f, 0.f};
  const uint32_t zsym = a.symmetric ? 136u : 128u;

  auto load_b = [&](int g, uint4 (&b)[2][BREGS], float (&sc)[2], float (&zf)[2]) {
#pragma unroll
    for (int bn = 0; bn < 2; ++bn) {
#pragma unroll
      for (int i = 0; i < BREGS; ++i) b[bn][i] = make_uint4(0u, 0u, 0u, 0u);
      sc[bn] = 0.f;
      zf[bn] = 0.f;
      if (nok[bn]) {
        if constexpr (INT4) {
          const uint4* p = reinterpret_cast<const uint4*>(qw + (size_t)ncol[bn] * words + g * 16 + h * 8);
          b[bn][0] = p[0];
          b[bn][1] = p[1];
          sc[bn] = bf16_bits_to_f32(scl[(size_t)ncol[bn] * G + g]);
          uint32_t z = zsym;
          if (qz) z = 128u + ((qz[(size_t)ncol[bn] * GW + (g >> 3)] >> (4 * (g & 7))) & 0xFu);
          zf[bn] = (float)z;
        } else {
          const uint4* p = reinterpret_cast<const uint4*>(a.W + (size_t)ncol[bn] * a.K + (size_t)g * kGroup + h * 64);
#pragma unroll
          for (int i = 0; i < 8; ++i) b[bn][i] = p[i];
        }
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int bm = 0; bm < 2; ++bm)
#pragma unroll
    for (int bn = 0; bn < 2; ++bn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bm][bn][r] = 0.0f;
  const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf, const uint4 (&b)[2][BREGS], const float (&sc)[2], const float (&zf)[2]) {
    const uint16_t* abase = &sA[buf][(wm * 64 + l32) * kLDA + h * 64];
    if constexpr (INT4) {
      f32x16 tmp[2][2];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bf16x8 af[2], bf[2];
#pragma unroll
        for (int bm = 0; bm < 2; ++bm)
          af[bm] = *reinterpret_cast<const bf16x8*>(abase + bm * 32 * kLDA + j * 8);
#pragma unroll
        for (int bn = 0; bn < 2; ++bn) {
          const uint4 wv = b[bn][j >> 2];
          const uint32_t word = (j & 3) == 0 ? wv.x : (j & 3) == 1 ? wv.y : (j & 3) == 2 ? wv.z : wv.w;
          const uint4 pr = make_uint4(nibble_pair(word, 0), nibble_pair(word, 1), nibble_pair(word, 2),
                                      nibble_pair(word, 3));
          bf[bn] = __builtin_bit_cast(bf16x8, pr);
        }
#pragma unroll
        for (int bm = 0; bm < 2; ++bm)
#pragma unroll
          for (int bn = 0; bn < 2; ++bn)
            tmp[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[bm], bf[bn], j == 0 ? zero16 : tmp[bm][bn], 0, 0, 0);
      }
      // fold: acc += sc * (tmp - (128 + z) * rowsum)
#pragma unroll
      for (int bm = 0; bm < 2; ++bm) {
        float rsv[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 f = *reinterpret_cast<const float4*>(&sRS[buf][wm * 64 + bm * 32 + 8 * i + 4 * h]);
          rsv[4 * i + 0] = f.x;
          rsv[4 * i + 1] = f.y;
          rsv[4 * i + 2] = f.z;
          rsv[4 * i + 3] = f.w;
        }
#pragma unroll
        for (int bn = 0; bn < 2; ++bn)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            acc[bm][bn][r] = fmaf(sc[bn], fmaf(-zf[bn], rsv[r], tmp[bm][bn][r]), acc[bm][bn][r]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bf16x8 af[2], bf[2];
#pragma unroll
        for (int bm = 0; bm < 2; ++bm)
          af[bm] = *reinterpret_cast<const bf16x8*>(abase + bm * 32 * kLDA + j * 8);
#pragma unroll
        for (int bn = 0; bn < 2; ++bn) bf[bn] = __builtin_bit_cast(bf16x8, b[bn][j]);
#pragma unroll
        for (int bm = 0; bm < 2; ++bm)
#pragma unroll
          for (int bn = 0; bn < 2; ++bn)
            acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[bm], bf[bn], acc[bm][bn], 0, 0, 0);
      }
    }
  };

  // software pipeline: global loads of group g+1 are in flight during group g
  load_a(0);
  load_b(0, bcur, sc_cur, zf_cur);
  store_a(0);
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    const bool more = g + 1 < G;
    if (more) {
      load_a(g + 1);
      load_b(g + 1, bnext, sc_next, zf_next);
    }
    compute(buf, bcur, sc_cur, zf_cur);
    if (more) store_a(buf ^ 1);
    __syncthreads();
#pragma unroll
    for (int bn = 0; bn < 2; ++bn) {
#pragma unroll
      for (int i = 0; i < BREGS; ++i) bcur[bn][i] = bnext[bn][i];
      sc_cur[bn] = sc_next[bn];
      zf_cur[bn] = zf_next[bn];
    }
  }

  // epilogue.  Output layout of a 32x32 block: lane holds column l32 and rows
  // 8*i + 4*h + j for register 4*i + j.
  if constexpr (EPI == EPI_STORE) {
#pragma unroll
    for (int bm = 0; bm < 2; ++bm)
#pragma unroll
      for (int bn = 0; bn < 2; ++bn) {
        if (!nok[bn]) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * 64 + bm * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (row < a.M) a.Y[(size_t)row * a.N + ncol[bn]] = (uint16_t)f32_to_bf16_bits(acc[bm][bn][r]);
        }
      }
  } else {
    const uint16_t* Yref = a.Yref;
    float s = 0.0f;
#pragma unroll
    for (int bm = 0; bm < 2; ++bm)
#pragma unroll
      for (int bn = 0; bn < 2; ++bn) {
        if (!nok[bn]) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * 64 + bm * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (row < a.M) {
            const float d = acc[bm][bn][r] - bf16_bits_to_f32(Yref[(size_t)row * a.N + ncol[bn]]);
            s = fmaf(d, d, s);
          }
        }
      }
    s = wave_sum(s);
    if (lane == 0) sRed[wave] = s;
    __syncthreads();
    if (tid == 0) {
      const float tot = (sRed[0] + sRed[1]) + (sRed[2] + sRed[3]);
      const size_t tiles = (size_t)gridDim.x * gridDim.y;
      a.partials[(size_t)zc_idx * tiles + (size_t)blockIdx.y * gridDim.x + blockIdx.x] = tot;
    }
  }
}

// rs[z][g][m] = fp32 sum of X[z][m][128 g .. 128 g + 127] (fixed order); rows
// M .. mpad-1 are written as 0.  Defined in gemm.hip.
int launch_group_rowsum(const uint16_t* X, size_t x_stride, int M, int K, int mpad, float* rs,
                        size_t rs_stride, int C, hipStream_t stream);

}  // namespace w4
