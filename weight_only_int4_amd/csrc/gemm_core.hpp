// MFMA core of the W4A16 prefill contraction, shared by w4a16_gemm and the AWQ
// grid loss.  Y = X W_hat^T with X bf16 [M][K] and W_hat given either as packed
// int4 groups (q - z) * sc or, for the unquantized reference, as bf16 [N][K].
//
// Workgroup tile 128 x 128, 4 waves in a 2 x 2 grid, wave tile 64 x 64 made of
// 2 x 2 v_mfma_f32_32x32x16_bf16 blocks.  One main-loop step covers one
// 128-channel quantization group:
//   * the activation tile (128 rows x 128 channels bf16, 32 KB) goes from global
//     memory straight into LDS (global_load_lds_dwordx4, no registers), double
//     buffered; inside a 256-byte row the 16-byte chunk c is stored at position
//     c ^ (row & 15), which makes the fragment reads bank-conflict free;
//   * for int4 weights the activations arrive pre-arranged: every 8-channel run
//     holds the pairs (x0,x4)(x1,x5)(x2,x6)(x3,x7), the order in which one packed
//     word expands (written so by the prologue kernel);
//   * each lane's weight operand for one MFMA is exactly one packed uint32 word
//     (8 consecutive channels of its output column), read straight from global
//     memory one group ahead and expanded in registers to bf16 integers 128 + q;
//   * the 8 MFMAs of a group accumulate exact integer-weight products
//     sum_k x (128 + q) into a per-group fp32 tile, folded into the output
//     accumulator with one FMA: acc += sc * tmp;
//   * the zero-point term -sum_g rowsum_g(X)[m] * sc[n,g] (128 + z[n,g]) is a
//     small contraction over groups, also done on the MFMA: the prologue kernel
//     writes rowsum_g(X) as three bf16 parts (hi + mid + lo, exact) and
//     -sc (128 + z) as two (exact: it has at most 16 significant bits) into
//     16-slot rows, 5 products per group, 3 groups per K=16 step; one such step
//     per three groups accumulates straight into acc.
// The k-slots of the MFMA are assigned so that lane half h, step j covers
// channels 64h + 8j .. 64h + 8j + 7 of the group: each lane's 8 words of a group
// are contiguous (two 16-byte loads).
#pragma once

#include "internal.hpp"

namespace w4 {

constexpr int kBM = 128;
constexpr int kBN = 128;

enum { EPI_STORE = 0, EPI_SQDIFF = 1 };

struct GemmCoreArgs {
  const uint16_t* X;       // [M][K] bf16 (+ z * x_stride); pair-arranged for int4 weights
  size_t x_stride;
  int M, K, N;
  // int4 weights
  const uint32_t* qweight; // [N][K/8] (+ z * qw_stride)
  size_t qw_stride;
  const uint16_t* scales;  // [N][K/128]
  size_t sc_stride;
  const uint16_t* rsx;     // [mpad][kz] bf16 split group row sums of X (+ z * rsx_stride)
  size_t rsx_stride;
  const uint16_t* cz;      // [N][kz] bf16 split -sc (128 + z) (+ z * cz_stride)
  size_t cz_stride;
  int kz;                  // 16 * ceil(G / 3)
  // bf16 weights (reference path)
  const uint16_t* W;       // [N][K]
  // epilogue
  uint16_t* Y;             // EPI_STORE: [M][N] bf16
  const uint16_t* Yref;    // EPI_SQDIFF: [M][N] bf16
  float* partials;         // EPI_SQDIFF: [z][tiles]
};

// Workgroup -> output tile.  Workgroups are dispatched round-robin over the 8
// XCDs (workgroup L runs on XCD L mod 8) and each XCD has its own L2, so
// consecutive slots of one XCD get a contiguous range of the tile order; that
// order walks 8-tile-tall bands of M column by column, so the workgroups
// resident on an XCD at one time share A rows and B columns in its L2.
__device__ __forceinline__ void tile_coords(int L, int MT, int NT, int& tm, int& tn) {
  const int T = MT * NT;
  constexpr int kXcd = 8, kBand = 8;
  int t = L;
  if (T % kXcd == 0) t = (L % kXcd) * (T / kXcd) + L / kXcd;
  const int band_tiles = kBand * NT;
  const int band = t / band_tiles;
  const int rows = min(kBand, MT - band * kBand);
  const int r = t - band * band_tiles;
  tm = band * kBand + r % rows;
  tn = r / rows;
}

// Per-group weight operand of one lane: INT4 -> its 8 packed words of the group
// for each of its two 32-column blocks (2 x uint4) plus the raw bf16 scale bits
// (converted when used, so no wait is needed right after the prefetch);
// bf16 -> its 64 channels of the group for each block (8 x uint4).
template <bool INT4>
struct BStage {
  static constexpr int REGS = INT4 ? 2 : 8;
  uint4 w[2][REGS];
  uint32_t scb[2];
};

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum).
#define W4_WAIT_VMCNT0() __builtin_amdgcn_s_waitcnt(0x0F70)

template <bool INT4, int EPI>
__global__ __launch_bounds__(256, 2) void gemm_core_kernel(GemmCoreArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t sA0[kBM * 128];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[kBM * 128];
  __shared__ float sRed[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, l32 = lane & 31;
  int tm, tn;
  tile_coords(blockIdx.x, (a.M + kBM - 1) / kBM, (a.N + kBN - 1) / kBN, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int zc_idx = blockIdx.z;
  const int G = a.K >> 7;
  const int words = a.K >> 3;
  const int T3 = (G + 2) / 3;

  // activation DMA: instruction i of wave w fills LDS rows 4 (8 w + i) .. +3;
  // lane -> row 4 (8 w + i) + lane / 16, LDS chunk lane % 16, which holds the
  // row's logical chunk (lane % 16) ^ (row & 15).  Rows past M read row M-1
  // (always valid): their finite results are never stored or scored.
  const uint16_t* X = a.X + (size_t)zc_idx * a.x_stride;
  const int dchunk = lane & 15;
  uint32_t doff[8];          // element offset of this lane's source chunk, without the group term
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 4 * (8 * wave + i) + (lane >> 4);
    const int grow = min(m0 + row, a.M - 1);
    doff[i] = (uint32_t)grow * (uint32_t)a.K + (uint32_t)((dchunk ^ (row & 15)) * 8);
  }
  auto load_a = [&](int g, uint16_t* sbuf) {
    const uint16_t* src = X + (size_t)g * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_global_load_lds(src + doff[i], sbuf + (8 * wave + i) * 512, 16, 0, 0);
  };

  // weight rows of this lane (clamped to N-1; columns past N get scale 0 and are not stored)
  int ncol[2], nrow[2];
  bool nok[2];
#pragma unroll
  for (int bn = 0; bn < 2; ++bn) {
    ncol[bn] = n0 + wn * 64 + bn * 32 + l32;
    nok[bn] = ncol[bn] < a.N;
    nrow[bn] = min(ncol[bn], a.N - 1);
  }
  const uint32_t* qw = nullptr;
  const uint16_t* scl = nullptr;
  const uint16_t* rsx = nullptr;
  const uint16_t* czp = nullptr;
  if constexpr (INT4) {
    qw = a.qweight + (size_t)zc_idx * a.qw_stride;
    scl = a.scales + (size_t)zc_idx * a.sc_stride;
    rsx = a.rsx + (size_t)zc_idx * a.rsx_stride + (size_t)(m0 + wm * 64 + l32) * a.kz + h * 8;
    czp = a.cz + (size_t)zc_idx * a.cz_stride + h * 8;
  }

  auto load_b = [&](int g, BStage<INT4>& B) {
#pragma unroll
    for (int bn = 0; bn < 2; ++bn) {
      if constexpr (INT4) {
        const uint4* p = reinterpret_cast<const uint4*>(qw + (size_t)nrow[bn] * words + g * 16 + h * 8);
        B.w[bn][0] = p[0];
        B.w[bn][1] = p[1];
        B.scb[bn] = scl[(size_t)nrow[bn] * G + g];
      } else {
        const uint4* p = reinterpret_cast<const uint4*>(a.W + (size_t)nrow[bn] * a.K + (size_t)g * kGroup + h * 64);
#pragma unroll
        for (int i = 0; i < 8; ++i) B.w[bn][i] = p[i];
      }
    }
  };

  // fragment reads: row wm*64 + bm*32 + l32, logical chunk 8h + j at LDS chunk
  // (8h + j) ^ (row & 15); row & 15 = l32 & 15
  const int sw = l32 & 15;
  const int frag_row = (wm * 64 + l32) * 128;
  auto frag = [&](const uint16_t* sbuf, int bm, int j) {
    return *reinterpret_cast<const bf16x8*>(sbuf + frag_row + bm * 32 * 128 + (((8 * h + j) ^ sw) * 8));
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int bm = 0; bm < 2; ++bm)
#pragma unroll
    for (int bn = 0; bn < 2; ++bn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bm][bn][r] = 0.0f;

  const uint32_t nib_mask = opaque_vgpr(0x000F000Fu);
  auto compute = [&](const uint16_t* sbuf, const BStage<INT4>& B) {
    if constexpr (INT4) {
      f32x16 tmp[2][2];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bf16x8 af[2], bf[2];
#pragma unroll
        for (int bm = 0; bm < 2; ++bm) af[bm] = frag(sbuf, bm, j);
#pragma unroll
        for (int bn = 0; bn < 2; ++bn) {
          const uint4 wv = B.w[bn][j >> 2];
          const uint32_t word = (j & 3) == 0 ? wv.x : (j & 3) == 1 ? wv.y : (j & 3) == 2 ? wv.z : wv.w;
          const uint4 pr = make_uint4(nibble_pair_m(word, 0, nib_mask), nibble_pair_m(word, 1, nib_mask),
                                      nibble_pair_m(word, 2, nib_mask), nibble_pair_m(word, 3, nib_mask));
          bf[bn] = __builtin_bit_cast(bf16x8, pr);
        }
#pragma unroll
        for (int bm = 0; bm < 2; ++bm)
#pragma unroll
          for (int bn = 0; bn < 2; ++bn) {
            if (j == 0)
              tmp[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[bm], bf[bn], f32x16{}, 0, 0, 0);
            else
              tmp[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[bm], bf[bn], tmp[bm][bn], 0, 0, 0);
          }
      }
      // fold: acc += sc * tmp (the zero-point term is accumulated separately);
      // columns past N get scale 0
      float sc[2];
#pragma unroll
      for (int bn = 0; bn < 2; ++bn) sc[bn] = nok[bn] ? bf16_bits_to_f32(B.scb[bn]) : 0.0f;
#pragma unroll
      for (int bm = 0; bm < 2; ++bm)
#pragma unroll
        for (int bn = 0; bn < 2; ++bn)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[bm][bn][r] = fmaf(sc[bn], tmp[bm][bn][r], acc[bm][bn][r]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bf16x8 af[2], bf[2];
#pragma unroll
        for (int bm = 0; bm < 2; ++bm) af[bm] = frag(sbuf, bm, j);
#pragma unroll
        for (int bn = 0; bn < 2; ++bn) bf[bn] = __builtin_bit_cast(bf16x8, B.w[bn][j]);
#pragma unroll
        for (int bm = 0; bm < 2; ++bm)
#pragma unroll
          for (int bn = 0; bn < 2; ++bn)
            acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[bm], bf[bn], acc[bm][bn], 0, 0, 0);
      }
    }
  };

  // zero-point step t (t < ceil(G/3)): operands loaded before the step's group is
  // computed, the 4 MFMAs issued after it
  auto zload = [&](int t, uint4 (&za)[2], uint4 (&zb)[2]) {
#pragma unroll
    for (int bm = 0; bm < 2; ++bm) za[bm] = *reinterpret_cast<const uint4*>(rsx + (size_t)bm * 32 * a.kz + t * 16);
#pragma unroll
    for (int bn = 0; bn < 2; ++bn) zb[bn] = *reinterpret_cast<const uint4*>(czp + (size_t)nrow[bn] * a.kz + t * 16);
  };
  auto zmfma = [&](const uint4 (&za)[2], const uint4 (&zb)[2]) {
#pragma unroll
    for (int bm = 0; bm < 2; ++bm)
#pragma unroll
      for (int bn = 0; bn < 2; ++bn)
        acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, za[bm]),
                                                               __builtin_bit_cast(bf16x8, zb[bn]), acc[bm][bn], 0, 0, 0);
  };

  // one pipeline step: prefetch group g+1 (activations into `nbuf`, weights into
  // Bn), compute group g from `cbuf` and Bc, wait for the prefetch, barrier
  auto step = [&](int g, const uint16_t* cbuf, uint16_t* nbuf, const BStage<INT4>& Bc, BStage<INT4>& Bn) {
    uint4 za[2], zb[2];
    const bool zstep = INT4 && g < T3;
    if constexpr (INT4) {
      if (zstep) zload(g, za, zb);
    }
    if (g + 1 < G) {
      load_a(g + 1, nbuf);
      load_b(g + 1, Bn);
    }
    compute(cbuf, Bc);
    if constexpr (INT4) {
      if (zstep) zmfma(za, zb);
    }
    W4_WAIT_VMCNT0();
    __syncthreads();
  };

  BStage<INT4> B0, B1;
  load_a(0, sA0);
  load_b(0, B0);
  W4_WAIT_VMCNT0();
  __syncthreads();
  for (int g = 0; g < G; g += 2) {
    step(g, sA0, sA1, B0, B1);
    if (g + 1 >= G) break;
    step(g + 1, sA1, sA0, B1, B0);
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
      a.partials[(size_t)zc_idx * gridDim.x + blockIdx.x] = tot;
    }
  }
}

// Operands of the zero-point contraction (defined in gemm.hip), for C problems:
//   rsx[c][m][16t + s] (m < mpad; rows >= M are 0): group row sums of X[c] split
//   into bf16 parts, cz[c][n][16t + s]: -sc (128 + z) split into bf16 parts, with
//   slot s = 5j + u for group 3t + j: rs parts (hi, hi, mid, mid, lo) against
//   c parts (hi, lo, hi, lo, hi); slot 15 and slots of groups >= G are 0.
// When xp is not NULL it also writes X[c] pair-arranged (every 8-channel run as
// (x0,x4)(x1,x5)(x2,x6)(x3,x7)) into xp[c] ([M][K], same strides as X).
inline int zterm_kz(int K) { return 16 * (((K >> 7) + 2) / 3); }
int launch_zterm_prep(const uint16_t* X, size_t x_stride, int M, int K, int mpad, const uint16_t* scales,
                      size_t sc_stride, const uint32_t* qzeros, size_t qz_stride, int symmetric, int N,
                      uint16_t* rsx, size_t rsx_stride, uint16_t* cz, size_t cz_stride, uint16_t* xp, int C,
                      hipStream_t stream);

}  // namespace w4
