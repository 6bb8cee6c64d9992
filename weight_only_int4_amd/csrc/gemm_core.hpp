// MFMA core of the W4A16 prefill contraction, shared by w4a16_gemm and the AWQ
// grid loss.  Y = X W_hat^T with X bf16 [M][K] and W_hat given either as packed
// int4 groups (q - z) * sc or, for the unquantized reference, as bf16 [N][K].
//
// Workgroup tile 128 x 128, 4 waves in a 2 x 2 grid, wave tile 64 x 64 made of
// 2 x 2 v_mfma_f32_32x32x16_bf16 blocks.  One main-loop step covers one
// 128-channel quantization group.
//
// Every operand of a group travels from global memory straight into LDS
// (global_load_lds: no registers), STAGES groups deep.  These copies are issued
// from inline assembly, so the compiler's wait-counter bookkeeping does not see
// them: it would otherwise wait for every copy in flight, including those of
// later groups, before each LDS read.  The kernel waits for exactly the copies of
// the group it is about to use (vmcnt counts one wave's copies, which complete in
// issue order), then synchronises the workgroup with a bare s_barrier.
//
// Per stage (int4 weights):
//   * activations: 128 rows x 128 channels bf16 (32 KB); inside a 256-byte row
//     the 16-byte chunk c is stored at position c ^ (row & 15).  They arrive
//     pre-arranged: every 8-channel run holds the pairs (x0,x4)(x1,x5)(x2,x6)
//     (x3,x7), the order in which one packed word expands (written so by the
//     prologue kernel);
//   * packed words: 128 columns x 16 words (8 KB); inside a column's 64 bytes the
//     16-byte chunk c is stored at position c ^ ((col >> 2) & 3);
//   * zero-point operands of one K=16 step (8 KB, see below);
//   * scales of the group: 128 bf16, one copy per wave (the prologue writes them
//     group-major, zero past N).
// Each lane's weight operand for one MFMA is one packed uint32 word (8
// consecutive channels of its output column), expanded in registers to bf16
// integers 128 + q.  The 8 MFMAs of a group accumulate exact integer-weight
// products sum_k x (128 + q) into a per-group fp32 tile, folded into the output
// accumulator with one FMA: acc += sc * tmp.  The zero-point term
// -sum_g rowsum_g(X)[m] * sc[n,g] (128 + z[n,g]) is a small contraction over
// groups, also done on the MFMA: the prologue writes rowsum_g(X) as three bf16
// parts (hi + mid + lo, exact) and -sc (128 + z) as two (exact: it has at most
// 16 significant bits) into 16-slot rows, 5 products per group, 3 groups per
// K=16 step; one such step per three groups accumulates straight into acc.
// The k-slots of the MFMA are assigned so that lane half h, step j covers
// channels 64h + 8j .. 64h + 8j + 7 of the group: each lane's 8 words of a group
// are contiguous.
#pragma once

#include <type_traits>

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
  const uint16_t* sct;     // [K/128][npad] bf16 scales, group-major, 0 for columns >= N (+ z * sct_stride)
  size_t sct_stride;
  int npad;                // N rounded up to 128
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

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Global -> LDS copies: lane l writes 16 (or 4) bytes at LDS byte address
// m0 + 16 l (4 l).  M0 is set by the compiler from the "{m0}" operand; the
// s_nop covers the one wait state the hardware needs between an M0 write and an
// LDS copy.  The source address is a per-lane 64-bit VGPR pair.
__device__ __forceinline__ void lds_copy16(const void* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_copy4(const void* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

// Workgroup barrier without a memory fence.  LDS reads are complete (lgkmcnt);
// global->LDS copies are covered by the explicit vmcnt waits before it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS byte layout of one pipeline stage.
template <bool INT4>
struct GemmSmem {
  static constexpr int kA = 0;                                   // activations, 32 KB
  static constexpr int kB = kBM * 256;                           // int4: packed words 8 KB; bf16: weights 32 KB
  static constexpr int kZ = kB + (INT4 ? kBN * 64 : kBN * 256);  // int4: zero-point operands 8 KB
  static constexpr int kS = kZ + (INT4 ? 8192 : 0);              // int4: scales, 4 waves x 256 B
  static constexpr int kStage = kS + (INT4 ? 1024 : 0);
  static constexpr int kStages = INT4 ? 3 : 2;
  // copies issued per stage and wave: activations 8 (+ int4: words 2, zero-point 2,
  // scales 1; bf16: weights 8)
  static constexpr int kCopies = INT4 ? 13 : 16;
  static_assert(kStage * kStages <= 160 * 1024, "LDS");
};

template <bool INT4, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_core_kernel(GemmCoreArgs a) {
  using SM = GemmSmem<INT4>;
  constexpr int S = SM::kStages;
  constexpr int D = S - 1;                 // prefetch distance in groups
  constexpr int L = SM::kCopies;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[S * SM::kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, l32 = lane & 31;
  int tm, tn;
  tile_coords(blockIdx.x, (a.M + kBM - 1) / kBM, (a.N + kBN - 1) / kBN, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int zc_idx = blockIdx.z;
  const int G = a.K >> 7;
  const int T3 = (G + 2) / 3;
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;   // LDS byte address (low half of the generic one)

  // ---- copy sources, per lane, without the group term ----
  // activations: copy i of wave w fills rows 4 (8 w + i) .. +3; lane -> row
  // 4 (8 w + i) + lane / 16, stored chunk lane % 16, which holds logical chunk
  // (lane % 16) ^ (row & 15).  Rows past M read row M-1 (always valid): their
  // finite results are never stored or scored.
  const uint16_t* X = a.X + (size_t)zc_idx * a.x_stride;
  const uint16_t* asrc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 4 * (8 * wave + i) + (lane >> 4);
    const int grow = min(m0 + row, a.M - 1);
    asrc[i] = X + (size_t)grow * a.K + (((lane & 15) ^ (row & 15)) * 8);
  }
  // weights.  int4: copy i (of 8, wave w issues 2w, 2w+1) fills LDS chunks 64 i + lane:
  // column (64 i + lane) / 4, stored chunk lane % 4, logical chunk (lane % 4) ^ ((col >> 2) & 3).
  // (LDS serves a 16-byte read 16 lanes at a time over 64 banks: 16 consecutive
  // columns then hit 16 distinct 16-byte bank groups.)
  // bf16: like the activations, rows = columns n.  Columns past N read column N-1.
  const unsigned char* wsrc[INT4 ? 2 : 8];
  if constexpr (INT4) {
    const uint32_t* qw = a.qweight + (size_t)zc_idx * a.qw_stride;
    const int words = a.K >> 3;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int p = 64 * (2 * wave + u) + lane;
      const int col = p >> 2;
      const int chunk = (p & 3) ^ ((col >> 2) & 3);
      wsrc[u] = reinterpret_cast<const unsigned char*>(qw + (size_t)min(n0 + col, a.N - 1) * words + chunk * 4);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 4 * (8 * wave + i) + (lane >> 4);
      wsrc[i] = reinterpret_cast<const unsigned char*>(a.W + (size_t)min(n0 + row, a.N - 1) * a.K +
                                                       (((lane & 15) ^ (row & 15)) * 8));
    }
  }
  // zero-point operands: copy i (of 8, wave w issues 2w, 2w+1) fills Z bytes
  // 1024 i + 16 lane; i < 4: row parts of tile rows 32 i .. +31, i >= 4: column
  // parts of tile columns 32 (i-4) .. +31; lane -> entry 32 (i % 4) + lane / 2,
  // stored half lane % 2 holding logical half (lane % 2) ^ ((entry >> 3) & 1)
  const uint16_t* zsrc[2] = {nullptr, nullptr};
  const uint16_t* ssrc = nullptr;
  if constexpr (INT4) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = 2 * wave + u;
      const int e = 32 * (i & 3) + (lane >> 1);
      const int half = (lane & 1) ^ ((e >> 3) & 1);
      if (i < 4)
        zsrc[u] = a.rsx + (size_t)zc_idx * a.rsx_stride + (size_t)(m0 + e) * a.kz + half * 8;
      else
        zsrc[u] = a.cz + (size_t)zc_idx * a.cz_stride + (size_t)min(n0 + e, a.N - 1) * a.kz + half * 8;
    }
    // scales: 128 bf16 of the tile's columns, 4 bytes per lane
    ssrc = a.sct + (size_t)zc_idx * a.sct_stride + n0 + 2 * lane;
  }

  auto load_stage = [&](int g, int s) {
    const uint32_t st = smem_base + s * SM::kStage;
#pragma unroll
    for (int i = 0; i < 8; ++i) lds_copy16(asrc[i] + g * 128, st + SM::kA + (8 * wave + i) * 1024);
    if constexpr (INT4) {
#pragma unroll
      for (int u = 0; u < 2; ++u) lds_copy16(wsrc[u] + g * 64, st + SM::kB + (2 * wave + u) * 1024);
      // zero-point step t = g (a repeat of step 0 for g >= ceil(G/3), so every
      // stage issues the same copies; it is not used)
      const int t = g < T3 ? g : 0;
#pragma unroll
      for (int u = 0; u < 2; ++u) lds_copy16(zsrc[u] + t * 16, st + SM::kZ + (2 * wave + u) * 1024);
      lds_copy4(ssrc + (size_t)g * a.npad, st + SM::kS + wave * 256);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) lds_copy16(wsrc[i] + g * 256, st + SM::kB + (8 * wave + i) * 1024);
    }
  };

  // fragment reads of a 256-byte-row tile (activations; bf16 weights): row r,
  // logical chunk 8h + j at stored chunk (8h + j) ^ (r & 15); r & 15 = l32 & 15
  const int sw = l32 & 15;
  auto frag = [&](const unsigned char* tile, int row, int j) {
    return *reinterpret_cast<const bf16x8*>(tile + row * 256 + (((8 * h + j) ^ sw) * 16));
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int bm = 0; bm < 2; ++bm)
#pragma unroll
    for (int bn = 0; bn < 2; ++bn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bm][bn][r] = 0.0f;

  const uint32_t nib_mask = opaque_vgpr(0x000F000Fu);
  auto compute = [&](int s, bool zstep) {
    const unsigned char* st = smem + s * SM::kStage;
    const unsigned char* sa = st + SM::kA;
    const unsigned char* sb = st + SM::kB;
    if constexpr (INT4) {
      // this lane's 8 words of each of its two columns
      uint4 wv[2][2];
#pragma unroll
      for (int bn = 0; bn < 2; ++bn) {
        const int col = wn * 64 + bn * 32 + l32;
#pragma unroll
        for (int c = 0; c < 2; ++c)
          wv[bn][c] = *reinterpret_cast<const uint4*>(sb + col * 64 + (((2 * h + c) ^ ((col >> 2) & 3)) * 16));
      }
      f32x16 tmp[2][2];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bf16x8 af[2], bf[2];
#pragma unroll
        for (int bm = 0; bm < 2; ++bm) af[bm] = frag(sa, wm * 64 + bm * 32 + l32, j);
#pragma unroll
        for (int bn = 0; bn < 2; ++bn) {
          const uint4 w4v = wv[bn][j >> 2];
          const uint32_t word = (j & 3) == 0 ? w4v.x : (j & 3) == 1 ? w4v.y : (j & 3) == 2 ? w4v.z : w4v.w;
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
      // zero-point step (accumulates straight into acc)
      if (zstep) {
        const unsigned char* sz = st + SM::kZ;
        bf16x8 za[2], zb[2];
#pragma unroll
        for (int bm = 0; bm < 2; ++bm) {
          const int e = wm * 64 + bm * 32 + l32;
          za[bm] = *reinterpret_cast<const bf16x8*>(sz + e * 32 + ((h ^ ((e >> 3) & 1)) * 16));
        }
#pragma unroll
        for (int bn = 0; bn < 2; ++bn) {
          const int e = wn * 64 + bn * 32 + l32;
          zb[bn] = *reinterpret_cast<const bf16x8*>(sz + 4096 + e * 32 + ((h ^ ((e >> 3) & 1)) * 16));
        }
#pragma unroll
        for (int bm = 0; bm < 2; ++bm)
#pragma unroll
          for (int bn = 0; bn < 2; ++bn)
            acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(za[bm], zb[bn], acc[bm][bn], 0, 0, 0);
      }
      // fold: acc += sc * tmp (scales of columns past N are 0)
      const uint16_t* ss = reinterpret_cast<const uint16_t*>(st + SM::kS + wave * 256);
      float sc[2];
#pragma unroll
      for (int bn = 0; bn < 2; ++bn) sc[bn] = bf16_bits_to_f32(ss[wn * 64 + bn * 32 + l32]);
#pragma unroll
      for (int bm = 0; bm < 2; ++bm)
#pragma unroll
        for (int bn = 0; bn < 2; ++bn)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[bm][bn][r] = fmaf(sc[bn], tmp[bm][bn][r], acc[bm][bn][r]);
    } else {
      (void)zstep;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bf16x8 af[2], bf[2];
#pragma unroll
        for (int bm = 0; bm < 2; ++bm) af[bm] = frag(sa, wm * 64 + bm * 32 + l32, j);
#pragma unroll
        for (int bn = 0; bn < 2; ++bn) bf[bn] = frag(sb, wn * 64 + bn * 32 + l32, j);
#pragma unroll
        for (int bm = 0; bm < 2; ++bm)
#pragma unroll
          for (int bn = 0; bn < 2; ++bn)
            acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[bm], bf[bn], acc[bm][bn], 0, 0, 0);
      }
    }
  };

  // Pipeline.  Stage s holds group g with g % S == s.  Iteration g waits until
  // this wave's copies of group g are complete (groups g+1 .. g+D-1 may stay in
  // flight), barriers -- after which every wave's group-g copies are in LDS and
  // every wave has finished reading group g-1 -- then issues the copies of group
  // g + D into the stage group g-1 used, and computes group g.
#pragma unroll
  for (int p = 0; p < D; ++p)
    if (p < G) load_stage(p, p);

  auto iteration = [&](auto sidx, int g) {
    constexpr int s = decltype(sidx)::value;
    const int ahead = min(D - 1, G - 1 - g);   // groups after g already issued
    static_assert(D <= 2, "waits below cover at most one stage in flight");
    if (ahead >= 1) wait_vmcnt<L>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (g + D < G) load_stage(g + D, (s + D) % S);
    compute(s, INT4 && g < T3);
  };

  for (int g = 0; g < G; g += S) {
    iteration(std::integral_constant<int, 0>{}, g);
    if (g + 1 >= G) break;
    iteration(std::integral_constant<int, 1>{}, g + 1);
    if constexpr (S >= 3) {
      if (g + 2 >= G) break;
      iteration(std::integral_constant<int, 2>{}, g + 2);
    }
  }

  // epilogue.  Output layout of a 32x32 block: lane holds column l32 and rows
  // 8*i + 4*h + j for register 4*i + j.
  bool nok[2];
  int ncol[2];
#pragma unroll
  for (int bn = 0; bn < 2; ++bn) {
    ncol[bn] = n0 + wn * 64 + bn * 32 + l32;
    nok[bn] = ncol[bn] < a.N;
  }
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
    // all copies have completed (the last iteration waited for vmcnt 0) and every
    // wave is past its last LDS read after this barrier: stage 0 is free
    float* sRed = reinterpret_cast<float*>(smem);
    lds_barrier();
    if (lane == 0) sRed[wave] = s;
    __syncthreads();
    if (tid == 0) {
      const float tot = (sRed[0] + sRed[1]) + (sRed[2] + sRed[3]);
      a.partials[(size_t)zc_idx * gridDim.x + blockIdx.x] = tot;
    }
  }
}

// Operands written by the prologue kernel (defined in gemm.hip), for C problems:
//   rsx[c][m][16t + s] (m < mpad; rows >= M are 0): group row sums of X[c] split
//   into bf16 parts, cz[c][n][16t + s]: -sc (128 + z) split into bf16 parts, with
//   slot s = 5j + u for group 3t + j: rs parts (hi, hi, mid, mid, lo) against
//   c parts (hi, lo, hi, lo, hi); slot 15 and slots of groups >= G are 0;
//   sct[c][g][n] (n < npad): the scales group-major, 0 for n >= N.
// When xp is not NULL it also writes X[c] pair-arranged (every 8-channel run as
// (x0,x4)(x1,x5)(x2,x6)(x3,x7)) into xp[c] ([M][K], same strides as X).
inline int zterm_kz(int K) { return 16 * (((K >> 7) + 2) / 3); }
inline int gemm_npad(int N) { return (N + kBN - 1) / kBN * kBN; }
int launch_zterm_prep(const uint16_t* X, size_t x_stride, int M, int K, int mpad, const uint16_t* scales,
                      size_t sc_stride, const uint32_t* qzeros, size_t qz_stride, int symmetric, int N,
                      uint16_t* rsx, size_t rsx_stride, uint16_t* cz, size_t cz_stride, uint16_t* sct,
                      size_t sct_stride, uint16_t* xp, int C, hipStream_t stream);

}  // namespace w4
