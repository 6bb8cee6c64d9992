// MFMA core of the W4A16 prefill contraction, shared by w4a16_gemm and the AWQ
// grid loss.  Y = X W_hat^T with X bf16 [M][K] and W_hat given as packed int4
// groups (q - z) * sc.
//
// Workgroup tile 64 x 128, 4 waves: wave w computes all 64 rows of columns
// 32 w .. +31 as 2 v_mfma_f32_32x32x16_bf16 blocks, so every packed weight word is
// expanded once per tile.  Two or three workgroups share a CU (three stages of
// 25 KB of LDS each, or two stages for three workgroups): while one waits at its
// per-group barrier the others keep the matrix cores busy.  One main-loop step
// covers one 128-channel quantization group.
//
// Every operand of a group travels from global memory straight into LDS
// (global_load_lds: no registers), one or two groups ahead.  These copies are issued
// from inline assembly, so the compiler's wait-counter bookkeeping does not see
// them: it would otherwise wait for every copy in flight, including those of
// later groups, before each LDS read.  The kernel waits for exactly the copies of
// the group it is about to use (vmcnt counts one wave's copies, which complete in
// issue order), then synchronises the workgroup with a bare s_barrier.
//
// Per stage (int4 weights):
//   * activations: 64 rows x 128 channels bf16 (16 KB); inside a 256-byte row
//     the 16-byte chunk c is stored at position c ^ (row & 15).  They arrive
//     pre-arranged: every 8-channel run holds the pairs (x0,x4)(x1,x5)(x2,x6)
//     (x3,x7), the order in which one packed word expands (written so by the
//     prologue kernel);
//   * packed words: 128 columns x 16 words (8 KB); inside a column's 64 bytes the
//     16-byte chunk c is stored at position c ^ ((col >> 2) & 3);
//   * per column of the group: scale bits | bf16(128 + z) << 16 (the prologue
//     writes them group-major, zero past N);
//   * per row of the group: the negated row sum of the group's activations as
//     three bf16 parts (hi, mid, lo, exact) and a zero.
// Each lane's weight operand for one MFMA is one packed uint32 word (8
// consecutive channels of its output column), expanded in registers to bf16
// integers 128 + q.  Per group the MFMAs first put the zero-point term
// -rowsum_g(X)[m] (128 + z[n,g]) into a per-group fp32 tile (one K=16 step with 3
// live k-slots: hi, mid, lo times 128 + z, all products exact), then accumulate
// the exact integer-weight products sum_k x (128 + q) on top: the tile holds
// sum_k x (q - z).  It is folded into the output accumulator with one FMA,
// acc += sc * tmp, at the start of the next group, while that group's LDS reads
// of packed words, column words and row sums are in flight.
// The k-slots of the MFMA are assigned so that lane half h, step j covers
// channels 64h + 8j .. 64h + 8j + 7 of the group: each lane's 8 words of a group
// are contiguous.
#pragma once

#include <type_traits>

#include "internal.hpp"

namespace w4 {

constexpr int kBM = 64;
constexpr int kBN = 128;

enum { EPI_STORE = 0, EPI_SQDIFF = 1 };

struct GemmCoreArgs {
  const uint16_t* X;       // [M][K] bf16 (+ z * x_stride), pair-arranged, rows up to M rounded to 128 readable
  size_t x_stride;
  int M, K, N;
  const uint32_t* qweight; // [N][K/8] (+ z * qw_stride)
  size_t qw_stride;
  const uint16_t* rsq;     // [K/128][mpad][4] bf16: -(group row sum of X) as hi, mid, lo, 0 (+ z * rsq_stride)
  size_t rsq_stride;
  const uint32_t* szq;     // [K/128][npad]: scale bits | bf16(128 + z) << 16, 0 for columns >= N (+ z * szq_stride)
  size_t szq_stride;
  int mpad, npad;          // M and N rounded up to 128
  // split over K: workgroup (tile, blockIdx.y) covers groups [gsplit y, gsplit (y + 1));
  // 0 = all groups
  int gsplit;
  // epilogue
  uint16_t* Y;             // EPI_STORE: [M][N] bf16 (ypart == NULL)
  float* ypart;            // EPI_STORE with a K split: fp32 partial sums, split y's [M][N] at y * ypart_stride
  size_t ypart_stride;
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

// Global -> LDS copies: lane l reads 16 (or 4) bytes at base + off (base a
// wave-uniform 64-bit address held in SGPRs, off a per-lane unsigned 32-bit byte
// offset) and writes them at LDS byte address m0 + 16 l (4 l).  M0 is set by the
// compiler from the "{m0}" operand; the s_nop covers the one wait state the
// hardware needs between an M0 write and an LDS copy.
__device__ __forceinline__ void lds_copy16(uint32_t off, const void* base, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_copy4(uint32_t off, const void* base, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}

// Workgroup barrier without a memory fence.  LDS reads are complete (lgkmcnt);
// global->LDS copies are covered by the explicit vmcnt waits before it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS byte layout of one pipeline stage.  int4: three stages and two workgroups
// per CU, or (WIDE) two stages and three workgroups per CU -- more waves to hide
// latency, one group less of prefetch; the launchers take WIDE when the grid is
// larger than one round of two workgroups per CU (measured, M = 2048: K = 2048,
// N = 6144, 1536 tiles, 70.6 -> 66.8 us; K = 6144, N = 2048, 512 tiles, stays on
// the three-stage kernel, which the wide one would slow from 69.8 to 76.5 us).
template <bool WIDE = false>
struct GemmSmem {
  static constexpr int kA = 0;                     // activations, 16 KB
  static constexpr int kB = kBM * 256;             // packed words, 8 KB
  static constexpr int kS = kB + kBN * 64;         // column words, 128 x 4 B
  static constexpr int kR = kS + 512;              // row sums, 64 x 8 B
  static constexpr int kStage = kR + 512;
  static constexpr int kStages = WIDE ? 2 : 3;
  static constexpr int kBlocksPerCU = WIDE ? 3 : 2;
  // copies issued per stage and wave (each moves 1 KB, or 256 B for the 4-byte
  // one): activations 4, packed words 2, column words or row sums 1
  static constexpr int kCopies = 7;
  static_assert(kStage * kStages * kBlocksPerCU <= 160 * 1024, "LDS");
};

constexpr int kGemmWaves = 4;

// Resident workgroups of the three-stage kernel on 256 CUs; a larger grid
// takes the WIDE kernel.
constexpr long long kCoreSlots = 2 * 256;
inline bool gemm_core_wide(long long workgroups) { return workgroups > kCoreSlots; }

template <int EPI, bool WIDE = false>
__global__ __launch_bounds__(kGemmWaves * 64, (GemmSmem<WIDE>::kBlocksPerCU)) void gemm_core_kernel(
    GemmCoreArgs a) {
  using SM = GemmSmem<WIDE>;
  constexpr int S = SM::kStages;
  constexpr int D = S - 1;                 // prefetch distance in groups
  constexpr int L = SM::kCopies;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[S * SM::kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // column block of the tile
  const int h = lane >> 5, l32 = lane & 31;
  int tm, tn;
  tile_coords(blockIdx.x, (a.M + kBM - 1) / kBM, (a.N + kBN - 1) / kBN, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int zc_idx = blockIdx.z;
  const int G = a.K >> 7;
  const int g0 = a.gsplit ? (int)blockIdx.y * a.gsplit : 0;   // this workgroup's groups: [g0, g0 + Gl)
  const int Gl = a.gsplit ? min(G - g0, a.gsplit) : G;
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;   // LDS byte address (low half of the generic one)

  // ---- copy sources: wave-uniform bases (without the group term) and per-lane byte offsets ----
  // Activations: copy i of wave w fills rows 4 u .. 4 u + 3 with u = w + 4 i;
  // lane -> row 4 u + lane / 16, stored chunk lane % 16 holding logical chunk
  // (lane % 16) ^ (row & 15), and row & 15 = 4 w + lane / 16 for every i.  X has
  // rows up to M rounded to 64 (the prologue pads them), so copy i is copy 0
  // moved by 16 rows and one offset serves all four (< 2 mpad K).
  const unsigned char* abase = reinterpret_cast<const unsigned char*>(a.X + (size_t)zc_idx * a.x_stride);
  const int arow = 4 * wave + (lane >> 4);
  const uint32_t achunk = (uint32_t)(((lane & 15) ^ (arow & 15)) * 8);
  const uint32_t aoff = ((uint32_t)(m0 + arow) * (uint32_t)a.K + achunk) * 2u;
  // Packed words: copy u (of 2) of wave w fills LDS chunks 64 (2 w + u) + lane:
  // column (64 (2 w + u) + lane) / 4, stored chunk lane % 4 holding logical chunk
  // (lane % 4) ^ ((col >> 2) & 3) (LDS serves a 16-byte read 16 lanes at a time
  // over 64 banks: 16 consecutive columns then hit 16 distinct 16-byte bank
  // groups); offsets < N K / 2.  Columns past N read column N-1.
  const unsigned char* wbase = reinterpret_cast<const unsigned char*>(a.qweight + (size_t)zc_idx * a.qw_stride);
  uint32_t woff[2];
  {
    const uint32_t words = (uint32_t)(a.K >> 3);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int p = 64 * (2 * wave + u) + lane;
      const int col = p >> 2;
      const int chunk = (p & 3) ^ ((col >> 2) & 3);
      woff[u] = (uint32_t)min(n0 + col, a.N - 1) * words * 4u + (uint32_t)chunk * 16u;
    }
  }
  // 4-byte copies: waves 0, 1 copy the column words of columns 64 w .. +63;
  // waves 2, 3 copy the row sums of rows 32 (w - 2) .. +31 (8 bytes each, 4 per lane)
  const unsigned char* mbase;
  uint32_t mdst;
  if (wave < 2) {
    mbase = reinterpret_cast<const unsigned char*>(a.szq + (size_t)zc_idx * a.szq_stride + n0 + 64 * wave);
    mdst = SM::kS + wave * 256;
  } else {
    mbase = reinterpret_cast<const unsigned char*>(a.rsq + (size_t)zc_idx * a.rsq_stride +
                                                   (size_t)(m0 + 32 * (wave - 2)) * 4);
    mdst = SM::kR + (wave - 2) * 256;
  }

  // Sources of one group's copies: wave-uniform base addresses.
  struct GroupSrc {
    const unsigned char* a;   // activations
    const unsigned char* w;   // packed words
    const unsigned char* m;   // row sums or column words
  };
  auto group_src = [&](int g) {
    GroupSrc r;
    r.a = abase + (size_t)g * 256;
    r.w = wbase + (size_t)g * 64;
    r.m = mbase + (size_t)g * (wave < 2 ? (size_t)a.npad * 4 : (size_t)a.mpad * 8);
    return r;
  };
  // copy k (0 .. L-1) of a group into the stage at LDS byte address st: 0-3
  // activations, 4-5 packed words, 6 column words / row sums
  auto copy_piece = [&](auto kidx, const GroupSrc& src, uint32_t st) {
    constexpr int k = decltype(kidx)::value;
    if constexpr (k < 4)
      lds_copy16(aoff, src.a + (size_t)k * 32 * a.K, st + SM::kA + (wave + 4 * k) * 1024);
    else if constexpr (k < 6)
      lds_copy16(woff[k - 4], src.w, st + SM::kB + (2 * wave + k - 4) * 1024);
    else
      lds_copy4(4u * (uint32_t)lane, src.m, st + mdst);
  };
  // the copies that go with MFMA step j of the group being computed: the packed
  // words and the column words / row sums first (steps 0-2), so that they can be
  // waited for one group earlier than the activations (steps 3-6)
  auto copies_of_step = [&](auto jidx, const GroupSrc& src, uint32_t st) {
    constexpr int j = decltype(jidx)::value;
    if constexpr (j < L) copy_piece(std::integral_constant<int, j < 3 ? j + 4 : j - 3>{}, src, st);
  };

  // fragment reads of the activation tile: row
  // 32 rb + l32 (rb = 32-row block), logical chunk 8h + j at stored chunk
  // (8h + j) ^ (l32 & 15), i.e. byte (l32 * 256 + ((8h ^ (l32 & 15)) * 16)) ^ (16 j)
  // + 8192 rb: one XOR per step, the rest immediate offsets
  const uint32_t fbase = (uint32_t)(l32 * 256 + (((8 * h) ^ (l32 & 15)) * 16));
  uint32_t fb = fbase;
  auto frag = [&](const unsigned char* tile, int rb, int j) {
    return *reinterpret_cast<const bf16x8*>(tile + ((fb ^ (uint32_t)(16 * j)) + 8192u * rb));
  };
  const int col = 32 * wave + l32;         // this lane's output column within the tile

  f32x16 acc[2];
#pragma unroll
  for (int bm = 0; bm < 2; ++bm)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[bm][r] = 0.0f;
  // per-group products of the last group computed and its scale, folded
  // into acc at the start of the next group (0 * 0 before the first)
  f32x16 tmp[2];
#pragma unroll
  for (int bm = 0; bm < 2; ++bm)
#pragma unroll
    for (int r = 0; r < 16; ++r) tmp[bm][r] = 0.0f;
  float sc_prev = 0.0f;

  const uint32_t nib_mask = opaque_vgpr(0x000F000Fu);
  // what a lane needs of a group besides the activations -- its 8 packed
  // words, its column word and the row sums of its two row blocks.  Three stages:
  // read one group ahead (see the pipeline below), so no group starts on an LDS
  // round trip; two stages (WIDE): read at the start of the group, whose copies
  // are the only ones complete at its barrier (the third workgroup on the CU
  // covers the wait).
  struct GroupMisc {
    uint4 wv[2];
    uint32_t szw;
    uint2 rv[2];
  };
  auto read_misc = [&](const unsigned char* st, GroupMisc& gm) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
      gm.wv[c] = *reinterpret_cast<const uint4*>(st + SM::kB + col * 64 + (((2 * h + c) ^ ((col >> 2) & 3)) * 16));
    gm.szw = reinterpret_cast<const uint32_t*>(st + SM::kS)[col];
#pragma unroll
    for (int bm = 0; bm < 2; ++bm) gm.rv[bm] = *reinterpret_cast<const uint2*>(st + SM::kR + (32 * bm + l32) * 8);
  };
  GroupMisc gcur{}, gnext{};
  // Computes the group in stage s; between its MFMA steps it issues the copies of
  // the group described by nsrc into the stage at LDS byte address nst.  The
  // activation fragments of step j+1 are read before the MFMAs of step j.  Uses
  // gcur and, during step 4, reads the next group's GroupMisc (stage s+1) into
  // gnext.
  auto compute = [&](int s, const GroupSrc& nsrc, uint32_t nst) {
    const unsigned char* st = smem + s * SM::kStage;
    const unsigned char* sa = st + SM::kA;
    // recomputed per group: hoisted out of the loop, the eight per-step
    // addresses would stay live in registers for the whole kernel
    fb = opaque_vgpr(fbase);
    bf16x8 af[2][2];
#pragma unroll
    for (int bm = 0; bm < 2; ++bm) af[0][bm] = frag(sa, bm, 0);
    {
      if constexpr (D == 1) read_misc(st, gcur);
      // fold the previous group's blocks, acc += sc_prev * tmp, while the reads
      // above are in flight (two stages: this group's misc words arrive from LDS now)
#pragma unroll
      for (int bm = 0; bm < 2; ++bm)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[bm][r] = fmaf(sc_prev, tmp[bm][r], acc[bm][r]);
      __builtin_amdgcn_sched_barrier(0);
      const uint4* wv = gcur.wv;
      // zero-point step operands: k-slots 0..2 (lane half 0) hold the row sum parts
      // against 128 + z three times; every other slot is 0
      const float sc_cur = __uint_as_float(gcur.szw << 16);
      const uint32_t zbf = gcur.szw >> 16;
      const bf16x8 zb = __builtin_bit_cast(bf16x8, make_uint4(h ? 0u : zbf * 0x10001u, h ? 0u : zbf, 0u, 0u));
      bf16x8 za[2];
#pragma unroll
      for (int bm = 0; bm < 2; ++bm)
        za[bm] = __builtin_bit_cast(bf16x8, make_uint4(h ? 0u : gcur.rv[bm].x, h ? 0u : gcur.rv[bm].y, 0u, 0u));
      const unsigned char* st_next = smem + ((s + 1) % S) * SM::kStage;
      __builtin_amdgcn_sched_barrier(0);
      auto step = [&](auto jidx) {
        constexpr int j = decltype(jidx)::value;
        if constexpr (j < 7) {
#pragma unroll
          for (int bm = 0; bm < 2; ++bm) af[(j + 1) & 1][bm] = frag(sa, bm, j + 1);
        }
        if constexpr (j == 4 && D == 2) read_misc(st_next, gnext);
        // keep the reads of step j+1 ahead of the MFMAs of step j (the scheduler
        // would otherwise sink each read next to its use and expose LDS latency)
        __builtin_amdgcn_sched_barrier(0);
        copies_of_step(jidx, nsrc, nst);
        const uint4 w4v = wv[j >> 2];
        const uint32_t word = (j & 3) == 0 ? w4v.x : (j & 3) == 1 ? w4v.y : (j & 3) == 2 ? w4v.z : w4v.w;
        const bf16x8 bf = __builtin_bit_cast(
            bf16x8, make_uint4(nibble_pair_m(word, 0, nib_mask), nibble_pair_m(word, 1, nib_mask),
                               nibble_pair_m(word, 2, nib_mask), nibble_pair_m(word, 3, nib_mask)));
        if constexpr (j == 0) {
          // start this group's blocks with their zero-point terms
#pragma unroll
          for (int bm = 0; bm < 2; ++bm)
            tmp[bm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(za[bm], zb, f32x16{}, 0, 0, 0);
        }
#pragma unroll
        for (int bm = 0; bm < 2; ++bm)
          tmp[bm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[j & 1][bm], bf, tmp[bm], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      };
      step(std::integral_constant<int, 0>{});
      step(std::integral_constant<int, 1>{});
      step(std::integral_constant<int, 2>{});
      step(std::integral_constant<int, 3>{});
      step(std::integral_constant<int, 4>{});
      step(std::integral_constant<int, 5>{});
      step(std::integral_constant<int, 6>{});
      step(std::integral_constant<int, 7>{});
      // this group's scale (columns past N have 0); its fold happens in step 0 of
      // the next group (or after the loop)
      sc_prev = sc_cur;
      if constexpr (D == 2) gcur = gnext;
      (void)st_next;
    }
  };

  // Pipeline.  Stage s holds group g with g % S == s.  Iteration g waits until
  // this wave's copies of group g are complete (with 3 stages those of group
  // g+1, issued during iteration g-1, may stay in flight), barriers -- after which every
  // wave's group-g copies are in LDS and every wave has finished reading group
  // g-1 -- then computes group g while issuing the copies of group g + D into the
  // stage group g-1 used.  Past its last group a workgroup's copies repeat that group into
  // that stage, which nothing reads again: every stage issues the same L copies,
  // so the wait count is the same in every iteration.
  static_assert(D == 1 || D == 2, "at most one stage in flight at each wait");
#pragma unroll
  for (int p = 0; p < D; ++p) {
    const GroupSrc src = group_src(g0 + min(p, Gl - 1));
    const uint32_t st = smem_base + p * SM::kStage;
    copies_of_step(std::integral_constant<int, 0>{}, src, st);
    copies_of_step(std::integral_constant<int, 1>{}, src, st);
    copies_of_step(std::integral_constant<int, 2>{}, src, st);
    copies_of_step(std::integral_constant<int, 3>{}, src, st);
    copies_of_step(std::integral_constant<int, 4>{}, src, st);
    copies_of_step(std::integral_constant<int, 5>{}, src, st);
    copies_of_step(std::integral_constant<int, 6>{}, src, st);
    copies_of_step(std::integral_constant<int, 7>{}, src, st);
  }

  // Three stages: at the barrier of group g the copies still in flight are
  // the activation copies of group g+1 (its other copies, issued first, are
  // complete: every wave may read group g+1's GroupMisc during group g).  Two
  // stages: none (group g+1's copies are issued after this barrier).
  constexpr int kInFlight = D == 2 ? 4 : 0;
  if constexpr (D == 2) {
    wait_vmcnt<kInFlight>();
    lds_barrier();
    read_misc(smem, gcur);
  }
  auto iteration = [&](auto sidx, int g) {
    constexpr int s = decltype(sidx)::value;
    wait_vmcnt<kInFlight>();
    lds_barrier();
    const GroupSrc nsrc = group_src(g0 + min(g + D, Gl - 1));
    compute(s, nsrc, smem_base + ((s + D) % S) * SM::kStage);
  };

  for (int g = 0; g < Gl; g += S) {
    iteration(std::integral_constant<int, 0>{}, g);
    if (g + 1 >= Gl) break;
    iteration(std::integral_constant<int, 1>{}, g + 1);
    if constexpr (S == 3) {
      if (g + 2 >= Gl) break;
      iteration(std::integral_constant<int, 2>{}, g + 2);
    }
  }
  // the repeated copies of the last iterations must land before LDS is reused or released
  wait_vmcnt<0>();
#pragma unroll
  for (int bm = 0; bm < 2; ++bm)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[bm][r] = fmaf(sc_prev, tmp[bm][r], acc[bm][r]);

  // epilogue.  Output layout of a 32x32 block: lane holds column l32 and rows
  // 8*i + 4*h + j for register 4*i + j.
  const int ncol = n0 + col;
  const bool nok = ncol < a.N;
  if constexpr (EPI == EPI_STORE) {
    if (nok && a.ypart) {
      float* yp = a.ypart + (size_t)blockIdx.y * a.ypart_stride;
#pragma unroll
      for (int bm = 0; bm < 2; ++bm)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + 32 * bm + 8 * (r >> 2) + 4 * h + (r & 3);
          if (row < a.M) yp[(size_t)row * a.N + ncol] = acc[bm][r];
        }
    } else if (nok) {
#pragma unroll
      for (int bm = 0; bm < 2; ++bm)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + 32 * bm + 8 * (r >> 2) + 4 * h + (r & 3);
          if (row < a.M) a.Y[(size_t)row * a.N + ncol] = (uint16_t)f32_to_bf16_bits(acc[bm][r]);
        }
    }
  } else {
    // Squared differences against Yref.  The fp32 tile goes through LDS (rows of
    // 136 floats: the two lane halves, 4 rows apart, then hit different banks),
    // then each thread scores a quarter row with 16-byte reads of the tile and of
    // Yref.  The values are handed over as opaque bits: consumed as floats right
    // here, the optimizer may reshape the loop's accumulator into scalars and the
    // register allocator start copying it through AGPRs every group.
    constexpr int kTS = 136;
    static_assert(kBM * kTS * 4 + 4 * kGemmWaves <= S * SM::kStage, "score tile fits in the stage buffers");
    uint32_t* tile = reinterpret_cast<uint32_t*>(smem);
    lds_barrier();        // all copies have landed (vmcnt 0 above), every wave is past its last read
#pragma unroll
    for (int bm = 0; bm < 2; ++bm)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        tile[(32 * bm + 8 * (r >> 2) + 4 * h + (r & 3)) * kTS + col] =
            opaque_vgpr(__float_as_uint(acc[bm][r]));
    __syncthreads();
    const int trow = tid >> 2;                 // tile row scored by this thread
    const int tc0 = (tid & 3) * 32;            // first of its 32 tile columns
    float s = 0.0f;
    if (m0 + trow < a.M) {
      const uint16_t* yr = a.Yref + (size_t)(m0 + trow) * a.N + n0 + tc0;
      const float* tr = reinterpret_cast<const float*>(tile) + trow * kTS + tc0;
      const int ncols = min(32, a.N - n0 - tc0);     // may be <= 0
      if (ncols == 32 && (a.N & 7) == 0 && (reinterpret_cast<uintptr_t>(a.Yref) & 15) == 0) {
#pragma unroll
        for (int c8 = 0; c8 < 4; ++c8) {
          const uint4 yv = *reinterpret_cast<const uint4*>(yr + 8 * c8);
          const float4 t0 = *reinterpret_cast<const float4*>(tr + 8 * c8);
          const float4 t1 = *reinterpret_cast<const float4*>(tr + 8 * c8 + 4);
          const float tv[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
          const uint32_t yw[4] = {yv.x, yv.y, yv.z, yv.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float yf = __uint_as_float((e & 1) ? (yw[e >> 1] & 0xFFFF0000u) : (yw[e >> 1] << 16));
            const float d = tv[e] - yf;
            s = fmaf(d, d, s);
          }
        }
      } else {
        for (int c = 0; c < ncols; ++c) {
          const float d = tr[c] - bf16_bits_to_f32(yr[c]);
          s = fmaf(d, d, s);
        }
      }
    }
    s = wave_sum(s);
    float* sRed = reinterpret_cast<float*>(smem) + kBM * kTS;
    if (lane == 0) sRed[wave] = s;
    __syncthreads();
    if (tid == 0) {
      float tot = 0.0f;
#pragma unroll
      for (int w = 0; w < kGemmWaves; ++w) tot += sRed[w];
      a.partials[(size_t)zc_idx * gridDim.x + blockIdx.x] = tot;
    }
  }
}

// Operands written by the prologue kernel (defined in gemm.hip), for C problems
// (c = blockIdx.z of the core):
//   rsq[c][g][m][0..3] (m < mpad): -(sum of X[c][m][128 g .. 128 g + 127]) as the
//   bf16 parts hi, mid, lo (exact) and 0; 0 for rows >= M;
//   szq[c][g][n] (n < npad): scale bits | bf16(128 + z) << 16 (z = 8 when
//   symmetric); 0 for columns >= N.
// When xp is not NULL it also writes X[c] pair-arranged (every 8-channel run as
// (x0,x4)(x1,x5)(x2,x6)(x3,x7)) into xp[c] ([mpad][K], same strides as X; rows
// M .. mpad-1 zero).  Only the first rs_c problems (all when negative) get row sums
// and arranged rows: the others share the first one's activations.
__host__ __device__ inline int gemm_npad(int N) { return (N + kBN - 1) / kBN * kBN; }
int launch_gemm_prep(const uint16_t* X, size_t x_stride, int M, int K, int mpad, const uint16_t* scales,
                     size_t sc_stride, const uint32_t* qzeros, size_t qz_stride, int symmetric, int N,
                     uint16_t* rsq, size_t rsq_stride, uint32_t* szq, size_t szq_stride, uint16_t* xp, int C,
                     hipStream_t stream, int rs_c = -1);

}  // namespace w4
