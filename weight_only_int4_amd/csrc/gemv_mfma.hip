// Decode contraction Y = X W_hat^T on the matrix cores, for the larger decode
// batches (W4A16 GEMV, MFMA form; gemv_use_mfma below is the measured rule by which
// the launcher in gemv.hip picks it over the VALU form).
//
// Model card "GLM-5.2-QSRT-Fruit-Instruct", "Reproducible runtime": decode
// batches of at most 16 rows take their own path.  The VALU form (gemv.hip)
// spends M dot products on every unpacked weight pair, so from a few rows on it is
// bound by vector ALU work instead of memory.  Here one v_mfma_f32_16x16x32_bf16
// multiplies a block of 16 columns x 32 channels of unpacked weights with all 16
// activation rows (rows past M are don't-care rows whose outputs are never
// stored): the per-weight VALU work -- the unpacking and the per-group fold -- no
// longer grows with M.
//
// Design (CDNA4, wave64):
//  * MFMA operands: A = activations (16 rows x 32 k-slots), B = unpacked weights
//    (32 k-slots x 16 columns), D = fp32 16 x 16.  Lane l = j + 16 q holds row j
//    of A and column j of B in k-slots 8 q .. 8 q + 7, and column j, rows
//    4 q .. 4 q + 3 of D.  In step s (0..3) of a 128-channel group, lane quarter q
//    takes the group's packed word 4 q + s (channels 32 q + 8 s .. + 7) as its B
//    slots; its A slots in step s are the same 8 channels of row j, pair-arranged
//    as (x0,x4)(x1,x5)(x2,x6)(x3,x7) to match the order in which a word unpacks.
//  * Memory access: both operands are read so that every four consecutive lanes
//    hit one cache line, then rearranged -- the packed words (lanes 4 c .. 4 c + 3:
//    the 64 bytes of column c in a group) with ds_bpermute, the activations (16
//    lanes per 256-byte row, rows below M only) through a per-wave LDS staging area.
//  * A wave owns KT consecutive groups of one K split and streams the BPW blocks
//    of 16 columns of its slab; its A operands and the group row sums of X stay
//    in registers for the whole slab.  nwk waves cover the groups of a split; rw
//    slabs share a workgroup.
//  * Per block and group: the zero-point term -(128 + z) rowsum_g(x) (the row
//    sums also taken on the matrix cores, against a B of ones) is the
//    initial accumulator of the group's tile, four MFMAs add the exact products
//    x (128 + q) (bf16 integers below 2^8 times bf16 activations: exact in fp32),
//    and acc += sc * tile folds the group into the block's result.
//  * Loads are buffer loads (an out-of-range offset returns 0 and touches no
//    memory): columns past N and groups past the split read zeros, whose tiles
//    are 0 and whose scales are 0.
//  * The nwk partial tiles of a block meet in LDS and are added in wave order;
//    with a K split the fp32 sums go to the workspace and gemv_split_reduce adds
//    the splits in order.  Every sum has a fixed order: results are
//    reproducible bit for bit.
#include <atomic>

#include "internal.hpp"

namespace w4 {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

namespace {

// Groups per wave: 2 (about 100 VGPRs, up to 16 waves per workgroup) when K fits
// one workgroup that way (K <= 4096), else 4 (about 160 VGPRs, up to 12 waves).
constexpr int max_waves(int kt) { return kt == 4 ? 12 : 16; }
constexpr int kMaxWavesAny = 16;
constexpr int kBlockCols = 16;    // columns per MFMA block

struct MfmaArgs {
  const uint16_t* X;
  int M, K, N;
  const uint32_t* qweight;
  const uint16_t* scales;
  const uint32_t* qzeros;
  uint16_t* Y;
  float* partial;       // [splits][M][N] when splits > 1
  int gs;               // groups per split (the last split may hold fewer)
  int nwk;              // waves per slab (nwk * KT >= gs)
  int rw;               // slabs per workgroup
};

template <int KT, int BPW, bool SYM, bool NT>
__global__ __launch_bounds__(max_waves(KT) * 64) void gemv_mfma_kernel(MfmaArgs a) {
  constexpr int NB = 2;            // blocks in flight
  constexpr int bpw = BPW;
  // Dynamic LDS: per wave a staging area for one group of its activation rows
  // ([4 qm rows][256 bytes], qm = ceil(M / 4)), then, when nwk > 1, the partial
  // tiles [rw * nwk][BPW][qm * 16] of the lanes that hold rows below M (lane
  // quarters q < qm).
  extern __shared__ f32x4 lds_dyn[];
  const int qm = (a.M + 3) >> 2;
  f32x4* red = lds_dyn + (size_t)(blockDim.x >> 6) * qm * 4 * 16;

  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x >> 6;
  const int slab = wid / a.nwk;
  const int wave = wid - slab * a.nwk;
  const int j = lane & 15, q = lane >> 4;
  const int G = a.K >> 7;
  const int GW = (G + 7) >> 3;
  const int gend = min(G, ((int)blockIdx.y + 1) * a.gs);
  const int g0 = (int)blockIdx.y * a.gs + wave * KT;     // this wave's groups: [g0, g0 + KT) below gend
  const uint32_t wrow = (uint32_t)a.K / 2u, srow = (uint32_t)G * 2u, zrow = (uint32_t)GW * 4u;
  const auto rwt = make_rsrc(a.qweight, (uint32_t)a.N * wrow);
  const auto rsc = make_rsrc(a.scales, (uint32_t)a.N * srow);
  const auto rzp = make_rsrc(SYM ? static_cast<const void*>(a.scales) : a.qzeros, SYM ? 0u : (uint32_t)a.N * zrow);
  const auto rx = make_rsrc(a.X, (uint32_t)a.M * (uint32_t)a.K * 2u);
  // slab S of TS takes the blocks S, S + TS, S + 2 TS, ... (block b of the slab starts
  // at column n_first + b * n_step), so that the blocks spread evenly over the slabs
  const int TS = (int)gridDim.x * a.rw;
  const int n_first = ((int)blockIdx.x * a.rw + slab) * kBlockCols;
  const int n_step = TS * kBlockCols;

  // byte offsets inside one row of each array; out of range for groups past the split
  uint32_t kw[KT], ks[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    const bool ok = g0 + t < gend;
    kw[t] = ok ? (uint32_t)(g0 + t) * 64u + 16u * (uint32_t)(lane & 3) : kOob;
    ks[t] = ok ? (uint32_t)(g0 + t) * 2u : kOob;
  }
  static_assert(8 % KT == 0, "the wave's groups share one zero word");
  const uint32_t kz = g0 < gend ? (uint32_t)(g0 >> 3) * 4u : kOob;

  // Prologue: the activations of the wave's groups, then the first NB blocks, all
  // issued before anything waits.  Activations are read row-contiguously (load u
  // of a group: rows 4 u .. 4 u + 3, sixteen lanes of 16 bytes per row, only the
  // first qm loads and only rows below M) and later rearranged through LDS into
  // the operand layout.
  const int xr_row = lane >> 4, xr_chunk = lane & 15;
  uint32_t xr[KT][4][4] = {};
#pragma unroll
  for (int t = 0; t < KT; ++t) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = 4 * u + xr_row;
      if (u < qm && r < a.M) {
        const uint32_t xo = g0 + t < gend ? ((uint32_t)r * (uint32_t)a.K + (uint32_t)(g0 + t) * 128u +
                                             8u * (uint32_t)xr_chunk) * 2u
                                          : kOob;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0);
        xr[t][u][0] = v[0]; xr[t][u][1] = v[1]; xr[t][u][2] = v[2]; xr[t][u][3] = v[3];
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  struct Batch {
    u32x4 w[KT];
    uint16_t sc[KT];     // kept 16-bit: widening at the load would wait for it right there
    uint32_t z;
  };
  // Block b of the slab (past N: nothing read).  Packed words: lanes 4 c .. 4 c + 3
  // read the 64 bytes of column n_first + b n_step + c in one group, so that every four
  // consecutive lanes hit one cache line; the lanes trade them into the operand
  // layout before use (see process).  Scale and zero word: this lane's own column
  // n_first + b n_step + j.  The row offsets are computed per load, not kept per block.
  auto load = [&](int b, Batch& B) {
    const uint32_t n = (uint32_t)min(n_first + b * n_step + j, a.N);
    const uint32_t nw = (uint32_t)min(n_first + b * n_step + (lane >> 2), a.N);
    const uint32_t ow = opaque_vgpr(nw * wrow), os = opaque_vgpr(n * srow);
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      B.w[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rwt, ow + kw[t], 0, NT ? kLoadNt : 0));
      B.sc[t] = __builtin_amdgcn_raw_buffer_load_b16(rsc, os + ks[t], 0, 0);
    }
    if constexpr (!SYM) B.z = __builtin_amdgcn_raw_buffer_load_b32(rzp, n * zrow + kz, 0, 0);
  };
  Batch B[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
    if (i < BPW) load(i, B[i]);
  __builtin_amdgcn_sched_barrier(0);

  // A operands and row sums.  Per group the wave writes its activation rows to its
  // LDS staging area (16-byte chunk c of row r at r * 256 + ((c ^ r) & 15) * 16, so
  // that the reads below hit 16 distinct bank groups) and reads back, for lane
  // (j, q) and step s, chunk 4 q + s of row j (rows past M repeat row M - 1: their
  // outputs are never stored).  The group sums of the rows come from the matrix
  // cores: the group's four A operands against a B of bf16 ones put
  // sum_k x[r][k] (exact products, fp32 sums) in every column of the tile, so each
  // lane receives the sums of its own output rows 4 q .. 4 q + 3 in place.
  uint4* xs = reinterpret_cast<uint4*>(lds_dyn + (size_t)wid * qm * 4 * 16);
  const int jr = min(j, a.M - 1);
  bf16x8 xa[KT][4];
  f32x4 zx[KT];        // -(128 + z) row sums (symmetric: z = 8), or the plain row sums
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
#pragma unroll
  for (int t = 0; t < KT; ++t) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = 4 * u + xr_row;
      if (u < qm) xs[r * 16 + ((xr_chunk ^ r) & 15)] = make_uint4(xr[t][u][0], xr[t][u][1], xr[t][u][2], xr[t][u][3]);
    }
    uint32_t xq[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 v = xs[jr * 16 + (((4 * q + s) ^ jr) & 15)];
      xq[s][0] = v.x; xq[s][1] = v.y; xq[s][2] = v.z; xq[s][3] = v.w;
    }
    f32x4 r = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t e[4];
      pair_activations(xq[s], e);
      xa[t][s] = __builtin_bit_cast(bf16x8, make_uint4(e[0], e[1], e[2], e[3]));
      r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[t][s], ones, r, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) zx[t][i] = SYM ? -136.0f * r[i] : r[i];
  }
  const uint32_t nib_mask = opaque_vgpr(0x000F000Fu);
  // operand lane j + 16 q takes the words of column j, chunk q from lane 4 j + q
  const int perm_addr = (4 * j + q) * 4;

  auto store = [&](int m, int n, float v) {
    if (a.partial)
      a.partial[((size_t)blockIdx.y * a.M + m) * a.N + n] = v;
    else
      a.Y[(size_t)m * a.N + n] = (uint16_t)f32_to_bf16_bits(v);
  };

  auto process = [&](const Batch& Bc, int b) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      f32x4 tile;
      if constexpr (SYM) {
        tile = zx[t];
      } else {
        const float c = (float)(128u + ((Bc.z >> (4 * ((g0 + t) & 7))) & 0xFu));
#pragma unroll
        for (int i = 0; i < 4; ++i) tile[i] = -c * zx[t][i];
      }
      uint32_t wt[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) wt[e] = (uint32_t)__builtin_amdgcn_ds_bpermute(perm_addr, (int)Bc.w[t][e]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t w = wt[s];
        const bf16x8 bw = __builtin_bit_cast(
            bf16x8, make_uint4(nibble_pair_m(w, 0, nib_mask), nibble_pair_m(w, 1, nib_mask),
                               nibble_pair_m(w, 2, nib_mask), nibble_pair_m(w, 3, nib_mask)));
        tile = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[t][s], bw, tile, 0, 0, 0);
      }
      const float sc = bf16_bits_to_f32(Bc.sc[t]);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(sc, tile[i], acc[i]);
    }
    if (a.nwk == 1) {
      const int n = n_first + b * n_step + j;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * q + i < a.M && n < a.N) store(4 * q + i, n, acc[i]);
    } else if (q < qm) {
      red[((slab * a.nwk + wave) * bpw + b) * (qm * 16) + lane] = acc;
    }
  };

  // NB blocks in flight: each buffer is refilled as soon as its block is computed
  // (straight-line code, so that every wait is for exactly the loads it needs)
#pragma unroll
  for (int b = 0; b < BPW; ++b) {
    process(B[b % NB], b);
    if (b + NB < BPW) load(b + NB, B[b % NB]);
    __builtin_amdgcn_sched_barrier(0);
  }

  if (a.nwk > 1) {
    __syncthreads();
    // element (slab, block, row m < M, column c): the tiles of the slab's waves in
    // wave order; consecutive threads take consecutive columns of a row
    const int E = bpw * a.M * kBlockCols;
    for (int e = threadIdx.x; e < a.rw * E; e += blockDim.x) {
      const int sl = e / E, r = e - sl * E;
      const int b = r / (a.M * kBlockCols), r2 = r - b * (a.M * kBlockCols);
      const int m = r2 / kBlockCols, c = r2 - m * kBlockCols;
      const int n = ((int)blockIdx.x * a.rw + sl) * kBlockCols + b * n_step + c;
      if (n < a.N) {
        const int src = c + 16 * (m >> 2);
        float s = 0.0f;
        for (int w = 0; w < a.nwk; ++w) s += red[((sl * a.nwk + w) * bpw + b) * (qm * 16) + src][m & 3];
        store(m, n, s);
      }
    }
  }
}

struct MfmaPlan {
  int kt, splits, gs, nwk;
};

// K split into `splits` ranges of gs groups (the last one may be shorter), each
// covered by nwk waves of kt groups.
MfmaPlan plan_mfma(int K) {
  const int G = K / kGroup;
  MfmaPlan p;
  p.kt = G <= 2 * max_waves(2) ? 2 : 4;
  const int chunks = (G + p.kt - 1) / p.kt;
  p.splits = (chunks + max_waves(p.kt) - 1) / max_waves(p.kt);
  p.nwk = (chunks + p.splits - 1) / p.splits;
  p.gs = p.nwk * p.kt;
  return p;
}

// Waves per workgroup the launch aims for when one slab needs fewer.
constexpr int kWgWaves = 4;
constexpr size_t kLdsPerCu = 160 * 1024;
constexpr size_t kMaxLds = kLdsPerCu;
constexpr size_t kDefaultLds = 64 * 1024;   // dynamic LDS a launch may take without raising the limit

// Allows an instantiation more than 64 KB of dynamic LDS (once per device).
template <int KT, int BPW, bool SYM, bool NT>
bool allow_large_lds() {
  static std::atomic<int> state[64];       // 0 not yet, 1 done, -1 failed
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  int st = state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    st = hipFuncSetAttribute(reinterpret_cast<const void*>(gemv_mfma_kernel<KT, BPW, SYM, NT>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsPerCu) == hipSuccess
             ? 1
             : -1;
    state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1;
}

// Resident workgroups per CU of one instantiation at a block size, from its
// registers alone (cached per block size); the LDS of the partial tiles is
// applied on top by the caller.
// Largest blocks per slab an instantiation takes: with four asymmetric groups per
// wave, more than two blocks would spill registers.
constexpr int max_bpw(int kt, bool sym) { return kt == 4 && !sym ? 2 : 8; }
constexpr int clamp_bpw(int kt, bool sym, int b) { return b < max_bpw(kt, sym) ? b : max_bpw(kt, sym); }

template <int KT, int BPW, bool SYM, bool NT>
int mfma_blocks_per_cu(int threads) {
  static std::atomic<int> cache[kMaxWavesAny + 1];
  const int slot = threads / kWave;
  int nblk = cache[slot].load(std::memory_order_relaxed);
  if (nblk == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nblk, gemv_mfma_kernel<KT, BPW, SYM, NT>, threads, 0) !=
            hipSuccess ||
        nblk < 1)
      nblk = 1;
    cache[slot].store(nblk, std::memory_order_relaxed);
  }
  return nblk;
}

int device_cu_count() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Blocks per slab: the fewest (1 to 8) with which one round of resident
// workgroups covers every block (the slabs take the blocks round-robin, so each
// holds that many or one less); when no count fits one round, the largest.
template <int KT, bool SYM, bool NT>
int launch_kt(MfmaArgs a, const MfmaPlan& p, hipStream_t stream) {
  const int rw = p.nwk >= kWgWaves ? 1 : kWgWaves / p.nwk;
  a.nwk = p.nwk;
  a.rw = rw;
  a.gs = p.gs;
  const int threads = p.nwk * rw * kWave;
  const long long nb = (a.N + kBlockCols - 1) / kBlockCols;
  const long long cus = device_cu_count();
  const int qm = (a.M + 3) / 4;
  auto lds = [&](int bpw) {
    const size_t xs = (size_t)rw * p.nwk * qm * 4 * 256;
    return xs + (p.nwk > 1 ? (size_t)rw * p.nwk * bpw * qm * 16 * sizeof(f32x4) : (size_t)0);
  };
  auto by_regs = [&](int bpw) {
    switch (bpw) {
      case 1: return mfma_blocks_per_cu<KT, clamp_bpw(KT, SYM, 1), SYM, NT>(threads);
      case 2: return mfma_blocks_per_cu<KT, clamp_bpw(KT, SYM, 2), SYM, NT>(threads);
      case 3: return mfma_blocks_per_cu<KT, clamp_bpw(KT, SYM, 3), SYM, NT>(threads);
      case 4: return mfma_blocks_per_cu<KT, clamp_bpw(KT, SYM, 4), SYM, NT>(threads);
      case 5: return mfma_blocks_per_cu<KT, clamp_bpw(KT, SYM, 5), SYM, NT>(threads);
      case 6: return mfma_blocks_per_cu<KT, clamp_bpw(KT, SYM, 6), SYM, NT>(threads);
      case 7: return mfma_blocks_per_cu<KT, clamp_bpw(KT, SYM, 7), SYM, NT>(threads);
      default: return mfma_blocks_per_cu<KT, clamp_bpw(KT, SYM, 8), SYM, NT>(threads);
    }
  };
  auto per_cu = [&](int bpw) {
    const size_t l = lds(bpw);
    const long long r = by_regs(bpw);
    return l ? std::min<long long>(r, (long long)(kLdsPerCu / l)) : r;
  };
  auto wgs = [&](int bpw) { return ((nb + bpw - 1) / bpw + rw - 1) / rw * p.splits; };
  int best = 1;
  for (int b = 1; b <= max_bpw(KT, SYM) && lds(b) <= kMaxLds; ++b) {
    best = b;
    if (wgs(b) <= cus * per_cu(b)) break;
  }
  const dim3 grid((unsigned)(((nb + best - 1) / best + rw - 1) / rw), (unsigned)p.splits);
  const size_t sh = lds(best);
  auto go = [&](auto kernel, auto allow) {
    if (sh > kDefaultLds && !allow()) return W4_ERR_HIP;
    hipLaunchKernelGGL(kernel, grid, dim3(threads), sh, stream, a);
    return W4_OK;
  };
  switch (best) {
    case 1: return go(gemv_mfma_kernel<KT, clamp_bpw(KT, SYM, 1), SYM, NT>, allow_large_lds<KT, clamp_bpw(KT, SYM, 1), SYM, NT>);
    case 2: return go(gemv_mfma_kernel<KT, clamp_bpw(KT, SYM, 2), SYM, NT>, allow_large_lds<KT, clamp_bpw(KT, SYM, 2), SYM, NT>);
    case 3: return go(gemv_mfma_kernel<KT, clamp_bpw(KT, SYM, 3), SYM, NT>, allow_large_lds<KT, clamp_bpw(KT, SYM, 3), SYM, NT>);
    case 4: return go(gemv_mfma_kernel<KT, clamp_bpw(KT, SYM, 4), SYM, NT>, allow_large_lds<KT, clamp_bpw(KT, SYM, 4), SYM, NT>);
    case 5: return go(gemv_mfma_kernel<KT, clamp_bpw(KT, SYM, 5), SYM, NT>, allow_large_lds<KT, clamp_bpw(KT, SYM, 5), SYM, NT>);
    case 6: return go(gemv_mfma_kernel<KT, clamp_bpw(KT, SYM, 6), SYM, NT>, allow_large_lds<KT, clamp_bpw(KT, SYM, 6), SYM, NT>);
    case 7: return go(gemv_mfma_kernel<KT, clamp_bpw(KT, SYM, 7), SYM, NT>, allow_large_lds<KT, clamp_bpw(KT, SYM, 7), SYM, NT>);
    default: return go(gemv_mfma_kernel<KT, clamp_bpw(KT, SYM, 8), SYM, NT>, allow_large_lds<KT, clamp_bpw(KT, SYM, 8), SYM, NT>);
  }
}

}  // namespace

// Which form runs a decode GEMV.  Measured on MI355X (kernel time per call,
// VALU form / MFMA form, asymmetric decode-block linears with warm caches and the
// symmetric 27B-shaped ones): K = 2048, N = 4096: 4.4 / 4.1 us at M = 3; K = 2048,
// N = 12288: 6.8 / 6.4 at M = 3; K = 5120, N = 17408: 15.6 / 12.1 at M = 3;
// K = 17408, N = 5120: 23.2 / 16.4 at M = 3 but 11.6 / 16.4 at M = 2 (the K split's
// second launch); K = 6144, N = 2048: 5.4 / 5.9 at M = 3, 6.2 / 5.9 at M = 4;
// K = 2048, N = 2048: 3.7 / 4.0 at M = 4, 4.4 / 4.1 at M = 6, 4.8 / 4.0 at M = 8.
bool gemv_use_mfma(int M, int K, int N) {
  if (M >= 5) return true;
  if (M >= 3 && N >= 4096) return true;
  return M == 4 && (long long)N * K / 2 >= (4LL << 20);
}

// Packed weights up to this size take the non-temporal hint (a measured rule).
// Cold at M = 8: 8 MB 5.93 -> 5.65 us, 16 and 24 MB unchanged, 20 MB (K = 5120)
// 9.3 -> 9.7 us, 30-45 MB 6-17% slower; the decode sweep's linears (2-12.6 MB)
// 7% faster at M = 3-16.
constexpr long long kMfmaNtMaxBytes = 16LL << 20;

size_t gemv_mfma_workspace_bytes(int M, int K, int N) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  const MfmaPlan p = plan_mfma(K);
  return p.splits > 1 ? (size_t)p.splits * M * N * sizeof(float) : 0;
}

int launch_gemv_mfma(const uint16_t* X, int M, int K, int N, const uint32_t* qweight, const uint16_t* scales,
                     const uint32_t* qzeros, int symmetric, uint16_t* Y, void* workspace, hipStream_t stream) {
  if (M == 0 || N == 0) return W4_OK;
  if (M > kBlockCols) return W4_ERR_UNSUPPORTED;
  if (int st = gemv_check_size(M, K, N)) return st;
  const MfmaPlan p = plan_mfma(K);
  MfmaArgs a{X, M, K, N, qweight, scales, qzeros, Y, p.splits > 1 ? static_cast<float*>(workspace) : nullptr,
             p.gs, p.nwk, 1};
  const bool nt = (long long)N * K / 2 <= kMfmaNtMaxBytes;
  int st;
  if (p.kt == 2)
    st = symmetric ? (nt ? launch_kt<2, true, true>(a, p, stream) : launch_kt<2, true, false>(a, p, stream))
                   : (nt ? launch_kt<2, false, true>(a, p, stream) : launch_kt<2, false, false>(a, p, stream));
  else
    st = symmetric ? (nt ? launch_kt<4, true, true>(a, p, stream) : launch_kt<4, true, false>(a, p, stream))
                   : (nt ? launch_kt<4, false, true>(a, p, stream) : launch_kt<4, false, false>(a, p, stream));
  if (st) return st;
  W4_CHECK_LAUNCH();
  if (p.splits > 1) {
    return launch_gemv_split_reduce(static_cast<const float*>(workspace), p.splits, (size_t)M * N, Y, stream);
  }
  return W4_OK;
}

}  // namespace w4
