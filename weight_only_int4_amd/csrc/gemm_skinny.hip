// Contraction Y = X W_hat^T for short activation blocks (17 <= M <= 48 rows) on the
// matrix cores, in one pass over the packed weights and without a prologue.
//
// Model card "GLM-5.2-QSRT-Fruit-Instruct", "Reproducible runtime": W4A16 serves
// prefill and every row count above the decode ceiling; model card
// "Qwen3.6-27B-W4A16": int4 group-128 weights against 16-bit activations.  At a
// few dozen rows the weights dominate the bytes (0.52 B per weight against
// M x 2 B per input channel of activations), so the kernel streams every packed
// word once and keeps the activations where no wave has to fetch them again.
//
// Design (CDNA4, wave64, v_mfma_f32_16x16x32_bf16):
//  * A workgroup is 16 waves.  Wave w owns one 128-channel group g (of its K
//    split) and holds all M activation rows of that group in registers as MFMA
//    A operands (RB = ceil(M / 16) = 2 or 3 row blocks x 4 steps of 32 channels), with the
//    rows' group sums (taken on the matrix cores against a B of bf16 ones).
//  * The workgroup streams a set of 16-column blocks.  Per block every wave
//    unpacks its group's 16 x 128 codes once (one packed word per lane and step,
//    traded into operand order with ds_bpermute), multiplies them with all RB
//    row blocks (128 + q as exact bf16 integers), starts each tile from the
//    zero-point term -(128 + z) rowsum and scales it by the group's bf16 scale.
//  * The waves' tiles of a block meet in LDS (two slots, one barrier per
//    block) and are added in wave order, one output per thread; with a K split
//    the fp32 sums go to the workspace and the split-order reduction of the
//    decode GEMV adds the splits.  Every sum has a fixed order: results are
//    reproducible bit for bit.
//  * Loads are range-checked buffer loads: rows past M, columns past N and
//    groups past the split read zeros (their tiles are 0) and touch no memory.
#include <algorithm>
#include <atomic>

#include "internal.hpp"

namespace w4 {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

namespace {

// Waves per workgroup = groups per K split (four per SIMD, at most 128 registers).
// Above 48 rows the activation operands and row sums (80 registers) leave too few
// for the rest, and 12 waves per workgroup measured slower than the tiled core.
constexpr int kSkWaves = 16;
constexpr int kSkCols = 16;         // columns per block

struct SkinnyArgs {
  const uint16_t* X;
  int M, K, N;
  const uint32_t* qweight;
  const uint16_t* scales;
  const uint32_t* qzeros;
  uint16_t* Y;
  float* partial;   // [splits][M][N] when splits > 1, else NULL
  int gs;           // groups per split (<= waves per workgroup)
  int nblk;         // blocks per workgroup, even; workgroup x takes x, x + gx, ...
};

template <int RB, bool SYM>
__global__ __launch_bounds__(kSkWaves * kWave) void gemm_skinny_kernel(SkinnyArgs a) {
  constexpr int NW = kSkWaves;
  // red[slot][wave][rb][i][lane]: element i of lane's tile of row block rb
  extern __shared__ float red[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int j = lane & 15, q = lane >> 4;
  const int G = a.K >> 7;
  const int g = (int)blockIdx.y * a.gs + wave;
  const bool gok = wave < a.gs && g < G;
  const int GW = (G + 7) >> 3;
  const uint32_t wrow = (uint32_t)a.K / 2u, srow = (uint32_t)G * 2u, zrow = (uint32_t)GW * 4u;
  const auto rwt = make_rsrc(a.qweight, (uint32_t)a.N * wrow);
  const auto rsc = make_rsrc(a.scales, (uint32_t)a.N * srow);
  const auto rzp = make_rsrc(SYM ? static_cast<const void*>(a.scales) : a.qzeros, SYM ? 0u : (uint32_t)a.N * zrow);
  const auto rx = make_rsrc(a.X, (uint32_t)a.M * (uint32_t)a.K * 2u);
  const int gx = (int)gridDim.x;
  // output: Y [M][N] bf16, or the split's fp32 partial [M][N] at element ypo of the workspace
  const uint32_t MN = (uint32_t)a.M * (uint32_t)a.N;
  const auto rout = a.partial ? make_rsrc(a.partial, (uint32_t)gridDim.y * MN * 4u) : make_rsrc(a.Y, MN * 2u);
  const uint32_t ypo = (uint32_t)blockIdx.y * MN;
  const uint32_t kw = gok ? (uint32_t)g * 64u + 16u * (uint32_t)(lane & 3) : kOob;
  const uint32_t ks = gok ? (uint32_t)g * 2u : kOob;
  const uint32_t kz = gok ? (uint32_t)(g >> 3) * 4u : kOob;

  struct Blk {
    u32x4 w;
    uint16_t sc;
    uint32_t z;
  };
  // Block b of this workgroup: columns (blockIdx.x + b gx) * 16 + 0..15.  Packed
  // words: lanes 4 c .. 4 c + 3 read the 64 bytes of column c in group g (four
  // consecutive lanes per cache line); scale and zero word: the lane's column j.
  auto load = [&](int b, Blk& B) {
    const int n0 = ((int)blockIdx.x + b * gx) * kSkCols;
    const uint32_t n = (uint32_t)min(n0 + j, a.N);
    const uint32_t nw = (uint32_t)min(n0 + (lane >> 2), a.N);
    // products kept in registers of their own: fused into 64-bit multiply-adds, they
    // would read the unused high half from a register a load in flight is writing
    B.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rwt, opaque_vgpr(nw * wrow) + kw, 0, 0));
    B.sc = __builtin_amdgcn_raw_buffer_load_b16(rsc, opaque_vgpr(n * srow) + ks, 0, 0);
    if constexpr (!SYM) B.z = __builtin_amdgcn_raw_buffer_load_b32(rzp, opaque_vgpr(n * zrow) + kz, 0, 0);
  };

  // Activations in operand order: row block rb, step s, lane (j, q) takes row
  // 16 rb + j, channels 128 g + 32 q + 8 s .. + 7 (one 16-byte load).
  uint32_t xr[RB][4][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = 16 * rb + j;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t xo = (gok && r < a.M)
                              ? ((uint32_t)r * (uint32_t)a.K + (uint32_t)g * 128u + 32u * (uint32_t)q + 8u * (uint32_t)s) * 2u
                              : kOob;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0);
      xr[rb][s][0] = v[0]; xr[rb][s][1] = v[1]; xr[rb][s][2] = v[2]; xr[rb][s][3] = v[3];
    }
  }
  // Blocks past the workgroup's count lie past N (every workgroup's count times gx
  // covers all blocks), so their loads are out of range: issued unconditionally,
  // they keep the count of loads in flight the same on every path.
  Blk B0, B1;
  load(0, B0);
  load(1, B1);
  __builtin_amdgcn_sched_barrier(0);

  // A operands (pair-arranged to match the unpacking order) and the row sums of
  // the group: the four A operands of a row block against a B of ones put
  // sum_k x[r][k] in every column, so lane (j, q) receives the sums of its own
  // output rows 16 rb + 4 q .. + 3.
  bf16x8 xa[RB][4];
  f32x4 zx[RB];
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    f32x4 r = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t e[4];
      pair_activations(xr[rb][s], e);
      xa[rb][s] = __builtin_bit_cast(bf16x8, make_uint4(e[0], e[1], e[2], e[3]));
      r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[rb][s], ones, r, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) zx[rb][i] = SYM ? -136.0f * r[i] : r[i];
  }
  const uint32_t nib_mask = opaque_vgpr(0x000F000Fu);
  const int perm_addr = (4 * j + q) * 4;     // operand lane (j, q) takes column j's chunk q from lane 4 j + q
  const int zsh = 4 * (g & 7);

  // this wave's tile of block b, scaled
  auto tiles = [&](const Blk& Bc, f32x4 (&t)[RB]) {
    if constexpr (SYM) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) t[rb] = zx[rb];
    } else {
      const float c = (float)(128u + ((Bc.z >> zsh) & 0xFu));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) t[rb][i] = -c * zx[rb][i];
    }
    uint32_t wt[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) wt[e] = (uint32_t)__builtin_amdgcn_ds_bpermute(perm_addr, (int)Bc.w[e]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t w = wt[s];
      const bf16x8 bw = __builtin_bit_cast(
          bf16x8, make_uint4(nibble_pair_m(w, 0, nib_mask), nibble_pair_m(w, 1, nib_mask),
                             nibble_pair_m(w, 2, nib_mask), nibble_pair_m(w, 3, nib_mask)));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) t[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[rb][s], bw, t[rb], 0, 0, 0);
    }
    const float sc = bf16_bits_to_f32(Bc.sc);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) t[rb][i] *= sc;
  };

  constexpr int kSlot = NW * RB * 4 * kWave;           // floats per slot
  // The outputs this thread adds up: index t = threadIdx.x + u NW 64 < RB 256 is
  // row block t >> 8, element (t >> 6) & 3, lane t & 63 of the tile.
  constexpr int NU = (RB * 256 + NW * kWave - 1) / (NW * kWave);

  // One block: this wave's tile from buffer Bc, refill Bc with block b + 2, the
  // tile into LDS slot b & 1, one barrier, then the block's outputs added over the
  // waves in wave order (one output per thread and pass).  Slot b & 1 is next
  // written in step b + 2, after the barrier of step b + 1, which every reader of
  // step b has passed.
  auto step = [&](int b, Blk& Bc) {
    f32x4 tl[RB];
    if (gok) {
      tiles(Bc, tl);
    } else {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) tl[rb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    load(b + 2, Bc);
    float* slot = red + (b & 1) * kSlot;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) slot[((wave * RB + rb) * 4 + i) * kWave + lane] = tl[rb][i];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int t = (int)threadIdx.x + u * NW * kWave;
      const int orb = t >> 8, ol = t & 63;
      const int om = 16 * orb + 4 * (ol >> 4) + ((t >> 6) & 3);
      const int n = ((int)blockIdx.x + b * gx) * kSkCols + (ol & 15);
      if (t >= RB * 256 || om >= a.M || n >= a.N) continue;
      float v[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) v[w] = slot[w * RB * 4 * kWave + t];
      float sum = v[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) sum += v[w];
      const uint32_t o = (uint32_t)om * (uint32_t)a.N + (uint32_t)n;
      if (a.partial)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sum), rout, (o + ypo) * 4u, 0, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_bits(sum), rout, o * 2u, 0, 0);
    }
  };
  // two named buffers (no indexed register arrays) take the blocks in turn; the
  // count is even (a block past N computes zeros and stores nothing)
  for (int b = 0; b < a.nblk; b += 2) {
    step(b, B0);
    step(b + 1, B1);
  }
}

struct SkinnyPlan {
  int splits, gs, nblk, gx;
};

int sk_cu_count() {
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

// K split into ranges of at most one group per wave, as even as possible;
// blocks per workgroup: the fewest (rounded up to even) with which one workgroup
// per CU covers every block of every split, so that all workgroups run in one
// round.
SkinnyPlan plan_skinny(int K, int N, int cus) {
  SkinnyPlan p;
  const int G = K / kGroup;
  p.splits = (G + kSkWaves - 1) / kSkWaves;
  p.gs = (G + p.splits - 1) / p.splits;
  p.splits = (G + p.gs - 1) / p.gs;
  const long long nb = (N + kSkCols - 1) / kSkCols;
  const long long per_split = std::max<long long>(1, cus / p.splits);
  p.nblk = (int)std::max<long long>(1, (nb + per_split - 1) / per_split);
  p.nblk += p.nblk & 1;
  p.gx = (int)((nb + p.nblk - 1) / p.nblk);
  return p;
}

template <int RB, bool SYM>
int launch_rb(const SkinnyArgs& a, const SkinnyPlan& p, hipStream_t stream) {
  const size_t lds = 2 * (size_t)kSkWaves * RB * 4 * kWave * sizeof(float);
  static std::atomic<int> state[64];       // 0 not yet, 1 done, -1 failed (per device)
  if (lds > 64 * 1024) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return W4_ERR_HIP;
    int st = state[dev].load(std::memory_order_relaxed);
    if (st == 0) {
      st = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_skinny_kernel<RB, SYM>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) == hipSuccess
               ? 1
               : -1;
      state[dev].store(st, std::memory_order_relaxed);
    }
    if (st != 1) return W4_ERR_HIP;
  }
  hipLaunchKernelGGL((gemm_skinny_kernel<RB, SYM>), dim3((unsigned)p.gx, (unsigned)p.splits), dim3(kSkWaves * kWave), lds,
                     stream, a);
  return W4_OK;
}

}  // namespace

bool gemm_use_skinny(int M, int K, int N) {
  return M > W4_GEMV_MAX_M && M <= kSkinnyMaxM && (long long)N * K / 2 < (1LL << 31) && 2LL * M * K < (1LL << 31);
}

size_t gemm_skinny_workspace_bytes(int M, int K, int N) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  const SkinnyPlan p = plan_skinny(K, N, 256);
  return p.splits > 1 ? (size_t)p.splits * M * N * sizeof(float) : 0;
}

int launch_gemm_skinny(const uint16_t* X, int M, int K, int N, const uint32_t* qweight, const uint16_t* scales,
                       const uint32_t* qzeros, int symmetric, uint16_t* Y, void* workspace, hipStream_t stream) {
  if (M == 0 || N == 0) return W4_OK;
  if (!gemm_use_skinny(M, K, N)) return W4_ERR_UNSUPPORTED;
  // the split count is a function of K alone, so the workspace size query (made
  // without a device) and the launch agree
  const SkinnyPlan p = plan_skinny(K, N, sk_cu_count());
  SkinnyArgs a{X, M, K, N, qweight, scales, qzeros, Y, p.splits > 1 ? static_cast<float*>(workspace) : nullptr,
               p.gs, p.nblk};
  const int rb = (M + 15) / 16;
  const bool sym = symmetric != 0;
  int st;
  switch (rb) {   // 17 to 48 rows: two or three row blocks
    case 2: st = sym ? launch_rb<2, true>(a, p, stream) : launch_rb<2, false>(a, p, stream); break;
    default: st = sym ? launch_rb<3, true>(a, p, stream) : launch_rb<3, false>(a, p, stream); break;
  }
  if (st) return st;
  W4_CHECK_LAUNCH();
  if (p.splits > 1) return launch_gemv_split_reduce(static_cast<const float*>(workspace), p.splits, (size_t)M * N, Y, stream);
  return W4_OK;
}

}  // namespace w4
