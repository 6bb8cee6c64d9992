// Decode contraction Y = X W_hat^T for 1 <= M <= 16 rows (W4A16 GEMV): the
// launcher, the vector-ALU form for the smallest batches (M <= 4; which form runs
// is gemv_use_mfma's measured rule, the matrix-core form being gemv_mfma.hip) and
// the reduction of K-split partials both forms share.
//
// Model card "GLM-5.2-QSRT-Fruit-Instruct", "Reproducible runtime": decode
// batches of at most 16 rows take their own path; model card
// "Qwen3.6-27B-W4A16", opening paragraph: int4 weights, 16-bit activations.
//
// Design of the vector-ALU form (CDNA4, wave64):
//  * A workgroup owns a contiguous slab of output rows (BPW batches of R rows)
//    and a range of input channels (all of K unless K is split over
//    grid.y).  Its waves split the channel range: every lane holds WPL packed
//    words (8 WPL channels inside one 128-group) at a fixed position, with the
//    matching activations in registers as bf16 pairs (x_j, x_j+4) and their fp32
//    sum.
//  * Each wave streams its slice of every row of the slab: per row and lane one
//    16-byte load of packed words (WPL = 4 words, 32 channels), one 2-byte scale
//    load and (asymmetric) one 4-byte zero-word load.  These are buffer loads: an offset past the end of
//    the buffer returns 0 without a memory access, so lanes past the channel
//    range and rows past N need neither branches nor clamped re-reads.  The
//    batch loop is unrolled (BPW is a template parameter): straight-line code in
//    which NB batches are in flight (a buffer is refilled as soon as its batch
//    is computed) and every wait is for exactly the loads it needs.
//  * A word expands into four pairs of exact bf16 integers 128+q (shift, AND-OR);
//    v_dot2_f32_bf16 accumulates in fp32, and the zero point and scale are applied
//    once per lane and row:
//      sum_k x_k (q_k - z) sc = sc * (-(128 + z) sum_k x_k + sum_k x_k (128 + q_k)).
//  * The R*M partials of a batch are reduced across the wave by a transposing
//    butterfly of lane swaps (permlane 32/16) and DPP permutations: no LDS.  With
//    one wave per row the results are stored at once; otherwise every wave parks
//    its per-row sums in LDS and the workgroup adds them in wave order after the
//    last batch (one barrier per workgroup).
#include <atomic>

#include "internal.hpp"

namespace w4 {

struct GemvArgs {
  const uint16_t* X;
  int K, N;
  const uint32_t* qweight;
  const uint16_t* scales;
  const uint32_t* qzeros;
  uint16_t* Y;
  float* partial;       // [splits][M][N] when splits > 1
  int wps;              // packed words per split (multiple of WPL)
  int nwk;              // waves covering one slab's channel range
  int rw;               // slabs per workgroup (one group of nwk waves each)
};

// The packed words are read once per launch, each wave load covering whole cache
// lines, so they take the non-temporal hint (measured: decode sweep 3.96 -> 3.69 us
// per launch at M = 1, 4.82 -> 4.41 at M = 2; cold 27B shapes at M = 1 11.5 -> 10.9
// and 11.8 -> 11.2 us); so do the scales (sweep 3.68 -> 3.59 us, cold unchanged).
template <int WPL>
__device__ __forceinline__ void load_words(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* w) {
  static_assert(WPL == 4, "one 16-byte load of four packed words per lane and row");
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kLoadNt);
  w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// keep + the partner's `send`, partners paired by lane bit B:
//   B = 3, 2: the mirrors l <-> 15 - l, l <-> 7 - l inside each 16-lane row;
//   B = 1, 0: l ^ 2, l ^ 1 (quad permutations).
template <int B>
__device__ __forceinline__ float pair_sum(float keep, float send) {
  if constexpr (B == 3) return keep + dpp<0x140>(send);        // row_mirror
  else if constexpr (B == 2) return keep + dpp<0x141>(send);   // row_half_mirror
  else if constexpr (B == 1) return keep + dpp<0x4E>(send);    // quad_perm [2,3,0,1]
  else return keep + dpp<0xB1>(send);                          // quad_perm [1,0,3,2]
}

// Transposing butterfly over the 64 lanes for V (power of two) values per lane,
// one stage per lane bit B = 5 .. 0 (partners 32 apart, 16 apart, then the
// in-row pairings of pair_sum).  The pairing masks (32, 16, 15, 7, 2, 1) span the
// 6 lane bits and each flips the bit its stage splits on.  While more than one
// value remains, a lane keeps the half selected by its bit B (the upper half when
// set) and adds the partner's copy of that half; then plain sums.  Afterwards
// value index lane >> (6 - log2 V), summed over all lanes, is in every lane.
template <int V, int B>
struct WaveReduce {
  __device__ static __forceinline__ void run(float* a, int lane) {
    if constexpr (B >= 0) {
      if constexpr (V > 1) {
        constexpr int H = V / 2;
        if constexpr (B >= 4) {
#pragma unroll
          for (int i = 0; i < H; ++i) a[i] = B == 5 ? swap_sum32(a[i], a[i + H]) : swap_sum16(a[i], a[i + H]);
        } else {
          const bool upper = (lane >> B) & 1;
#pragma unroll
          for (int i = 0; i < H; ++i) {
            const float send = upper ? a[i] : a[i + H];
            const float keep = upper ? a[i + H] : a[i];
            a[i] = pair_sum<B>(keep, send);
          }
        }
        WaveReduce<H, B - 1>::run(a, lane);
      } else {
        if constexpr (B == 5) a[0] = swap_sum32(a[0], a[0]);
        else if constexpr (B == 4) a[0] = swap_sum16(a[0], a[0]);
        else a[0] = pair_sum<B>(a[0], a[0]);
        WaveReduce<1, B - 1>::run(a, lane);
      }
    }
  }
};

constexpr int pow2_ceil(int v) { return v <= 1 ? 1 : 2 * pow2_ceil((v + 1) / 2); }
constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// Up to 16 waves per workgroup for M <= 2 (128 VGPRs per lane), 8 above (256).
constexpr int gemv_max_waves(int M) { return M <= 2 ? 16 : 8; }

template <int M, int WPL, int R, int BPW, int NB, bool SYM>
__global__ __launch_bounds__(gemv_max_waves(M) * 64) void gemv_kernel(GemvArgs a) {
  constexpr int V = R * M;
  constexpr int VP = pow2_ceil(V);
  constexpr int LOGV = ilog2(VP);
  __shared__ float red[16][BPW * R * M];    // per-row sums of every wave when nwk > 1

  const int lane = threadIdx.x & (kWave - 1);
  const int nw = a.nwk;
  const int slab = threadIdx.x / (nw * kWave);       // this wave's slab within the workgroup
  const int t = threadIdx.x - slab * nw * kWave;     // thread index within the slab's waves
  const int wave = t >> 6;
  const int words = a.K >> 3;
  const int G = a.K >> 7;
  const int GW = (G + 7) >> 3;
  // this lane's WPL words start at word t WPL of the split; byte offsets inside
  // one row of each array, out of range when they lie past the split or past K
  const int wl = blockIdx.y * a.wps + t * WPL;
  const bool active = (t * WPL < a.wps) && (wl < words);
  const int g = active ? wl >> 4 : 0;
  const int zsh = 4 * (g & 7);
  const uint32_t kw = active ? (uint32_t)wl * 4u : kOob;
  const uint32_t ks = active ? (uint32_t)g * 2u : kOob;
  const uint32_t kz = active ? (uint32_t)(g >> 3) * 4u : kOob;
  const uint32_t kx = active ? (uint32_t)wl * 16u : kOob;
  const uint32_t wrow = (uint32_t)words * 4u, srow = (uint32_t)G * 2u, zrow = (uint32_t)GW * 4u;
  const auto rw = make_rsrc(a.qweight, (uint32_t)a.N * wrow);
  const auto rs = make_rsrc(a.scales, (uint32_t)a.N * srow);
  const auto rz = make_rsrc(SYM ? static_cast<const void*>(a.scales) : a.qzeros, SYM ? 0u : (uint32_t)a.N * zrow);
  const auto rx = make_rsrc(a.X, (uint32_t)(M * a.K) * 2u);
  const int n_first = (blockIdx.x * a.rw + slab) * BPW * R;   // first row of the slab

  struct Batch {
    uint32_t w[R][WPL];
    uint16_t sc[R];     // kept 16-bit: widening at the load would wait for it right there
    uint32_t z[R];
  };
  // batch i of the slab; rows past N read nothing
  auto load = [&](int i, Batch& B) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t row = (uint32_t)min(n_first + i * R + r, a.N);
      load_words<WPL>(rw, row * wrow + kw, B.w[r]);
      B.sc[r] = __builtin_amdgcn_raw_buffer_load_b16(rs, row * srow + ks, 0, kLoadNt);
      if constexpr (!SYM) B.z[r] = __builtin_amdgcn_raw_buffer_load_b32(rz, row * zrow + kz, 0, 0);
    }
  };

  // Prologue: every load -- this lane's activations, then the first NB batches --
  // is issued before anything waits for one (the scheduling fence keeps the compiler
  // from sinking each load next to its use, one memory round trip per load).
  uint32_t xr[M][WPL][4];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)(m * a.K) * 2u + kx + 16u * i, 0, 0);
      xr[m][i][0] = v[0]; xr[m][i][1] = v[1]; xr[m][i][2] = v[2]; xr[m][i][3] = v[3];
    }
  __builtin_amdgcn_sched_barrier(0);
  Batch B[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
    if (i < BPW) load(i, B[i]);
  __builtin_amdgcn_sched_barrier(0);

  uint32_t xp[M][WPL][4];
  float xs[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    xs[m] = 0.0f;
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
      pair_activations(xr[m][i], xp[m][i]);
#pragma unroll
      for (int q = 0; q < 4; ++q)   // the pair's sum: one dot product with (1, 1) (exact products, fp32 sums)
        xs[m] = dot2_bf16(xr[m][i][q], 0x3F803F80u, xs[m]);
    }
  }
  // symmetric: the zero-point term -(128 + 8) sum_k x_k is the same for every row
  float zx[M];
#pragma unroll
  for (int m = 0; m < M; ++m) zx[m] = -136.0f * xs[m];
  // the nibble mask stays in a register, so AND and OR fuse into one v_and_or_b32
  const uint32_t nib_mask = opaque_vgpr(0x000F000Fu);

  auto store = [&](int m, int n, float v) {
    if (a.partial)
      a.partial[((size_t)blockIdx.y * M + m) * a.N + n] = v;
    else
      a.Y[(size_t)m * a.N + n] = (uint16_t)f32_to_bf16_bits(v);
  };

  auto process = [&](const Batch& Bc, int i) {
    float part[VP];
#pragma unroll
    for (int v = V; v < VP; ++v) part[v] = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float sc = bf16_bits_to_f32(Bc.sc[r]);
      const float zc = SYM ? 0.0f : (float)(128u + ((Bc.z[r] >> zsh) & 0xFu));
      uint32_t bp[WPL][4];
#pragma unroll
      for (int w = 0; w < WPL; ++w)
#pragma unroll
        for (int p = 0; p < 4; ++p) bp[w][p] = nibble_pair_m(Bc.w[r][w], p, nib_mask);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float acc = SYM ? zx[m] : -zc * xs[m];
#pragma unroll
        for (int w = 0; w < WPL; ++w)
#pragma unroll
          for (int p = 0; p < 4; ++p) acc = dot2_bf16(xp[m][w][p], bp[w][p], acc);
        part[r * M + m] = sc * acc;
      }
    }
    WaveReduce<VP, 5>::run(part, lane);
    const int idx = lane >> (6 - LOGV);
    const bool writer = (lane & ((kWave >> LOGV) - 1)) == 0 && idx < V;
    const int rloc = i * R + idx / M;
    const int m = idx % M;
    if (nw == 1) {
      const int n = n_first + rloc;
      if (writer && n < a.N) store(m, n, part[0]);
    } else if (writer) {
      red[slab * nw + wave][rloc * M + m] = part[0];
    }
  };

#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    process(B[i % NB], i);
    if (i + NB < BPW) load(i + NB, B[i % NB]);
    __builtin_amdgcn_sched_barrier(0);
  }

  if (nw > 1) {
    __syncthreads();
    constexpr int E = BPW * R * M;
    for (int e = threadIdx.x; e < a.rw * E; e += blockDim.x) {
      const int sl = e / E, i = e - sl * E;
      const int n = (blockIdx.x * a.rw + sl) * BPW * R + i / M;
      if (n < a.N) {
        float s = 0.0f;
        for (int w = 0; w < nw; ++w) s += red[sl * nw + w][i];
        store(i % M, n, s);
      }
    }
  }
}

// Y[i] = bf16(sum over splits k of partial[k * stride + i]) for i < count, fp32 in
// split order.  Four outputs per thread; the loads of up to eight splits are issued
// before their adds (a dependent load per split made the kernel one memory round
// trip per split long).
constexpr int kReduceBatch = 8;
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* partial, int splits, size_t stride,
                                                           size_t count, uint16_t* Y) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= count) return;
  if (i + 4 <= count && (stride & 3) == 0) {
    float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int k0 = 0; k0 < splits; k0 += kReduceBatch) {
      float4 v[kReduceBatch];
#pragma unroll
      for (int u = 0; u < kReduceBatch; ++u)
        if (k0 + u < splits) v[u] = *reinterpret_cast<const float4*>(partial + (size_t)(k0 + u) * stride + i);
#pragma unroll
      for (int u = 0; u < kReduceBatch; ++u)
        if (k0 + u < splits) {
          s.x = k0 + u == 0 ? v[u].x : s.x + v[u].x;
          s.y = k0 + u == 0 ? v[u].y : s.y + v[u].y;
          s.z = k0 + u == 0 ? v[u].z : s.z + v[u].z;
          s.w = k0 + u == 0 ? v[u].w : s.w + v[u].w;
        }
    }
    *reinterpret_cast<uint2*>(Y + i) = make_uint2(f32_to_bf16_bits(s.x) | (f32_to_bf16_bits(s.y) << 16),
                                                  f32_to_bf16_bits(s.z) | (f32_to_bf16_bits(s.w) << 16));
  } else {
    const size_t e = count - i < 4 ? count - i : 4;
    for (size_t j = 0; j < e; ++j) {
      float s = 0.0f;
      for (int k0 = 0; k0 < splits; k0 += kReduceBatch) {
        float v[kReduceBatch];
#pragma unroll
        for (int u = 0; u < kReduceBatch; ++u)
          if (k0 + u < splits) v[u] = partial[(size_t)(k0 + u) * stride + i + j];
#pragma unroll
        for (int u = 0; u < kReduceBatch; ++u)
          if (k0 + u < splits) s = k0 + u == 0 ? v[u] : s + v[u];
      }
      Y[i + j] = (uint16_t)f32_to_bf16_bits(s);
    }
  }
}

namespace {

// Words per lane, rows per batch and batches in flight of the vector-ALU form,
// which serves M <= 4 (the activations of one lane take 16 M registers).
constexpr int kGemvMaxM = 4;
constexpr int gemv_wpl(int M) { return 4; }
constexpr int gemv_rows(int M) { return 2; }
constexpr int gemv_nb(int M) { return 2; }

struct GemvPlan {
  int wpl, nw, splits, wps;
};

// Waves per workgroup the launch aims for when one slab needs fewer: slabs of
// a workgroup share its dispatch (a K = 2048 GEMV is one wave per slab).
#ifndef W4_GEMV_WG_WAVES
#define W4_GEMV_WG_WAVES 4
#endif
constexpr int kGemvWgWaves = W4_GEMV_WG_WAVES;

// K split into `splits` ranges of wps words, each covered by nw waves.
GemvPlan plan_gemv(int M, int K) {
  GemvPlan p;
  p.wpl = gemv_wpl(M);
  const int words = K / 8;
  const int max_wps = gemv_max_waves(M) * kWave * p.wpl;
  p.splits = (words + max_wps - 1) / max_wps;
  const int wps = (words + p.splits - 1) / p.splits;
  p.wps = (wps + p.wpl - 1) / p.wpl * p.wpl;
  p.nw = (p.wps / p.wpl + kWave - 1) / kWave;
  return p;
}

// Per-device and per-instantiation caches of launch-plan queries.  Host threads
// may launch concurrently: the slots are atomics, and a slot filled twice by
// racing first calls gets the same value both times.
int device_cus() {
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

template <int M, int BPW, bool SYM>
constexpr auto gemv_instance() {
  static_assert(M >= 1 && M <= kGemvMaxM, "larger batches take the matrix-core form");
  return gemv_kernel<M, gemv_wpl(M), gemv_rows(M), BPW, gemv_nb(M), SYM>;
}

// Resident workgroups per CU of one instantiation at a block size (cached).
template <int M, int BPW, bool SYM>
int gemv_blocks_per_cu(int threads) {
  static std::atomic<int> cache[17];
  const int slot = threads / kWave;
  int nblk = cache[slot].load(std::memory_order_relaxed);
  if (nblk == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nblk, gemv_instance<M, BPW, SYM>(), threads, 0) != hipSuccess ||
        nblk < 1)
      nblk = 1;
    cache[slot].store(nblk, std::memory_order_relaxed);
  }
  return nblk;
}

// Batches per workgroup.  Among 1, 2, 3, 4, 5, 6 and 8, those with which one round
// of resident workgroups covers all rows; the fewest of them, unless another
// gives the busiest CU at least 10% fewer batches (workgroups land unevenly on
// the CUs when their count is not a multiple of the CU count: K = 17408,
// N = 5120, M = 1 takes 5 -- 512 workgroups, two per CU -- over 4, whose 640
// left half the CUs a third one: 12.1 -> 11.5 us).  When none fits, 4, 8 or 16,
// whichever gives the busiest CU the least work: ceil(workgroups / CUs) x
// (batches + 2), the 2 standing for a workgroup's activation loads (measured at
// M = 8: K = 5120, N = 17408 takes 8 -- 544 workgroups of 16 batches left 32 CUs
// a third one -- and K = 17408, N = 5120 keeps 16).
template <int M, bool SYM>
void launch_m(GemvArgs a, const GemvPlan& p, hipStream_t stream) {
  constexpr int R = gemv_rows(M);
  // slabs per workgroup: several slabs share a workgroup when one slab needs few waves
  const int rw = p.nw >= kGemvWgWaves ? 1 : kGemvWgWaves / p.nw;
  a.nwk = p.nw;
  a.rw = rw;
  const int threads = p.nw * rw * kWave;
  const long long nb = (a.N + R - 1) / R;
  const long long cus = device_cus();
  auto wgs = [&](int bpw) { return ((nb + bpw - 1) / bpw + rw - 1) / rw * p.splits; };
  auto busiest = [&](int bpw) { return (wgs(bpw) + cus - 1) / cus * bpw; };
  auto per_cu = [&](int bpw) {
    switch (bpw) {
      case 1: return gemv_blocks_per_cu<M, 1, SYM>(threads);
      case 2: return gemv_blocks_per_cu<M, 2, SYM>(threads);
      case 3: return gemv_blocks_per_cu<M, 3, SYM>(threads);
      case 4: return gemv_blocks_per_cu<M, 4, SYM>(threads);
      case 5: return gemv_blocks_per_cu<M, 5, SYM>(threads);
      case 6: return gemv_blocks_per_cu<M, 6, SYM>(threads);
      default: return gemv_blocks_per_cu<M, 8, SYM>(threads);
    }
  };
  int first = 0, best = 0;
  for (int b : {1, 2, 3, 4, 5, 6, 8}) {
    if (wgs(b) > cus * per_cu(b)) continue;
    if (first == 0)
      first = best = b;
    else if (busiest(b) < busiest(best))
      best = b;
  }
  if (first != 0 && 10 * busiest(best) > 9 * busiest(first)) best = first;
  if (best == 0) {
    auto load = [&](int bpw) { return (wgs(bpw) + cus - 1) / cus * (bpw + 2); };
    best = load(4) < load(8) && load(4) < load(16) ? 4 : (load(8) < load(16) ? 8 : 16);
  }
  const dim3 grid((unsigned)(((nb + best - 1) / best + rw - 1) / rw), (unsigned)p.splits);
  switch (best) {
    case 1: hipLaunchKernelGGL((gemv_instance<M, 1, SYM>()), grid, dim3(threads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((gemv_instance<M, 2, SYM>()), grid, dim3(threads), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((gemv_instance<M, 3, SYM>()), grid, dim3(threads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((gemv_instance<M, 4, SYM>()), grid, dim3(threads), 0, stream, a); break;
    case 5: hipLaunchKernelGGL((gemv_instance<M, 5, SYM>()), grid, dim3(threads), 0, stream, a); break;
    case 6: hipLaunchKernelGGL((gemv_instance<M, 6, SYM>()), grid, dim3(threads), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((gemv_instance<M, 8, SYM>()), grid, dim3(threads), 0, stream, a); break;
    default: hipLaunchKernelGGL((gemv_instance<M, 16, SYM>()), grid, dim3(threads), 0, stream, a); break;
  }
}

template <int M>
void launch_sym(const GemvArgs& a, const GemvPlan& p, bool symmetric, hipStream_t stream) {
  if (symmetric)
    launch_m<M, true>(a, p, stream);
  else
    launch_m<M, false>(a, p, stream);
}

}  // namespace

// The kernels' buffer loads take 32-bit byte offsets: the packed weights (N K / 2
// bytes) and the 16 activation rows either form addresses (2 x 16 x K bytes) stay
// below 2^31.
int gemv_check_size(int M, int K, int N) {
  (void)M;
  if ((long long)N * K / 2 >= (1LL << 31) || 2LL * W4_GEMV_MAX_M * K >= (1LL << 31)) return W4_ERR_SHAPE;
  return W4_OK;
}

size_t gemv_workspace_bytes(int M, int K, int N) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  if (gemv_use_mfma(M, K, N)) return gemv_mfma_workspace_bytes(M, K, N);
  const GemvPlan p = plan_gemv(M, K);
  return p.splits > 1 ? (size_t)p.splits * M * N * sizeof(float) : 0;
}

int launch_gemv(const uint16_t* X, int M, int K, int N, const uint32_t* qweight,
                const uint16_t* scales, const uint32_t* qzeros, int symmetric, uint16_t* Y,
                void* workspace, hipStream_t stream) {
  if (M == 0 || N == 0) return W4_OK;
  if (M <= W4_GEMV_MAX_M && gemv_use_mfma(M, K, N))
    return launch_gemv_mfma(X, M, K, N, qweight, scales, qzeros, symmetric, Y, workspace, stream);
  if (int st = gemv_check_size(M, K, N)) return st;
  const GemvPlan p = plan_gemv(M, K);
  GemvArgs a{X, K, N, qweight, scales, qzeros, Y, p.splits > 1 ? static_cast<float*>(workspace) : nullptr, p.wps};
  const bool sym = symmetric != 0;
  switch (M) {
    case 1: launch_sym<1>(a, p, sym, stream); break;
    case 2: launch_sym<2>(a, p, sym, stream); break;
    case 3: launch_sym<3>(a, p, sym, stream); break;
    case 4: launch_sym<4>(a, p, sym, stream); break;
    default: return W4_ERR_UNSUPPORTED;   // M >= 5 always takes the matrix-core form
  }
  W4_CHECK_LAUNCH();
  if (p.splits > 1) {
    return launch_gemv_split_reduce(static_cast<const float*>(workspace), p.splits, (size_t)M * N, Y, stream);
  }
  return W4_OK;
}

int launch_split_reduce(const float* partial, int splits, size_t stride, size_t count, uint16_t* Y,
                        hipStream_t stream) {
  const size_t blocks = (count + 1023) / 1024;
  if (blocks > 0x7FFFFFFFu) return W4_ERR_SHAPE;
  hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, partial, splits, stride, count,
                     Y);
  W4_CHECK_LAUNCH();
  return W4_OK;
}

int launch_gemv_split_reduce(const float* partial, int splits, size_t MN, uint16_t* Y, hipStream_t stream) {
  return launch_split_reduce(partial, splits, MN, MN, Y, stream);
}

}  // namespace w4
