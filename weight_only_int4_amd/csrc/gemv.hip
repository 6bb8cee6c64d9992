// Decode contraction Y = X W_hat^T for 1 <= M <= 16 rows (W4A16 GEMV).
//
// Model card "GLM-5.2-QSRT-Fruit-Instruct", "Reproducible runtime": decode
// batches of at most 16 rows take their own path; model card
// "Qwen3.6-27B-W4A16", opening paragraph: int4 weights, 16-bit activations.
//
// Design (CDNA4, wave64, VALU): a workgroup owns a contiguous slice of input
// channels ("split") and a run of output rows.  Each lane keeps its WPL words
// (8*WPL channels, inside one 128-group) of activations in registers as bf16
// pairs, then streams the matching packed words of every row with one 16/8/4-byte
// coalesced load, turns each word into four bf16 pairs of exact integers 128+q
// with one shift and one AND-OR, and accumulates v_dot2_f32_bf16 products in fp32.
// The zero point and scale are applied once per lane and row:
//   sum_k x_k (q_k - z) sc = sc * (sum_k x_k (128 + q_k) - (128 + z) sum_k x_k).
// Lane partials are reduced across the wavefront (transposing butterfly, one
// value per lane at the end) and across waves through LDS, in a fixed order.
#include "internal.hpp"

namespace w4 {

struct GemvArgs {
  const uint16_t* X;
  int K, N;
  const uint32_t* qweight;
  const uint16_t* scales;
  const uint32_t* qzeros;
  int symmetric;
  uint16_t* Y;
  float* partial;       // [splits][M][N] when splits > 1
  int wps;              // packed words per split (multiple of WPL)
};

// Butterfly reduction of V values per lane across the 64 lanes of a wave.
// The first log2(V) steps halve the values each lane carries (each lane keeps
// the half selected by its lane bit and adds its partner's copy); the rest are
// plain xor sums.  Afterwards a[0] of every lane holds the wave total of value
// index lane / (64 / V).
template <int V, int O>
struct WaveReduce {
  __device__ static __forceinline__ void run(float* a, int lane) {
    if constexpr (V > 1) {
      constexpr int H = V / 2;
      const bool upper = (lane & O) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float send = upper ? a[i] : a[i + H];
        const float keep = upper ? a[i + H] : a[i];
        a[i] = keep + __shfl_xor(send, O, kWave);
      }
      WaveReduce<H, O / 2>::run(a, lane);
    } else if constexpr (O >= 1) {
      a[0] += __shfl_xor(a[0], O, kWave);
      WaveReduce<1, O / 2>::run(a, lane);
    }
  }
};

constexpr int pow2_ceil(int v) { return v <= 1 ? 1 : 2 * pow2_ceil((v + 1) / 2); }

template <int WPL>
struct WordVec;
template <>
struct WordVec<4> {
  __device__ static __forceinline__ void load(const uint32_t* p, uint32_t* w) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
};
template <>
struct WordVec<2> {
  __device__ static __forceinline__ void load(const uint32_t* p, uint32_t* w) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  }
};
template <>
struct WordVec<1> {
  __device__ static __forceinline__ void load(const uint32_t* p, uint32_t* w) { w[0] = *p; }
};

// A workgroup owns one K split and walks row batches b = blockIdx.x,
// blockIdx.x + gridDim.x, ... (R rows each); the grid is sized to the number of
// workgroups the device holds at once.  The lane's activations are loaded once.
// The packed words, scales and zero words of the next batch are loaded (from
// clamped, always-valid addresses, without branches around the loads) before
// the current batch is computed, so every wave keeps a batch of loads in flight
// while it computes and reduces.  Rows past N are computed on clamped data and
// never stored; lanes past the end of K carry zero activations.
template <int M, int WPL, int R>
struct GemvBatch {
  uint32_t w[R][WPL];
  uint16_t scb[R];      // kept 16-bit: widening at the load would wait for it right there
  uint32_t zw[R];
};

template <int M, int WPL, int R>
__device__ __forceinline__ void gemv_load_batch(const GemvArgs& a, int b, int wb, int g, int words, int G, int GW,
                                                GemvBatch<M, WPL, R>& B) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = min(b * R + r, a.N - 1);
    WordVec<WPL>::load(a.qweight + (size_t)n * words + wb, B.w[r]);
    B.scb[r] = a.scales[(size_t)n * G + g];
    // branch-free: symmetric weights read (and ignore) the first scale word, so
    // every batch issues the same loads and the waits on them stay exact
    const uint32_t* zp = a.symmetric ? reinterpret_cast<const uint32_t*>(a.scales)
                                     : a.qzeros + (size_t)n * GW + (g >> 3);
    B.zw[r] = *zp;
  }
}

// Up to 16 waves per workgroup for M <= 2 (128 VGPRs per lane), 8 above (256).
constexpr int gemv_max_waves(int M) { return M <= 2 ? 16 : 8; }

template <int M, int WPL, int R>
__global__ __launch_bounds__(gemv_max_waves(M) * 64) void gemv_kernel(GemvArgs a) {
  constexpr int V = R * M;
  constexpr int VP = pow2_ceil(V);
  constexpr int SPREAD = kWave / VP;          // lanes per reduced value
  __shared__ float red[2][16][VP];

  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t >> 6;
  const int nw = blockDim.x >> 6;
  const int words = a.K >> 3;
  const int G = a.K >> 7;
  const int GW = (G + 7) >> 3;
  const int wb_raw = blockIdx.y * a.wps + t * WPL;
  const bool active = (t * WPL < a.wps) && (wb_raw < words);
  const int wb = active ? wb_raw : 0;
  const int g = wb >> 4;
  const int nb = (a.N + R - 1) / R;
  int b = blockIdx.x;

  // Every load of the prologue -- this lane's activations, then the first batch --
  // is issued before anything waits for one (the scheduling fence keeps the
  // compiler from sinking each load next to its use, which would cost one memory
  // round trip per load).
  uint4 xr[M][WPL];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int i = 0; i < WPL; ++i)
      xr[m][i] = *reinterpret_cast<const uint4*>(a.X + (size_t)m * a.K + (size_t)(wb + i) * 8);
  GemvBatch<M, WPL, R> B0, B1;
  gemv_load_batch(a, b, wb, g, words, G, GW, B0);
  __builtin_amdgcn_sched_barrier(0);

  // this lane's activations as (x_j, x_j+4) bf16 pairs, and their fp32 sums
  uint32_t xp[M][WPL][4];
  float xs[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    xs[m] = 0.0f;
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
      const uint4 v = xr[m][i];
      uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) d[q] = active ? d[q] : 0u;
      pair_activations(d, xp[m][i]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xs[m] += __uint_as_float(d[q] << 16) + __uint_as_float(d[q] & 0xFFFF0000u);
    }
  }

  // compute batch `bb` from registers `B`, reduce and store; `par` selects the LDS buffer
  auto process = [&](const GemvBatch<M, WPL, R>& Bc, int bb, int par) {
    float part[VP];
#pragma unroll
    for (int v = V; v < VP; ++v) part[v] = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float sc = bf16_bits_to_f32(Bc.scb[r]);
      const float zc = a.symmetric ? 136.0f : (float)(128u + ((Bc.zw[r] >> (4 * (g & 7))) & 0xFu));
      uint32_t bp[WPL][4];
#pragma unroll
      for (int i = 0; i < WPL; ++i)
#pragma unroll
        for (int p = 0; p < 4; ++p) bp[i][p] = nibble_pair(Bc.w[r][i], p);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < WPL; ++i)
#pragma unroll
          for (int p = 0; p < 4; ++p) acc = dot2_bf16(xp[m][i][p], bp[i][p], acc);
        part[r * M + m] = sc * (acc - zc * xs[m]);
      }
    }
    WaveReduce<VP, 32>::run(part, lane);
    const int idx = lane / SPREAD;
    const bool writer = (lane % SPREAD) == 0 && idx < V;
    const int n0 = bb * R;
    if (nw == 1) {
      const int n = n0 + idx / M, m = idx % M;
      if (writer && n < a.N) {
        if (a.partial)
          a.partial[((size_t)blockIdx.y * M + m) * a.N + n] = part[0];
        else
          a.Y[(size_t)m * a.N + n] = (uint16_t)f32_to_bf16_bits(part[0]);
      }
    } else {
      // two LDS buffers alternate between batches, so one barrier per batch suffices
      if (writer) red[par][wave][idx] = part[0];
      __syncthreads();
      if (t < V) {
        const int n = n0 + t / M, m = t % M;
        float sum = 0.0f;
        for (int ww = 0; ww < nw; ++ww) sum += red[par][ww][t];
        if (n < a.N) {
          if (a.partial)
            a.partial[((size_t)blockIdx.y * M + m) * a.N + n] = sum;
          else
            a.Y[(size_t)m * a.N + n] = (uint16_t)f32_to_bf16_bits(sum);
        }
      }
    }
  };

  const int step = gridDim.x;
  // The next batch's loads are issued (and fenced) before the current batch is
  // computed.  They are issued unconditionally (past the last batch they repeat
  // it): with a branch around them the compiler can no longer count which loads
  // are outstanding and waits for all of them before computing.
  while (b < nb) {
    gemv_load_batch(a, min(b + step, nb - 1), wb, g, words, G, GW, B1);
    __builtin_amdgcn_sched_barrier(0);
    process(B0, b, 0);
    b += step;
    if (b >= nb) break;
    gemv_load_batch(a, min(b + step, nb - 1), wb, g, words, G, GW, B0);
    __builtin_amdgcn_sched_barrier(0);
    process(B1, b, 1);
    b += step;
  }
}

// Y[m][n] = bf16(sum over splits of partial[s][m][n]), splits in order.
__global__ __launch_bounds__(256) void gemv_split_reduce(const float* partial, int splits, size_t MN,
                                                         uint16_t* Y) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= MN) return;
  float s = 0.0f;
  for (int k = 0; k < splits; ++k) s += partial[(size_t)k * MN + i];
  Y[i] = (uint16_t)f32_to_bf16_bits(s);
}

namespace {

struct GemvPlan {
  int wpl, nw, splits, wps;
};

// words per lane and rows per workgroup for M activation rows
constexpr int gemv_wpl(int M) { return M <= 4 ? 4 : (M <= 8 ? 2 : 1); }
constexpr int gemv_rows(int M) { return M == 1 ? 4 : (M <= 8 ? 2 : 1); }

GemvPlan plan_gemv(int M, int K, int N) {
  (void)N;
  GemvPlan p;
  p.wpl = gemv_wpl(M);
  const int words = K / 8;
  const int max_wps = gemv_max_waves(M) * kWave * p.wpl;
  p.splits = (words + max_wps - 1) / max_wps;
  int wps = (words + p.splits - 1) / p.splits;
  p.wps = (wps + p.wpl - 1) / p.wpl * p.wpl;
  p.nw = (p.wps / p.wpl + kWave - 1) / kWave;
  return p;
}

// Resident workgroups per CU of one gemv instantiation at a block size (cached).
template <int M>
int gemv_blocks_per_cu(int threads) {
  static int cache[17] = {0};
  const int slot = threads / kWave;
  if (cache[slot] == 0) {
    int nblk = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nblk, gemv_kernel<M, gemv_wpl(M), gemv_rows(M)>, threads,
                                                     0) != hipSuccess ||
        nblk < 1)
      nblk = 1;
    cache[slot] = nblk;
  }
  return cache[slot];
}

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

template <int M>
void launch_m(const GemvArgs& a, const GemvPlan& p, hipStream_t stream) {
  constexpr int WPL = gemv_wpl(M);
  constexpr int R = gemv_rows(M);
  const int threads = p.nw * kWave;
  const long long nb = (a.N + R - 1) / R;
  const long long resident = (long long)device_cus() * gemv_blocks_per_cu<M>(threads);
  const long long per_split = (resident + p.splits - 1) / p.splits;
  const unsigned gx = (unsigned)(nb < per_split ? nb : per_split);
  hipLaunchKernelGGL((gemv_kernel<M, WPL, R>), dim3(gx, (unsigned)p.splits), dim3(threads), 0, stream, a);
}

}  // namespace

size_t gemv_workspace_bytes(int M, int K, int N) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  const GemvPlan p = plan_gemv(M, K, N);
  return p.splits > 1 ? (size_t)p.splits * M * N * sizeof(float) : 0;
}

int launch_gemv(const uint16_t* X, int M, int K, int N, const uint32_t* qweight,
                const uint16_t* scales, const uint32_t* qzeros, int symmetric, uint16_t* Y,
                void* workspace, hipStream_t stream) {
  if (M == 0 || N == 0) return W4_OK;
  const GemvPlan p = plan_gemv(M, K, N);
  GemvArgs a{X, K, N, qweight, scales, qzeros, symmetric, Y,
             p.splits > 1 ? static_cast<float*>(workspace) : nullptr, p.wps};
  switch (M) {
    case 1: launch_m<1>(a, p, stream); break;
    case 2: launch_m<2>(a, p, stream); break;
    case 3: launch_m<3>(a, p, stream); break;
    case 4: launch_m<4>(a, p, stream); break;
    case 5: launch_m<5>(a, p, stream); break;
    case 6: launch_m<6>(a, p, stream); break;
    case 7: launch_m<7>(a, p, stream); break;
    case 8: launch_m<8>(a, p, stream); break;
    case 9: launch_m<9>(a, p, stream); break;
    case 10: launch_m<10>(a, p, stream); break;
    case 11: launch_m<11>(a, p, stream); break;
    case 12: launch_m<12>(a, p, stream); break;
    case 13: launch_m<13>(a, p, stream); break;
    case 14: launch_m<14>(a, p, stream); break;
    case 15: launch_m<15>(a, p, stream); break;
    case 16: launch_m<16>(a, p, stream); break;
    default: return W4_ERR_UNSUPPORTED;
  }
  W4_CHECK_LAUNCH();
  if (p.splits > 1) {
    const size_t MN = (size_t)M * N;
    hipLaunchKernelGGL(gemv_split_reduce, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const float*>(workspace), p.splits, MN, Y);
    W4_CHECK_LAUNCH();
  }
  return W4_OK;
}

}  // namespace w4
