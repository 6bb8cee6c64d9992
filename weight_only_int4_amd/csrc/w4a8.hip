// W4A8 decode: the same stored int4 weights, 8-bit activations, an int8 MFMA
// contraction, for at most 16 activation rows.
//
// Model card "GLM-5.2-QSRT-Fruit-Instruct", "What is included" and "Size and
// memory": W4A8 decode execution uses the same stored weights as W4A16 (only the
// decode path changes); "Reproducible runtime": W4A8 serves decode batches of at
// most 16 rows, W4A16 everything above.  The pages do not say how activations
// become 8-bit; the reading here is per-row symmetric int8:
//   sx[m] = max_k |x[m][k]| / 127 (1 for an all-zero row), xq = clamp(rint(x / sx), -127, 127)
// (IEEE fp32 division, round half to even), and
//   Y[m][n] = sx[m] * sum_g sc[n][g] * (sum_{k in g} xq[m][k] q[n][k] - z[n][g] sum_{k in g} xq[m][k])
// with the group sums exact in int32 and the rest in fp32.
#include <algorithm>
#include <utility>

#include "internal.hpp"

namespace w4 {

namespace {

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kFar = 0x80000000u;   // a byte offset every buffer here treats as out of range

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
// sum over each 16-lane row (mirror, half mirror, quad permutations), in every lane
__device__ __forceinline__ int row16_sum_i(int v) {
  v += dpp_i<0x140>(v);
  v += dpp_i<0x141>(v);
  v += dpp_i<0x4E>(v);
  v += dpp_i<0xB1>(v);
  return v;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

}  // namespace

// One workgroup of 16 waves per activation row m.  Pass 1: absmax over the row (bf16
// -> fp32 is exact; the waves combine through LDS).  Pass 2: thread t handles the 8
// consecutive channels 8 (t + 1024 i); the 16 lanes of each 16-lane row then cover one
// 128-channel group, whose code sum the row's first lane writes to xsum.  Both passes
// load four chunks per thread before using them (K = 17408: 7.1 -> 5.4 us per call
// against four waves per row and one load at a time).
constexpr int kActThreads = 1024;                       // 16 waves per activation row
__global__ __launch_bounds__(kActThreads) void w4a8_quant_act_kernel(const uint16_t* X, int K, int8_t* Xq,
                                                                     float* sx, int32_t* xsum) {
#pragma clang fp contract(off)
  __shared__ float wmax[kActThreads / kWave];
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int chunks = K >> 3;
  const uint16_t* xr = X + (size_t)m * K;
  // both passes issue their loads four chunks at a time (one memory round trip per
  // four chunks instead of one per chunk)
  constexpr int kU = 4;
  float amax = 0.0f;
  for (int c0 = tid; c0 < chunks; c0 += kU * kActThreads) {
    uint4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = c0 + u * kActThreads;
      v[u] = c < chunks ? *reinterpret_cast<const uint4*>(xr + 8 * c) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t d[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(d[q] << 16)), fabsf(__uint_as_float(d[q] & 0xFFFF0000u))));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
  if (lane == 0) wmax[tid >> 6] = amax;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kActThreads / kWave; ++w) amax = fmaxf(amax, wmax[w]);
  const float s = amax > 0.0f ? amax / 127.0f : 1.0f;
  if (tid == 0) sx[m] = s;
  const int G = K >> 7;
  // thread t quantizes channels 8 (c0 + t) .. +7; 16 consecutive threads cover one group
  for (int cb = 0; cb < chunks; cb += kU * kActThreads) {
    uint4 vv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = cb + u * kActThreads + tid;
      vv[u] = c < chunks ? *reinterpret_cast<const uint4*>(xr + 8 * c) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = cb + u * kActThreads + tid;
      int part = 0;
      if (c < chunks) {
        const uint32_t d[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t b = (e & 1) ? (d[e >> 1] & 0xFFFF0000u) : (d[e >> 1] << 16);
          float q = __builtin_rintf(__uint_as_float(b) / s);
          q = fminf(fmaxf(q, -127.0f), 127.0f);
          const int qi = (int)q;
          part += qi;
          packed[e >> 2] |= ((uint32_t)qi & 0xFFu) << (8 * (e & 3));
        }
        *reinterpret_cast<uint2*>(Xq + (size_t)m * K + 8 * c) = make_uint2(packed[0], packed[1]);
      }
      part = row16_sum_i(part);
      const int g = (c >> 4);
      if ((lane & 15) == 0 && c < chunks && g < G) xsum[(size_t)m * G + g] = part;
    }
  }
}

// Workgroup: 16 output channels n0 .. n0+15 and all of K, or with a K split
// (grid.y > 1) the range of gsplit groups starting at g0 = blockIdx.y gsplit; its
// W waves take the groups g = g0 + w, g0 + w + W, ..., g0 + w + (NI - 1) W in turn.  Per group, lane l (row index
// l % 16, quarter q = l / 16) holds the 32 int8 activations of row m = l % 16 at
// channels 128 g + 32 q .. +31 (two 16-byte loads) and the 32 codes of output
// channel n0 + l % 16 at the same channels (one 16-byte load), plus that
// channel's scale and zero word of group g; two v_mfma_i32_16x16x64_i8
// (activations as A, codes as B) give the group's exact integer sums C[m][n]
// (lane l: rows m = 4 (l / 16) + r, column n = l % 16).  Codes expand to bytes
// with one AND (even nibbles) and one shift + AND (odd nibbles) per word; the
// activations are permuted to the same byte order.  All of a wave's groups are
// unrolled with four in flight.  The activation code sums of every group are
// staged in LDS once per workgroup; the zero-point and scale fold is one
// subtract-multiply-add per output per group; the W waves' fp32 sums meet in
// LDS at the end, are added in wave order and scaled by sx[m] -- or, with a K
// split, stored unscaled as the split's fp32 partial, which w4a8_split_reduce
// adds in split order before scaling.
template <int NI, bool NT>
__global__ __launch_bounds__(1024) void w4a8_gemv_kernel(const int8_t* Xq, const float* sx, const int32_t* xsum,
                                                         int M, int K, int N, const uint32_t* qweight,
                                                         const uint16_t* scales, const uint32_t* qzeros,
                                                         int symmetric, uint16_t* Y, int gsplit, float* part) {
#pragma clang fp contract(off)
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int G = K >> 7;
  // this workgroup's groups: [g0, g1) (grid.y splits K when gsplit > 0)
  const int g0 = gsplit ? (int)blockIdx.y * gsplit : 0;
  const int g1 = gsplit ? min(G, g0 + gsplit) : G;
  const int GW = (G + 7) >> 3;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int W = blockDim.x >> 6;          // waves: group g = wave + i W, i < NI
  const int n0 = blockIdx.x * 16;
  int32_t* s_xs = reinterpret_cast<int32_t*>(lds);                          // [G][16]
  float* s_red = reinterpret_cast<float*>(lds + (size_t)G * 64);            // [W][16][16]

  const int ln = lane & 15, q = lane >> 4;
  const uint32_t words = (uint32_t)(K >> 3);
  const auto rw = rsrc(qweight, (uint32_t)N * words * 4u);
  const auto rx = rsrc(Xq, (uint32_t)M * (uint32_t)K);
  const auto rs = rsrc(scales, (uint32_t)N * (uint32_t)G * 2u);
  const auto rz = rsrc(symmetric ? static_cast<const void*>(scales) : qzeros,
                       symmetric ? 0u : (uint32_t)N * (uint32_t)GW * 4u);
  // byte offsets of this lane's slice of group 0 (out of range past N / past M,
  // whatever the group offset added to them)
  const bool nok = n0 + ln < N;
  const uint32_t wbase = nok ? ((uint32_t)(n0 + ln) * words + 4u * q) * 4u : kFar;
  const uint32_t sbase = nok ? (uint32_t)(n0 + ln) * (uint32_t)G * 2u : kFar;
  const uint32_t zbase = nok ? (uint32_t)(n0 + ln) * (uint32_t)GW * 4u : kFar;
  const uint32_t xbase = (ln < M) ? (uint32_t)ln * (uint32_t)K + 32u * q : kFar;
  struct Slice {
    i32x4 w, x0, x1;
    uint16_t sc;
    uint32_t z;
  };
  // this lane's codes, activations, scale and zero word of group g: the lane part
  // of every offset is fixed, the group part is wave-uniform and goes in the
  // scalar offset; groups past g1 (the unrolled tail) re-read group g1-1
  auto load = [&](int g, Slice& L) {
    const int gc = min(g, g1 - 1);
    L.w = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, wbase, gc * 64, NT ? kLoadNt : 0));
    L.x0 = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xbase, gc * 128, 0));
    L.x1 = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xbase + 16u, gc * 128, 0));
    L.sc = __builtin_amdgcn_raw_buffer_load_b16(rs, sbase, gc * 2, 0);
    L.z = symmetric ? 0u : __builtin_amdgcn_raw_buffer_load_b32(rz, zbase, (gc >> 3) * 4, 0);
  };
  // the first P groups' loads go out before the staging below
  constexpr int P = NI < 4 ? NI : 4;
  Slice Ls[P];
#pragma unroll
  for (int i = 0; i < P; ++i) load(g0 + wave + i * W, Ls[i]);
  __builtin_amdgcn_sched_barrier(0);

  for (int e = t; e < G * 16; e += blockDim.x) {
    const int g = e >> 4, m = e & 15;
    s_xs[e] = m < M ? xsum[(size_t)m * G + g] : 0;
  }
  __syncthreads();

  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  auto process = [&](const Slice& L, int g) {
    uint32_t a[8], b[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t wi = (uint32_t)L.w[i];
      const uint32_t lo = (uint32_t)(i < 2 ? L.x0[2 * i] : L.x1[2 * i - 4]);
      const uint32_t hi = (uint32_t)(i < 2 ? L.x0[2 * i + 1] : L.x1[2 * i - 3]);
      // activations of channels 8i + (0, 2, 4, 6) and 8i + (1, 3, 5, 7):
      // v_perm_b32(hi, lo, sel) picks bytes of lo (0-3) and hi (4-7)
      a[2 * i] = __builtin_amdgcn_perm(hi, lo, 0x06040200u);
      a[2 * i + 1] = __builtin_amdgcn_perm(hi, lo, 0x07050301u);
      // codes of the same channels
      b[2 * i] = wi & 0x0F0F0F0Fu;
      b[2 * i + 1] = (wi >> 4) & 0x0F0F0F0Fu;
    }
    const i32x4 a0 = {(int)a[0], (int)a[1], (int)a[2], (int)a[3]}, a1 = {(int)a[4], (int)a[5], (int)a[6], (int)a[7]};
    const i32x4 b0 = {(int)b[0], (int)b[1], (int)b[2], (int)b[3]}, b1 = {(int)b[4], (int)b[5], (int)b[6], (int)b[7]};
    i32x4 c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, (i32x4){0, 0, 0, 0}, 0, 0, 0);
    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, c, 0, 0, 0);
    // groups past g1 (the unrolled tail) read group g1-1's staging and add nothing
    const bool live = g < g1;
    const int4 xs = *reinterpret_cast<const int4*>(s_xs + (live ? g : g1 - 1) * 16 + 4 * q);
    const int z = symmetric ? 8 : (int)((L.z >> (4 * (g & 7))) & 0xFu);
    const float sc = live ? bf16_bits_to_f32(L.sc) : 0.0f;
    const int xsv[4] = {xs.x, xs.y, xs.z, xs.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      acc[r] += sc * (float)(c[r] - z * xsv[r]);
      // materialize the running sum here: left free, the compiler defers every
      // group's fold to the end and keeps all the integer tiles alive (spills)
      asm volatile("" : "+v"(acc[r]));
    }
  };
  // groups g = wave + i W, i < NI (unrolled: the waits are exact); P slices in
  // flight, each refilled with the group P W further on once it is computed
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    process(Ls[i % P], g0 + wave + i * W);
    if (i + P < NI) load(g0 + wave + (i + P) * W, Ls[i % P]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) s_red[(wave * 16 + 4 * q + r) * 16 + ln] = acc[r];
  __syncthreads();
  for (int e = t; e < 256; e += blockDim.x) {
    const int m = e >> 4, n = e & 15;
    if (m < M && n0 + n < N) {
      float s = 0.0f;
      for (int w = 0; w < W; ++w) s += s_red[(w * 16 + m) * 16 + n];
      if (part)
        part[((size_t)blockIdx.y * M + m) * N + n0 + n] = s;
      else
        Y[(size_t)m * N + n0 + n] = (uint16_t)f32_to_bf16_bits(s * sx[m]);
    }
  }
}

namespace {

constexpr int kW4a8MaxNi = 25;       // 400 groups at 16 waves
using W4a8Kernel = void (*)(const int8_t*, const float*, const int32_t*, int, int, int, const uint32_t*,
                            const uint16_t*, const uint32_t*, int, uint16_t*, int, float*);

// Y[m][n] = bf16(sx[m] * sum over splits k of part[k][m][n]), fp32 in split order.
__global__ __launch_bounds__(256) void w4a8_split_reduce(const float* part, int splits, int M, int N,
                                                         const float* sx, uint16_t* Y) {
  const size_t MN = (size_t)M * N;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= MN) return;
  float s = 0.0f;
  for (int k = 0; k < splits; ++k) s += part[(size_t)k * MN + i];
  Y[i] = (uint16_t)f32_to_bf16_bits(s * sx[i / N]);
}

template <bool NT, int... I>
W4a8Kernel w4a8_pick(int ni, std::integer_sequence<int, I...>) {
  W4a8Kernel k = nullptr;
  ((ni == I + 2 ? (k = w4a8_gemv_kernel<I + 2, NT>, 0) : 0), ...);
  return k;
}

// Packed weights up to this size take the non-temporal hint (a measured rule).
// Cold, M = 1 / 16: 8 MB 6.24 -> 5.52 / 7.79 -> 7.35 us, 16-32 MB 3-10% / 0-3%
// faster, 42 MB (K = 5120) 1.5% / 3% slower; the decode sweep 7% / 6% faster.
constexpr long long kW4a8NtMaxBytes = 32LL << 20;

W4a8Kernel w4a8_kernel_for(int ni, bool nt) {
  return nt ? w4a8_pick<true>(ni, std::make_integer_sequence<int, kW4a8MaxNi - 1>{})
            : w4a8_pick<false>(ni, std::make_integer_sequence<int, kW4a8MaxNi - 1>{});
}

}  // namespace

int launch_w4a8_quantize(const uint16_t* X, int M, int K, int8_t* Xq, float* sx, int32_t* xsum,
                         hipStream_t stream) {
  if (M == 0) return W4_OK;
  hipLaunchKernelGGL(w4a8_quant_act_kernel, dim3((unsigned)M), dim3(kActThreads), 0, stream, X, K, Xq, sx, xsum);
  W4_CHECK_LAUNCH();
  return W4_OK;
}

// K split, a function of the shape only (the workspace size follows it): when K
// has at least 64 groups and the ceil(N / 16) column tiles are fewer than two per
// CU of 256, the groups are split into ranges of at least 16 so that the tiles x
// splits workgroups come near two per CU (K = 17408, N = 5120 takes 2: 20.1 ->
// 19.4 us at M = 1, 32.9 -> 30.2 us at M = 16).  Shorter K keeps one workgroup
// per tile: the second kernel's launch costs more than the split saves there (the
// decode sweep's K = 6144 down projection in 3 splits made the sweep 4% slower).
int w4a8_k_splits(int K, int N) {
  const int G = K >> 7;
  const long long tiles = (N + 15) / 16;
  if (G < 64 || tiles >= 2 * 256) return 1;
  const int s = (int)std::min<long long>((2 * 256 + tiles - 1) / tiles, G / 16);
  const int gs = (G + s - 1) / s;
  return (G + gs - 1) / gs;          // every split non-empty
}

size_t w4a8_workspace_bytes(int M, int K, int N) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  const int s = w4a8_k_splits(K, N);
  return s > 1 ? (size_t)s * M * N * sizeof(float) : 0;
}

// W waves per workgroup and NI = ceil(Gs / W) groups per wave (2 <= NI <= 25), Gs
// the groups of one split: the most waves (8, 4 or 2) with which one round of
// resident workgroups covers the ceil(N / 16) column tiles times the splits (about
// 20 resident waves per CU), at least ceil(Gs / 25).  LDS: per group of K the code
// sums of the 16 activation rows (int32), plus 16 x 16 fp32 sums per wave.
int w4a8_plan(int K, int N, int cus, int* ni, int* waves, size_t* lds) {
  const int GK = K >> 7;
  if (GK > kW4a8MaxNi * 16) return W4_ERR_UNSUPPORTED;   // 400 groups: the limit without a split
  const int splits = w4a8_k_splits(K, N);
  const int G = (GK + splits - 1) / splits;
  const long long tiles = (N + 15) / 16 * splits;
  int w = 2;
  for (int cand : {8, 4}) {
    if (tiles <= (long long)cus * (20 / cand)) {
      w = cand;
      break;
    }
  }
  w = std::max(std::min(w, G), (G + kW4a8MaxNi - 1) / kW4a8MaxNi);
  const int n = std::max(2, (G + w - 1) / w);
  const size_t bytes = (size_t)GK * 64 + (size_t)w * 16 * 16 * 4;
  if (w > 16 || n > kW4a8MaxNi || bytes > 64 * 1024) return W4_ERR_UNSUPPORTED;
  if (ni) *ni = n;
  if (waves) *waves = w;
  if (lds) *lds = bytes;
  return W4_OK;
}

int launch_w4a8_gemv(const int8_t* Xq, const float* sx, const int32_t* xsum, int M, int K, int N,
                     const uint32_t* qweight, const uint16_t* scales, const uint32_t* qzeros, int symmetric,
                     uint16_t* Y, void* workspace, hipStream_t stream) {
  if (M == 0 || N == 0) return W4_OK;
  // 32-bit buffer offsets: packed weights N K / 2 and activations M K below 2^31
  if ((long long)N * K / 2 >= (1LL << 31) || (long long)M * K >= (1LL << 31)) return W4_ERR_SHAPE;
  int ni = 0, waves = 0;
  size_t lds = 0;
  int cus = 256, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess || cus < 1)
    cus = 256;
  const int st = w4a8_plan(K, N, cus, &ni, &waves, &lds);
  if (st != W4_OK) return st;
  const int splits = w4a8_k_splits(K, N);
  const int G = K >> 7;
  const int gsplit = splits > 1 ? (G + splits - 1) / splits : 0;
  float* part = splits > 1 ? static_cast<float*>(workspace) : nullptr;
  const dim3 grid((unsigned)((N + 15) / 16), (unsigned)splits);
  hipLaunchKernelGGL(w4a8_kernel_for(ni, (long long)N * K / 2 <= kW4a8NtMaxBytes), grid, dim3(waves * 64), lds, stream, Xq, sx, xsum, M, K, N, qweight, scales,
                     qzeros, symmetric, Y, gsplit, part);
  W4_CHECK_LAUNCH();
  if (splits > 1) {
    const size_t MN = (size_t)M * N;
    hipLaunchKernelGGL(w4a8_split_reduce, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, stream, part, splits, M,
                       N, sx, Y);
    W4_CHECK_LAUNCH();
  }
  return W4_OK;
}

}  // namespace w4
