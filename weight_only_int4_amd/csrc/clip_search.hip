// Stock per-output-channel clipping search, model card "rebuttal_w4g128_awq_w2",
// "Clipping granularity" and the comparability caveat under the perplexity table:
// the d = 0 arm picks a clipping threshold per output channel (and group), each
// channel scored on its own error, where the look-ahead arm uses one shrink ratio.
//
// For output channel n, group g and ratio r_j:
//   v = fp32(W[n][k] * s[k]) over the 128 channels k of g,
//   w_hat = dequantized RTN of clamp(v, +-r_j * absmax(v)) (the quantizer of
//           awq_quantize_pack with clip r_j),  e = v - w_hat,
//   L[g][n][j] = sum_t (sum_k x'[t][k] e[k])^2 = e^T H_g e,
//   H_g = X'_g^T X'_g,  x' = bf16(X[t][k] / s[k])  (the deployed activations),
//   best[n][g] = first j of least L[g][n][j].
//
// Steps, all on the caller's stream:
//   1. gram_partial_kernel: H_g over token slices, bf16 MFMA (products of bf16
//      values are exact in fp32), one fp32 partial per (slice, g).
//   2. gram_finish_kernel: fixed-order sum of the slices, split of each entry into
//      bf16 hi + lo, stored in the A-operand order of step 3.
//   3. clip_loss_kernel: per lane pair one (n, g); for every ratio the lane pair
//      quantizes its group in registers, forms e as bf16 hi + lo, and the wave
//      computes (H_g E^T) for 32 channels with three bf16 MFMA products
//      (Hhi Ehi + Hhi Elo + Hlo Ehi); each lane then dots its half of e with its
//      half of H_g e.  H_g (hi and lo, 64 KiB) sits in LDS for the workgroup.
#include "internal.hpp"

#pragma clang fp contract(off)

namespace w4 {

namespace {

constexpr int kGramChunk = 64;           // tokens staged in LDS per step of the Gram kernel
constexpr int kXtStride = kGramChunk + 8;  // bf16 elements per channel row of the staged tile (bank spread)
constexpr int kClipWaves = 4;            // waves per workgroup of the loss kernel (32 channels each)
constexpr size_t kHpermBytes = 65536;    // hi + lo A operands of one group: 4 x 8 x 2 x 64 lanes x 16 B

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of H_g held by output slot o (0..127) of the loss kernel's MFMA blocks.
// Output lane l, block rb, register r sits at slot 32 rb + (r % 4) + 4 (l / 32) +
// 8 (r / 4); the slot is given the physical index 64 (l / 32) + 16 rb + r so that
// each lane holds H e at the same 64 indices whose e it holds.
__device__ __forceinline__ int out_slot_index(int o) {
  const int rb = o >> 5, i = o & 31;
  return 64 * ((i >> 2) & 1) + 16 * rb + (i & 3) + 4 * (i >> 3);
}

// ---------------------------------------------------------------------------------------
// 1. Gram partials.  grid (G, slices), 256 threads.  Slice ts covers tokens
// [ts * per, min(T, (ts + 1) * per)).  Wave w computes the 32x32 blocks (bi, bj) with
// bi in {2 (w / 2), 2 (w / 2) + 1}, bj in {2 (w % 2), 2 (w % 2) + 1}.  MFMA operand
// for channel block b: lane l holds x'[t0 + 16 step + 8 (l / 32) + 0..7][32 b + l % 32],
// read as 16 bytes from the token-contiguous staged tile.
__global__ __launch_bounds__(256) void gram_partial_kernel(const uint16_t* __restrict__ X, int T, int K,
                                                           const float* __restrict__ s, int per,
                                                           float* __restrict__ Hpart) {
  __shared__ __align__(16) uint16_t xt[kGroup * kXtStride];
  const int g = blockIdx.x;
  const int ts = blockIdx.y;
  const int G = gridDim.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t_begin = ts * per;
  const int t_end = min(T, t_begin + per);

  // staging assignment: token pair tp, channel octets oc and oc + 8
  const int tp = tid & 31;
  const int oc = tid >> 5;
  float sv[2][8];
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      sv[it][i] = s ? s[(size_t)g * kGroup + 8 * (oc + 8 * it) + i] : 1.0f;

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  const int bi0 = 2 * (wave >> 1), bj0 = 2 * (wave & 1);
  // the next chunk's rows are loaded into registers while the current one is multiplied
  uint4 d[2][2];
  auto load = [&](int t0) {
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = t0 + 2 * tp + u;
        d[it][u] = make_uint4(0u, 0u, 0u, 0u);
        if (t < t_end)
          d[it][u] = *reinterpret_cast<const uint4*>(X + (size_t)t * K + (size_t)g * kGroup + 8 * (oc + 8 * it));
      }
  };
  if (t_begin < t_end) load(t_begin);
  for (int t0 = t_begin; t0 < t_end; t0 += kGramChunk) {
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int c8 = 8 * (oc + 8 * it);
      uint32_t xv[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t w[4] = {d[it][u].x, d[it][u].y, d[it][u].z, d[it][u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = __uint_as_float(w[q] << 16) / sv[it][2 * q];
          const float hi = __uint_as_float(w[q] & 0xFFFF0000u) / sv[it][2 * q + 1];
          xv[u][q] = f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = i >> 1, sh = (i & 1) * 16;
        const uint32_t pair = ((xv[0][q] >> sh) & 0xFFFFu) | (((xv[1][q] >> sh) & 0xFFFFu) << 16);
        *reinterpret_cast<uint32_t*>(&xt[(c8 + i) * kXtStride + 2 * tp]) = pair;
      }
    }
    if (t0 + kGramChunk < t_end) load(t0 + kGramChunk);
    __syncthreads();
#pragma unroll
    for (int step = 0; step < kGramChunk / 16; ++step) {
      const int col = 16 * step + 8 * (lane >> 5);
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        fa[a] = *reinterpret_cast<const bf16x8*>(&xt[(32 * (bi0 + a) + (lane & 31)) * kXtStride + col]);
        fb[a] = *reinterpret_cast<const bf16x8*>(&xt[(32 * (bj0 + a) + (lane & 31)) * kXtStride + col]);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma_bf16(fa[a], fb[b], acc[a][b]);
    }
  }

  float* out = Hpart + ((size_t)ts * G + g) * (kGroup * kGroup);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 32 * (bi0 + a) + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
        const int j = 32 * (bj0 + b) + (lane & 31);
        out[i * kGroup + j] = acc[a][b][r];
      }
}

// ---------------------------------------------------------------------------------------
// 2. H_g = sum over slices (fp64, slice order), split h = hi + lo (bf16 each, lo of the
// exact fp32 remainder), written as the loss kernel's A operands:
//   Hperm[g][((rb * 8 + step) * 2 + part) * 64 + lane] = 8 bf16, element jj =
//   H[out_slot_index(32 rb + lane % 32)][64 (lane / 32) + 8 step + jj].
// One thread per (g, row, 8-column run), consecutive threads reading consecutive runs:
// grid G * 2048 / 256.  Row p = out_slot_index(o) for o = 32 rb + i with
// rb = (p / 16) % 4 and i = (p % 4) + 4 (p / 64) + 8 ((p % 16) / 4).
__global__ __launch_bounds__(256) void gram_finish_kernel(const float* __restrict__ Hpart, int slices, int G,
                                                          uint4* __restrict__ Hperm) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int g = idx >> 11;
  if (g >= G) return;
  const int row = (idx >> 4) & 127;
  const int run = idx & 15;
  double acc[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) acc[jj] = 0.0;
  for (int ts = 0; ts < slices; ++ts) {
    const float4* src =
        reinterpret_cast<const float4*>(Hpart + ((size_t)ts * G + g) * (kGroup * kGroup) + row * kGroup + 8 * run);
    const float4 a = src[0], b = src[1];
    acc[0] += (double)a.x;
    acc[1] += (double)a.y;
    acc[2] += (double)a.z;
    acc[3] += (double)a.w;
    acc[4] += (double)b.x;
    acc[5] += (double)b.y;
    acc[6] += (double)b.z;
    acc[7] += (double)b.w;
  }
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int jj = 0; jj < 8; jj += 2) {
    uint32_t hb[2], lb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float h = (float)acc[jj + u];
      hb[u] = f32_to_bf16_bits(h);
      lb[u] = f32_to_bf16_bits(h - bf16_bits_to_f32(hb[u]));
    }
    hi[jj >> 1] = hb[0] | (hb[1] << 16);
    lo[jj >> 1] = lb[0] | (lb[1] << 16);
  }
  const int rb = (row >> 4) & 3;
  const int i = (row & 3) + 4 * (row >> 6) + 8 * ((row & 15) >> 2);
  const int lane = i + 32 * (run >> 3);
  const int step = run & 7;
  uint4* dst = Hperm + (size_t)g * (kHpermBytes / 16) + (size_t)((rb * 8 + step) * 2) * 64 + lane;
  dst[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  dst[64] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
}

// ---------------------------------------------------------------------------------------
// 3. Losses and choices.  grid (ceil(N / 128), G), 256 threads.  Lane l of wave w owns
// channel n = 128 blockIdx.x + 32 w + l % 32 and the 64 group channels
// 64 (l / 32) + 0..63; the lane pair (l, l + 32) shares one (n, g).
template <bool SYM>
__global__ __launch_bounds__(256, 2) void clip_loss_kernel(const uint16_t* __restrict__ W, int N, int K,
                                                           const float* __restrict__ s,
                                                           const float* __restrict__ ratios, int R,
                                                           const uint4* __restrict__ Hperm,
                                                           float* __restrict__ losses,
                                                           uint8_t* __restrict__ best) {
  __shared__ __align__(16) uint4 hs[kHpermBytes / 16];
  const int g = blockIdx.y;
  const int G = gridDim.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int n = blockIdx.x * (32 * kClipWaves) + 32 * (tid >> 6) + (lane & 31);
  const bool live = n < N;

  {
    const uint4* src = Hperm + (size_t)g * (kHpermBytes / 16);
#pragma unroll 4
    for (int i = tid; i < (int)(kHpermBytes / 16); i += 256) hs[i] = src[i];
  }

  // v = W * s over this lane's 64 channels of the group
  float v[64];
  {
    const size_t base = (size_t)n * K + (size_t)g * kGroup + 64 * half;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint4 d = make_uint4(0u, 0u, 0u, 0u);
      if (live) d = *reinterpret_cast<const uint4*>(W + base + 8 * c);
      const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[8 * c + 2 * q] = __uint_as_float(w[q] << 16);
        v[8 * c + 2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
      }
    }
    if (s) {
      const float4* sp = reinterpret_cast<const float4*>(s + (size_t)g * kGroup + 64 * half);
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float4 f = sp[c];
        v[4 * c + 0] = v[4 * c + 0] * f.x;
        v[4 * c + 1] = v[4 * c + 1] * f.y;
        v[4 * c + 2] = v[4 * c + 2] * f.z;
        v[4 * c + 3] = v[4 * c + 3] * f.w;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 64; ++i) v[i] = __builtin_canonicalizef(v[i]);
  // group minimum and maximum of v.  Clamping is monotone, so the clipped group's
  // minimum and maximum are the clamped ones, and its largest magnitude is the larger
  // magnitude of the two: the per-ratio statistics need no pass over the values.
  float vmin = v[0], vmax = v[0];
#pragma unroll
  for (int i = 1; i < 64; ++i) {
    vmin = fminf(vmin, v[i]);
    vmax = fmaxf(vmax, v[i]);
  }
  vmin = fminf(vmin, __shfl_xor(vmin, 32, kWave));
  vmax = fmaxf(vmax, __shfl_xor(vmax, 32, kWave));
  const float amax = fmaxf(fabsf(vmin), fabsf(vmax));
  __syncthreads();

  float best_loss = 0.0f;
  int best_j = 0;
  for (int j = 0; j < R; ++j) {
    // compiler-only fence: keeps the LDS operand reads inside the loop (hoisted, the
    // 256 registers of all of H_g's operands would not fit)
    asm volatile("" ::: "memory");
    // clip threshold t = ratio * absmax >= 0 for ratio > 0; a ratio >= 1 leaves every
    // value in [-t, t], which is the unclipped group.  med3(x, -t, t) is the clamp.
    const float t = ratios[j] * amax;
    auto clamped = [&](float x) { return __builtin_amdgcn_fmed3f(x, -t, t); };
    const float lo = clamped(vmin), hi = clamped(vmax);
    float sc, z;
    if (SYM) {
      sc = bf16_bits_to_f32(f32_to_bf16_bits(fmaxf(fmaxf(fabsf(lo), fabsf(hi)), 1e-5f) / 7.0f));
      z = 8.0f;                                        // stored offset: q = d + 8
    } else {
      sc = bf16_bits_to_f32(f32_to_bf16_bits(fmaxf(hi - lo, 1e-5f) / 15.0f));
      z = fminf(fmaxf(rintf(-lo / sc), 0.0f), 15.0f);
    }
    // stored codes q in 0..15 (bytes), d = q - z.  The code is rint of the IEEE quotient
    // c / sc, obtained exactly from the correctly rounded reciprocal 1 / sc with one FMA
    // correction (Markstein's division: q0 = c rsc, q = q0 + (c - sc q0) rsc), which
    // equals the IEEE quotient for every bf16 divisor (the same exhaustive check as the
    // quantizer's).
    const float rsc = 1.0f / sc;
    auto code = [&](float k) {
      return SYM ? __builtin_amdgcn_fmed3f(k, -8.0f, 7.0f) + 8.0f : __builtin_amdgcn_fmed3f(k + z, 0.0f, 15.0f);
    };
    uint32_t dq[16];
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float c = clamped(v[4 * w + u]);
        const float q0 = c * rsc;
        const float k = rintf(fmaf(fmaf(-sc, q0, c), rsc, q0));
        word = __builtin_amdgcn_cvt_pk_u8_f32(code(k), u, word);
      }
      dq[w] = word;
    }
    // e[m] = v[m] - d[m] sc with one rounding (d sc is exact: a small integer times a
    // bf16 value), the same in the products and in the epilogue
    auto err = [&](int m) {
      const float d = (float)((dq[m >> 2] >> (8 * (m & 3))) & 0xFFu) - z;
      return fmaf(-d, sc, v[m]);
    };

    f32x16 acc[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) acc[rb] = f32x16{};
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st & 1) asm volatile("" ::: "memory");   // operand reads at most two k-steps ahead
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float e0 = err(8 * st + 2 * q), e1 = err(8 * st + 2 * q + 1);
        const bf16x2 hp = {(__bf16)e0, (__bf16)e1};
        ph[q] = __builtin_bit_cast(uint32_t, hp);
        const bf16x2 lp = {(__bf16)(e0 - __uint_as_float(ph[q] << 16)),
                           (__bf16)(e1 - __uint_as_float(ph[q] & 0xFFFF0000u))};
        pl[q] = __builtin_bit_cast(uint32_t, lp);
      }
      const bf16x8 ehi = __builtin_bit_cast(bf16x8, make_uint4(ph[0], ph[1], ph[2], ph[3]));
      const bf16x8 elo = __builtin_bit_cast(bf16x8, make_uint4(pl[0], pl[1], pl[2], pl[3]));
      bf16x8 ah[4], al[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        ah[rb] = __builtin_bit_cast(bf16x8, hs[((rb * 8 + st) * 2) * 64 + lane]);
        al[rb] = __builtin_bit_cast(bf16x8, hs[((rb * 8 + st) * 2 + 1) * 64 + lane]);
      }
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) acc[rb] = mfma_bf16(ah[rb], ehi, acc[rb]);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) acc[rb] = mfma_bf16(ah[rb], elo, acc[rb]);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) acc[rb] = mfma_bf16(al[rb], ehi, acc[rb]);
    }

    // lane's half: sum over its 64 indices m of e[m] (H e)[m], (H e)[m] in block m / 16,
    // register m % 16.
    float part = 0.0f;
#pragma unroll
    for (int m = 0; m < 64; ++m) part = fmaf(err(m), acc[m >> 4][m & 15], part);
    const float other = __shfl_xor(part, 32, kWave);
    const float loss = half ? other + part : part + other;   // (lower half) + (upper half) in every lane
    if (j == 0 || loss < best_loss) {
      best_loss = loss;
      best_j = j;
    }
    if (live && half == 0 && losses) losses[((size_t)g * N + n) * R + j] = loss;
  }
  if (live && half == 0) best[(size_t)n * G + g] = (uint8_t)best_j;
}

struct ClipLayout {
  size_t hpart, hperm, total;
  int slices, per;
};

ClipLayout clip_layout(int T, int K) {
  ClipLayout L{};
  const int G = K / kGroup;
  const int chunks = max(1, (T + kGramChunk - 1) / kGramChunk);
  int slices = min(chunks, max(1, (256 + G - 1) / G));
  const int per_chunks = (chunks + slices - 1) / slices;
  slices = (chunks + per_chunks - 1) / per_chunks;
  L.slices = slices;
  L.per = per_chunks * kGramChunk;
  L.hpart = 0;
  L.hperm = align_up((size_t)slices * G * kGroup * kGroup * 4, 256);
  L.total = L.hperm + (size_t)G * kHpermBytes;
  return L;
}

}  // namespace

size_t clip_search_workspace_bytes(int T, int K) {
  if (T < 0 || K <= 0 || K % kGroup) return 0;
  return clip_layout(T, K).total;
}

int launch_clip_search(const uint16_t* X, int T, int K, int N, const uint16_t* W, const float* s,
                       const float* ratios, int R, int symmetric, float* losses, uint8_t* best,
                       void* workspace, hipStream_t stream) {
  if (N == 0) return W4_OK;
  const int G = K / kGroup;
  if (G > 65535) return W4_ERR_SHAPE;
  const ClipLayout L = clip_layout(T, K);
  char* ws = static_cast<char*>(workspace);
  float* hpart = reinterpret_cast<float*>(ws + L.hpart);
  uint4* hperm = reinterpret_cast<uint4*>(ws + L.hperm);
  hipLaunchKernelGGL(gram_partial_kernel, dim3((unsigned)G, (unsigned)L.slices), dim3(256), 0, stream, X, T, K, s,
                     L.per, hpart);
  W4_CHECK_LAUNCH();
  hipLaunchKernelGGL(gram_finish_kernel, dim3((unsigned)(G * 8)), dim3(256), 0, stream, hpart, L.slices, G, hperm);
  W4_CHECK_LAUNCH();
  const dim3 grid((unsigned)((N + 32 * kClipWaves - 1) / (32 * kClipWaves)), (unsigned)G);
  if (symmetric)
    hipLaunchKernelGGL(clip_loss_kernel<true>, grid, dim3(64 * kClipWaves), 0, stream, W, N, K, s, ratios, R, hperm,
                       losses, best);
  else
    hipLaunchKernelGGL(clip_loss_kernel<false>, grid, dim3(64 * kClipWaves), 0, stream, W, N, K, s, ratios, R, hperm,
                       losses, best);
  W4_CHECK_LAUNCH();
  return W4_OK;
}

}  // namespace w4
