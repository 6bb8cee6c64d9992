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

// One wave per activation row m.  Pass 1: absmax over the row (bf16 -> fp32 is
// exact).  Pass 2: lane l handles 8 consecutive channels 8 (l + 64 i); the 16
// lanes of each 16-lane row then cover one 128-channel group, whose code sum
// lane 16 r writes to xsum.
__global__ __launch_bounds__(64) void w4a8_quant_act_kernel(const uint16_t* X, int K, int8_t* Xq, float* sx,
                                                             int32_t* xsum) {
#pragma clang fp contract(off)
  const int m = blockIdx.x;
  const int lane = threadIdx.x;
  const int chunks = K >> 3;
  const uint16_t* xr = X + (size_t)m * K;
  float amax = 0.0f;
  for (int c = lane; c < chunks; c += kWave) {
    const uint4 v = *reinterpret_cast<const uint4*>(xr + 8 * c);
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(d[q] << 16)), fabsf(__uint_as_float(d[q] & 0xFFFF0000u))));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
  const float s = amax > 0.0f ? amax / 127.0f : 1.0f;
  if (lane == 0) sx[m] = s;
  const int G = K >> 7;
  for (int c0 = 0; c0 < chunks; c0 += kWave) {
    const int c = c0 + lane;
    int part = 0;
    if (c < chunks) {
      const uint4 v = *reinterpret_cast<const uint4*>(xr + 8 * c);
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
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
    const int g = (c0 >> 4) + (lane >> 4);
    if ((lane & 15) == 0 && g < G) xsum[(size_t)m * G + g] = part;
  }
}

// Workgroup: 16 output channels n0 .. n0+15 and all of K; its W waves take the
// groups g = w, w + W, ... in turn.  Per group, lane l (n = l % 16, quarter
// q = l / 16) holds the 32 codes of row n0 + n at channels 128 g + 32 q .. +31
// (one 16-byte load) and, for activation row m = l % 16, the matching 32 int8
// activations (two 16-byte loads); two v_mfma_i32_16x16x64_i8 give the group's
// exact integer sums C[n][m] (lane l: rows n = 4 (l / 16) + r, column m = l % 16).
// Codes expand to bytes with one AND (even nibbles) and one shift + AND (odd
// nibbles) per word; the activations are permuted to the same byte order.  The
// zero-point and scale fold per group reads the group's scales, zeros and
// activation code sums from LDS (staged once per workgroup); the W waves' fp32
// sums meet in LDS at the end, are added in wave order and scaled by sx[m].
template <int W>
__global__ __launch_bounds__(W * 64) void w4a8_gemv_kernel(const int8_t* Xq, const float* sx, const int32_t* xsum,
                                                           int M, int K, int N, const uint32_t* qweight,
                                                           const uint16_t* scales, const uint32_t* qzeros,
                                                           int symmetric, uint16_t* Y) {
#pragma clang fp contract(off)
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int G = K >> 7;
  const int GW = (G + 7) >> 3;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int n0 = blockIdx.x * 16;
  float* s_sc = reinterpret_cast<float*>(lds);                              // [G][16]
  int32_t* s_xs = reinterpret_cast<int32_t*>(lds + (size_t)G * 64);         // [G][16]
  uint8_t* s_z = lds + (size_t)G * 128;                                     // [G][16]
  float* s_red = reinterpret_cast<float*>(lds + (size_t)G * 144);           // [W][16][16]

  for (int e = t; e < G * 16; e += W * 64) {
    const int g = e >> 4, r = e & 15;
    const int n = n0 + r;
    float sc = 0.0f;
    uint32_t z = 8;
    if (n < N) {
      sc = bf16_bits_to_f32(scales[(size_t)n * G + g]);
      if (!symmetric) z = (qzeros[(size_t)n * GW + (g >> 3)] >> (4 * (g & 7))) & 0xFu;
    }
    s_sc[e] = sc;
    s_z[e] = (uint8_t)z;
    s_xs[e] = r < M ? xsum[(size_t)r * G + g] : 0;
  }
  __syncthreads();

  const int ln = lane & 15, q = lane >> 4;
  const uint32_t words = (uint32_t)(K >> 3);
  const auto rw = rsrc(qweight, (uint32_t)N * words * 4u);
  const auto rx = rsrc(Xq, (uint32_t)M * (uint32_t)K);
  // byte offsets of this lane's slice of group 0 (out of range past N / past M)
  const uint32_t wbase = (n0 + ln < N) ? ((uint32_t)(n0 + ln) * words + 4u * q) * 4u : kFar;
  const uint32_t xbase = (ln < M) ? (uint32_t)ln * (uint32_t)K + 32u * q : kFar;

  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int g = wave; g < G; g += W) {
    const auto wv = __builtin_amdgcn_raw_buffer_load_b128(rw, wbase + (uint32_t)g * 64u, 0, 0);
    const auto x0 = __builtin_amdgcn_raw_buffer_load_b128(rx, xbase + (uint32_t)g * 128u, 0, 0);
    const auto x1 = __builtin_amdgcn_raw_buffer_load_b128(rx, xbase + (uint32_t)g * 128u + 16u, 0, 0);
    const uint32_t w4[4] = {(uint32_t)wv[0], (uint32_t)wv[1], (uint32_t)wv[2], (uint32_t)wv[3]};
    const uint32_t xd[8] = {(uint32_t)x0[0], (uint32_t)x0[1], (uint32_t)x0[2], (uint32_t)x0[3],
                            (uint32_t)x1[0], (uint32_t)x1[1], (uint32_t)x1[2], (uint32_t)x1[3]};
    uint32_t a[8], b[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // codes of channels 8i + (0, 2, 4, 6) and 8i + (1, 3, 5, 7)
      a[2 * i] = w4[i] & 0x0F0F0F0Fu;
      a[2 * i + 1] = (w4[i] >> 4) & 0x0F0F0F0Fu;
      // activations of the same channels: v_perm_b32(hi, lo, sel) picks bytes of lo (0-3) and hi (4-7)
      b[2 * i] = __builtin_amdgcn_perm(xd[2 * i + 1], xd[2 * i], 0x06040200u);
      b[2 * i + 1] = __builtin_amdgcn_perm(xd[2 * i + 1], xd[2 * i], 0x07050301u);
    }
    const i32x4 a0 = {(int)a[0], (int)a[1], (int)a[2], (int)a[3]}, a1 = {(int)a[4], (int)a[5], (int)a[6], (int)a[7]};
    const i32x4 b0 = {(int)b[0], (int)b[1], (int)b[2], (int)b[3]}, b1 = {(int)b[4], (int)b[5], (int)b[6], (int)b[7]};
    i32x4 c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, (i32x4){0, 0, 0, 0}, 0, 0, 0);
    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, c, 0, 0, 0);
    const float4 sc4 = *reinterpret_cast<const float4*>(s_sc + g * 16 + 4 * q);
    const uint32_t z4 = *reinterpret_cast<const uint32_t*>(s_z + g * 16 + 4 * q);
    const int xs = s_xs[g * 16 + ln];
    const float scv[4] = {sc4.x, sc4.y, sc4.z, sc4.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int zr = (int)((z4 >> (8 * r)) & 0xFFu);
      acc[r] += scv[r] * (float)(c[r] - zr * xs);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) s_red[(wave * 16 + 4 * q + r) * 16 + ln] = acc[r];
  __syncthreads();
  if (t < 256) {
    const int n = t >> 4, m = t & 15;
    if (m < M && n0 + n < N) {
      float s = 0.0f;
      for (int w = 0; w < W; ++w) s += s_red[(w * 16 + n) * 16 + m];
      Y[(size_t)m * N + n0 + n] = (uint16_t)f32_to_bf16_bits(s * sx[m]);
    }
  }
}

int launch_w4a8_quantize(const uint16_t* X, int M, int K, int8_t* Xq, float* sx, int32_t* xsum,
                         hipStream_t stream) {
  if (M == 0) return W4_OK;
  hipLaunchKernelGGL(w4a8_quant_act_kernel, dim3((unsigned)M), dim3(64), 0, stream, X, K, Xq, sx, xsum);
  W4_CHECK_LAUNCH();
  return W4_OK;
}

size_t w4a8_gemv_lds_bytes(int K, int waves) { return (size_t)(K >> 7) * 144 + (size_t)waves * 16 * 16 * 4; }

int launch_w4a8_gemv(const int8_t* Xq, const float* sx, const int32_t* xsum, int M, int K, int N,
                     const uint32_t* qweight, const uint16_t* scales, const uint32_t* qzeros, int symmetric,
                     uint16_t* Y, hipStream_t stream) {
  if (M == 0 || N == 0) return W4_OK;
  // 32-bit buffer offsets: packed weights N K / 2 and activations M K below 2^31
  if ((long long)N * K / 2 >= (1LL << 31) || (long long)M * K >= (1LL << 31)) return W4_ERR_SHAPE;
  const int G = K >> 7;
  const int waves = G <= 32 ? 4 : 8;
  const size_t lds = w4a8_gemv_lds_bytes(K, waves);
  if (lds > 64 * 1024) return W4_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)((N + 15) / 16));
  if (waves == 4)
    hipLaunchKernelGGL(w4a8_gemv_kernel<4>, grid, dim3(256), lds, stream, Xq, sx, xsum, M, K, N, qweight, scales,
                       qzeros, symmetric, Y);
  else
    hipLaunchKernelGGL(w4a8_gemv_kernel<8>, grid, dim3(512), lds, stream, Xq, sx, xsum, M, K, N, qweight, scales,
                       qzeros, symmetric, Y);
  W4_CHECK_LAUNCH();
  return W4_OK;
}

}  // namespace w4
