// Round-to-nearest group-128 int4 quantization of W diag(s) with optional clip,
// and nibble packing (one wavefront per 8 groups of one row).
//
// What is computed follows model card "rebuttal_w4g128_awq_w2" (details table row
// "Scheme": 4-bit, group 128, asymmetric zero point; the scale-rewrite paragraph:
// the candidate weight is Q(W diag(s)); "Clipping granularity": one shrink ratio
// per linear) and model card "Qwen3.6-27B-W4A16" (opening paragraph: the
// symmetric, data-free form).  Exactness rules: scale rounded to bf16 (nearest
// even) before the codes are taken against it; codes from the IEEE fp32 quotient
// (div_by_scale below obtains it exactly); rint ties to even; no contraction of the
// multiply into later operations.
#include "internal.hpp"

#pragma clang fp contract(off)

namespace w4 {

// v / sc, equal to the IEEE fp32 quotient, from the correctly rounded reciprocal
// rsc = 1 / sc (one IEEE division per lane and group) and one FMA correction
// (Markstein's division): q0 = v rsc, r = v - sc q0 (exact with an FMA), q = q0 + r rsc.
// The quotient equals the IEEE one for every bf16 divisor significand and every fp32
// dividend significand (an exhaustive check over all 2^30 pairs in the tests);
// powers of two scale every step exactly, and every quotient that rounds to a nonzero
// code is at least 0.5 with sc >= 1e-5 / 15, so no step meets a subnormal where it
// matters.  Three VALU operations instead of the division's ten.
__device__ __forceinline__ float div_by_scale(float v, float sc, float rsc) {
  const float q0 = v * rsc;
  return fmaf(fmaf(-sc, q0, v), rsc, q0);
}

// grid: x = ceil(N * GW / 4) with GW = ceil(G / 8), z = candidate; block = 256.
// Wave -> (row n, zero-word gw): its 8 lane-octets own groups 8*gw .. 8*gw + 7,
// each lane 16 consecutive input channels of one group.
template <bool SYM>
__global__ __launch_bounds__(256) void quantize_pack_kernel(QuantArgs a) {
  const int lane = threadIdx.x & 63;
  const int G = a.K / kGroup;
  const int GW = (G + 7) / 8;
  const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (long long)a.N * GW) return;          // uniform per wave
  const int n = (int)(item / GW);
  const int gw = (int)(item % GW);
  const int j = lane >> 3;                          // group within the zero word
  const int p = lane & 7;                           // 16-channel part within the group
  const int g = gw * 8 + j;
  const bool valid = g < G;
  const int c = blockIdx.z;

  const float* s = a.s ? a.s + (size_t)c * a.s_stride : nullptr;
  const float ratio = a.ratios ? a.ratios[c] : a.ratio;

  float v[16];
  if (valid) {
    const uint4* src = reinterpret_cast<const uint4*>(a.W + (size_t)n * a.K + (size_t)g * kGroup + p * 16);
    const uint4 lo = src[0], hi = src[1];
    const uint32_t d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(d[i] << 16);
      v[2 * i + 1] = __uint_as_float(d[i] & 0xFFFF0000u);
    }
    if (s) {
      const float4* sp = reinterpret_cast<const float4*>(s + (size_t)g * kGroup + p * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 f = sp[i];
        v[4 * i + 0] = v[4 * i + 0] * f.x;
        v[4 * i + 1] = v[4 * i + 1] * f.y;
        v[4 * i + 2] = v[4 * i + 2] * f.z;
        v[4 * i + 3] = v[4 * i + 3] * f.w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0.0f;
  }

  // group reductions over the 8 lanes of an octet (xor 1, 2, 4 stays in the octet)
  auto octet_max = [](float x) {
    x = fmaxf(x, __shfl_xor(x, 1, kWave));
    x = fmaxf(x, __shfl_xor(x, 2, kWave));
    return fmaxf(x, __shfl_xor(x, 4, kWave));
  };
  auto octet_min = [](float x) {
    x = fminf(x, __shfl_xor(x, 1, kWave));
    x = fminf(x, __shfl_xor(x, 2, kWave));
    return fminf(x, __shfl_xor(x, 4, kWave));
  };

  if (ratio < 1.0f) {
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(v[i]));
    const float t = ratio * octet_max(am);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = fminf(fmaxf(v[i], -t), t);
  }

  uint32_t q[16];
  uint32_t sc_bits;
  uint32_t zero = 0;
  if (SYM) {
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(v[i]));
    am = octet_max(am);
    sc_bits = f32_to_bf16_bits(fmaxf(am, 1e-5f) / 7.0f);
    const float sc = bf16_bits_to_f32(sc_bits);
    const float rsc = 1.0f / sc;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      q[i] = (uint32_t)(int)(fminf(fmaxf(rintf(div_by_scale(v[i], sc, rsc)), -8.0f), 7.0f) + 8.0f);
  } else {
    float lo = v[0], hi = v[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      lo = fminf(lo, v[i]);
      hi = fmaxf(hi, v[i]);
    }
    lo = octet_min(lo);
    hi = octet_max(hi);
    sc_bits = f32_to_bf16_bits(fmaxf(hi - lo, 1e-5f) / 15.0f);
    const float sc = bf16_bits_to_f32(sc_bits);
    const float rsc = 1.0f / sc;
    const float z = fminf(fmaxf(rintf(div_by_scale(-lo, sc, rsc)), 0.0f), 15.0f);
    zero = (uint32_t)z;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      q[i] = (uint32_t)(fminf(fmaxf(rintf(div_by_scale(v[i], sc, rsc)) + z, 0.0f), 15.0f));
  }

  if (valid) {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      w0 |= q[i] << (4 * i);
      w1 |= q[8 + i] << (4 * i);
    }
    uint32_t* qw = a.qweight + (size_t)c * a.qw_stride;
    *reinterpret_cast<uint2*>(qw + (size_t)n * (a.K / 8) + (size_t)g * 16 + p * 2) = make_uint2(w0, w1);
    if (p == 0) {
      uint16_t* sc = a.scales + (size_t)c * a.sc_stride;
      sc[(size_t)n * G + g] = (uint16_t)sc_bits;
    }
  }
  if (!SYM) {
    // gather the 8 zero points of this word (lanes 0, 8, ..., 56); unused nibbles stay 0
    const uint32_t zv = valid ? zero : 0u;
    uint32_t word = 0;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) word |= (uint32_t)__shfl((int)zv, jj * 8, kWave) << (4 * jj);
    if (lane == 0) {
      uint32_t* qz = a.qzeros + (size_t)c * a.qz_stride;
      qz[(size_t)n * GW + gw] = word;
    }
  }
}

int launch_quantize_pack(const QuantArgs& a, int C, hipStream_t stream) {
  const int G = a.K / kGroup;
  const long long items = (long long)a.N * ((G + 7) / 8);
  const long long blocks = (items + 3) / 4;
  if (blocks == 0 || C == 0) return W4_OK;
  if (blocks > 0x7FFFFFFFLL || C > 65535) return W4_ERR_SHAPE;
  dim3 grid((unsigned)blocks, 1, (unsigned)C);
  if (a.symmetric)
    hipLaunchKernelGGL(quantize_pack_kernel<true>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(quantize_pack_kernel<false>, grid, dim3(256), 0, stream, a);
  W4_CHECK_LAUNCH();
  return W4_OK;
}

}  // namespace w4
