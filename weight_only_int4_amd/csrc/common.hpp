// Shared device helpers for the W4A16 kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/w4a16.h"

namespace w4 {

constexpr int kGroup = 128;          // input channels per quantization group
constexpr int kWave = 64;            // CDNA wavefront width

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
// clang vectors for __builtin_nontemporal_store / _load (HIP's uint4 is a struct)
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two int4 codes of one packed word as a bf16 pair of exact integers 128 + q.
// bf16 0x4300 is 128.0 with a mantissa step of 1, so OR-ing a nibble into the
// low mantissa bits yields 128 + q exactly.  For word w, pair p (0..3) holds
// (code of nibble p, code of nibble p + 4) = elements (p, p + 4) of the word's
// 8-channel run.
__device__ __forceinline__ uint32_t nibble_pair(uint32_t w, int p) {
  return ((w >> (4 * p)) & 0x000F000Fu) | 0x43004300u;
}

// Same, with the mask held in a register (see opaque_vgpr) so that the AND and
// the OR fuse into one v_and_or_b32 (VOP3 cannot encode two literal constants).
__device__ __forceinline__ uint32_t nibble_pair_m(uint32_t w, int p, uint32_t mask_vgpr) {
  return ((w >> (4 * p)) & mask_vgpr) | 0x43004300u;
}

// A constant the compiler must keep in a VGPR instead of folding it into literals.
__device__ __forceinline__ uint32_t opaque_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Reorder 8 consecutive bf16 activations (x0..x7 in 4 dwords) into the pairs
// (x0,x4) (x1,x5) (x2,x6) (x3,x7) that match nibble_pair's element order.
__device__ __forceinline__ void pair_activations(const uint32_t d[4], uint32_t e[4]) {
  // v_perm_b32(hi, lo, sel): selector bytes 0-3 pick bytes of lo, 4-7 bytes of hi
  e[0] = __builtin_amdgcn_perm(d[2], d[0], 0x05040100u);   // (lo16 d0, lo16 d2)
  e[1] = __builtin_amdgcn_perm(d[2], d[0], 0x07060302u);   // (hi16 d0, hi16 d2)
  e[2] = __builtin_amdgcn_perm(d[3], d[1], 0x05040100u);
  e[3] = __builtin_amdgcn_perm(d[3], d[1], 0x07060302u);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// Raw buffer resource over [base, base + bytes) (gfx9 word 3: untyped, range
// checked).  A load whose byte offset is >= bytes returns 0 and touches no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Cache-policy operand of the raw buffer loads: 0 = default, kLoadNt = the
// non-temporal (streaming) hint, for weights that one launch reads once.
constexpr int kLoadNt = 2;
// Lane offset that keeps every load out of range: all buffers here are smaller than
// 2^31 bytes, so row offset + kOob neither wraps nor lands in range.
constexpr uint32_t kOob = 0x80000000u;

// permlane32 swap of (x, y): lanes 0-31 end up with (x, x of lane + 32), lanes 32-63
// with (y of lane - 32, y); the sum of the pair is x summed over lanes l, l + 32 in
// the lower half and y summed over them in the upper half.  permlane16 likewise
// for lanes 16 apart (even 16-lane rows keep x, odd rows y).
__device__ __forceinline__ float swap_sum32(float x, float y) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float swap_sum16(float x, float y) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

}  // namespace w4

// Host-side launch-error helper: returns W4_ERR_HIP on a failed launch.
#define W4_CHECK_LAUNCH()                                   \
  do {                                                      \
    if (hipPeekAtLastError() != hipSuccess) {               \
      (void)hipGetLastError();                              \
      return W4_ERR_HIP;                                    \
    }                                                       \
  } while (0)
