// Elementwise steps of the decoder block, shared by the standalone kernels and the
// bf16 GEMM epilogues that fuse them, so that both compute them identically: fp32
// from bf16 inputs, no contraction, one bf16 rounding by the caller.
//
// Model card "qwen3-1.7b_q326_channel", "Model Architecture": SiLU-gated dense
// feed-forward and rotary position embedding (base 1e6, head size 128).
#pragma once

#include <hip/hip_runtime.h>

namespace w4 {

// silu(g) * u.
__device__ __forceinline__ float silu_mul_f32(float g, float u) {
#pragma clang fp contract(off)
  return g / (1.0f + expf(-g)) * u;
}

// Rotation of the pair (x1, x2) = (dim j, dim j + 64) of one head by the angle
// whose cosine and sine are c, s: (x1 c - x2 s, x2 c + x1 s).
__device__ __forceinline__ void rope_rotate(float x1, float x2, float c, float s, float& y1, float& y2) {
#pragma clang fp contract(off)
  y1 = x1 * c - x2 * s;
  y2 = x2 * c + x1 * s;
}

}  // namespace w4
