// Measurement helpers: a plain streaming read and an empty kernel.  They are
// the yardsticks the W4A16 kernels are measured against on the same device: the
// bandwidth a simple read of a buffer of a given size reaches, the duration of a
// launch that does nothing, and a kernel of known byte traffic for scaling the
// hardware's fetch counters.
#include "internal.hpp"

namespace w4 {

// Each thread reads U 16-byte chunks per iteration of a grid-stride loop and
// folds them into an XOR, written once per thread (so the reads cannot be
// removed); NT selects non-temporal loads.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U, bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  uint32_t acc = 0;
  size_t i = tid;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (NT)
        v[u] = __builtin_nontemporal_load(p + i + u * stride);
      else
        v[u] = p[i + u * stride];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[tid] = acc;
}

__global__ void empty_kernel() {}

}  // namespace w4

using namespace w4;

extern "C" int w4_probe_stream_read(const void* buf, size_t bytes, int unroll, int nontemporal, int blocks,
                                    uint32_t* sink, void* stream) {
  if (!buf || !sink) return W4_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) || (bytes & 15u)) return W4_ERR_ALIGN;
  if (blocks < 1 || blocks > (1 << 20)) return W4_ERR_SHAPE;
  if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) return W4_ERR_VALUE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const u32x4* p = static_cast<const u32x4*>(buf);
  const size_t n16 = bytes / 16;
  const dim3 g((unsigned)blocks), b(256);
#define W4_SR(U)                                                                          \
  if (nontemporal)                                                                        \
    hipLaunchKernelGGL((stream_read_kernel<U, true>), g, b, 0, s, p, n16, sink);          \
  else                                                                                    \
    hipLaunchKernelGGL((stream_read_kernel<U, false>), g, b, 0, s, p, n16, sink);
  switch (unroll) {
    case 1: W4_SR(1); break;
    case 2: W4_SR(2); break;
    case 4: W4_SR(4); break;
    default: W4_SR(8); break;
  }
#undef W4_SR
  W4_CHECK_LAUNCH();
  return W4_OK;
}

extern "C" int w4_probe_empty(void* stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
  W4_CHECK_LAUNCH();
  return W4_OK;
}
