// w4a16_gemv_noalloc: the decode GEMV for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops).  Same kernels and
// results as w4a16_gemv; the fp32 partial sums of a K split go to a static
// device array instead of a caller workspace.
#include <mutex>

#include "internal.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)W4_GEMV_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

}  // namespace

// One copy per device, loaded with the code object and held until the process
// ends.  In host code this name stands for the symbol, not for a device address:
// kernels receive the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::once_flag scratch_once[kMaxDevices];
void* scratch_ptr[kMaxDevices];
hipError_t scratch_err[kMaxDevices];

// Device address of `scratch` on the current device (fetched once per device).
int scratch_address(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return W4_ERR_HIP;
  std::call_once(scratch_once[dev], [dev] {
    void* p = nullptr;
    scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    scratch_ptr[dev] = p;
  });
  if (scratch_err[dev] != hipSuccess || !scratch_ptr[dev]) return W4_ERR_HIP;
  *ptr = scratch_ptr[dev];
  return W4_OK;
}

inline bool misaligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

}  // namespace

extern "C" int w4a16_gemv_noalloc(const uint16_t* X, int M, int K, int N, const uint32_t* qweight,
                                  const uint16_t* scales, const uint32_t* qzeros, int symmetric, int group_size,
                                  uint16_t* Y, void* stream) {
  using namespace w4;
  if (group_size != kGroup) return W4_ERR_UNSUPPORTED;
  if (N < 0 || K <= 0 || K % kGroup != 0 || M < 0) return W4_ERR_SHAPE;
  if (M > W4_GEMV_MAX_M) return W4_ERR_UNSUPPORTED;
  if (int st = gemv_check_size(M, K, N)) return st;
  if (gemv_workspace_bytes(M, K, N) > kScratchBytes) return W4_ERR_SCRATCH;
  if (!X || !Y) return W4_ERR_NULL;
  if (symmetric != 0 && symmetric != 1) return W4_ERR_VALUE;
  if (!qweight || !scales || (symmetric ? qzeros != nullptr : qzeros == nullptr)) return W4_ERR_NULL;
  if (misaligned16(X) || misaligned16(Y) || misaligned16(qweight) || misaligned16(scales) || misaligned16(qzeros))
    return W4_ERR_ALIGN;
  if (M == 0 || N == 0) return W4_OK;
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc) return rc;
  // every partial a split reads back is written by the same launch: nothing to clear
  return launch_gemv(X, M, K, N, qweight, scales, qzeros, symmetric, Y, ws, static_cast<hipStream_t>(stream));
}
