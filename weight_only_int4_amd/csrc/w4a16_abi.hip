// C-ABI entry points: argument validation (host only, before any HIP call) and
// dispatch to the kernel launchers.  See include/w4a16.h for the contract.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <thread>
#include <vector>

#include "internal.hpp"

using namespace w4;

namespace {

inline bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// shapes shared by the weight-consuming calls
int check_weight_shape(int N, int K, int group_size) {
  if (group_size != kGroup) return W4_ERR_UNSUPPORTED;
  if (N < 0 || K <= 0 || K % kGroup != 0) return W4_ERR_SHAPE;
  return W4_OK;
}

int check_packed(const uint32_t* qweight, const uint16_t* scales, const uint32_t* qzeros, int symmetric) {
  if (symmetric != 0 && symmetric != 1) return W4_ERR_VALUE;
  if (!qweight || !scales) return W4_ERR_NULL;
  if (symmetric ? qzeros != nullptr : qzeros == nullptr) return W4_ERR_NULL;
  if (misaligned(qweight) || misaligned(scales) || misaligned(qzeros)) return W4_ERR_ALIGN;
  return W4_OK;
}

}  // namespace

extern "C" {

const char* w4_status_string(int status) {
  switch (status) {
    case W4_OK: return "W4_OK";
    case W4_ERR_NULL: return "W4_ERR_NULL: a required pointer is NULL (or a forbidden one is set)";
    case W4_ERR_SHAPE: return "W4_ERR_SHAPE: size out of range or K not a multiple of 128";
    case W4_ERR_ALIGN: return "W4_ERR_ALIGN: an array pointer is not 16-byte aligned";
    case W4_ERR_UNSUPPORTED: return "W4_ERR_UNSUPPORTED: group_size != 128 or M beyond the decode path";
    case W4_ERR_WORKSPACE: return "W4_ERR_WORKSPACE: workspace missing or too small";
    case W4_ERR_HIP: return "W4_ERR_HIP: a HIP runtime call failed";
    case W4_ERR_VALUE: return "W4_ERR_VALUE: scalar argument out of range";
    case W4_ERR_SCRATCH: return "W4_ERR_SCRATCH: the problem needs more than the static scratch array holds";
    default: return "W4_ERR_UNKNOWN";
  }
}

int awq_quantize_pack(const uint16_t* W, int N, int K, const float* s, float clip_ratio, int symmetric,
                      int group_size, uint32_t* qweight, uint16_t* scales, uint32_t* qzeros, void* stream) {
  int st = check_weight_shape(N, K, group_size);
  if (st) return st;
  if (!W) return W4_ERR_NULL;
  st = check_packed(qweight, scales, qzeros, symmetric);
  if (st) return st;
  if (misaligned(W) || misaligned(s)) return W4_ERR_ALIGN;
  if (!(clip_ratio > 0.0f && clip_ratio <= 1.0f)) return W4_ERR_VALUE;
  if (N == 0) return W4_OK;
  QuantArgs a{};
  a.W = W;
  a.N = N;
  a.K = K;
  a.s = s;
  a.ratio = clip_ratio;
  a.symmetric = symmetric;
  a.qweight = qweight;
  a.scales = scales;
  a.qzeros = qzeros;
  return launch_quantize_pack(a, 1, static_cast<hipStream_t>(stream));
}

int w4a16_gemv(const uint16_t* X, int M, int K, int N, const uint32_t* qweight, const uint16_t* scales,
               const uint32_t* qzeros, int symmetric, int group_size, uint16_t* Y, void* workspace,
               size_t* workspace_bytes, void* stream) {
  int st = check_weight_shape(N, K, group_size);
  if (st) return st;
  if (M < 0) return W4_ERR_SHAPE;
  if (M > W4_GEMV_MAX_M) return W4_ERR_UNSUPPORTED;
  if ((st = gemv_check_size(M, K, N))) return st;
  const size_t need = gemv_workspace_bytes(M, K, N);
  if (!workspace && workspace_bytes) {
    *workspace_bytes = need;
    return W4_OK;
  }
  if (need > 0 && (!workspace || !workspace_bytes || *workspace_bytes < need)) return W4_ERR_WORKSPACE;
  if (!X || !Y) return W4_ERR_NULL;
  st = check_packed(qweight, scales, qzeros, symmetric);
  if (st) return st;
  if (misaligned(X) || misaligned(Y) || misaligned(workspace)) return W4_ERR_ALIGN;
  return launch_gemv(X, M, K, N, qweight, scales, qzeros, symmetric, Y, workspace,
                     static_cast<hipStream_t>(stream));
}

int w4a8_quantize_activations(const uint16_t* X, int M, int K, int8_t* Xq, float* sx, int32_t* xsum,
                              void* stream) {
  if (M < 0 || K <= 0 || K % kGroup != 0) return W4_ERR_SHAPE;
  if (M > W4_GEMV_MAX_M) return W4_ERR_UNSUPPORTED;
  if (M == 0) return W4_OK;
  if (!X || !Xq || !sx || !xsum) return W4_ERR_NULL;
  if (misaligned(X) || misaligned(Xq)) return W4_ERR_ALIGN;
  return launch_w4a8_quantize(X, M, K, Xq, sx, xsum, static_cast<hipStream_t>(stream));
}

int w4a8_gemv(const int8_t* Xq, const float* sx, const int32_t* xsum, int M, int K, int N,
              const uint32_t* qweight, const uint16_t* scales, const uint32_t* qzeros, int symmetric,
              int group_size, uint16_t* Y, void* workspace, size_t* workspace_bytes, void* stream) {
  int st = check_weight_shape(N, K, group_size);
  if (st) return st;
  if (M < 0) return W4_ERR_SHAPE;
  if (M > W4_GEMV_MAX_M) return W4_ERR_UNSUPPORTED;
  if (w4a8_plan(K, N, 256, nullptr, nullptr, nullptr) != W4_OK) return W4_ERR_UNSUPPORTED;
  if ((st = gemv_check_size(M, K, N))) return st;
  const size_t need = w4a8_workspace_bytes(M, K, N);
  if (!workspace && workspace_bytes) {
    *workspace_bytes = need;
    return W4_OK;
  }
  if (need > 0 && (!workspace || !workspace_bytes || *workspace_bytes < need)) return W4_ERR_WORKSPACE;
  if (M == 0 || N == 0) return W4_OK;
  if (!Xq || !sx || !xsum || !Y) return W4_ERR_NULL;
  st = check_packed(qweight, scales, qzeros, symmetric);
  if (st) return st;
  if (misaligned(Xq) || misaligned(Y) || misaligned(workspace)) return W4_ERR_ALIGN;
  return launch_w4a8_gemv(Xq, sx, xsum, M, K, N, qweight, scales, qzeros, symmetric, Y, workspace,
                          static_cast<hipStream_t>(stream));
}

int w4a16_gemm(const uint16_t* X, int M, int K, int N, const uint32_t* qweight, const uint16_t* scales,
               const uint32_t* qzeros, int symmetric, int group_size, uint16_t* Y, void* workspace,
               size_t* workspace_bytes, void* stream) {
  int st = check_weight_shape(N, K, group_size);
  if (st) return st;
  if (M < 0) return W4_ERR_SHAPE;
  if ((st = gemm_check_size(M, K, N))) return st;
  const size_t need = gemm_workspace_bytes(M, K, N);
  if (!workspace && workspace_bytes) {
    *workspace_bytes = need;
    return W4_OK;
  }
  if (need > 0 && (!workspace || !workspace_bytes || *workspace_bytes < need)) return W4_ERR_WORKSPACE;
  if (!X || !Y) return W4_ERR_NULL;
  st = check_packed(qweight, scales, qzeros, symmetric);
  if (st) return st;
  if (misaligned(X) || misaligned(Y) || misaligned(workspace)) return W4_ERR_ALIGN;
  return launch_gemm(X, M, K, N, qweight, scales, qzeros, symmetric, Y, workspace,
                     static_cast<hipStream_t>(stream));
}

int w4_bf16_linear(const uint16_t* X, int M, int K, int N, const uint16_t* W, uint16_t* Y, void* stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 64 || (long long)M * K >= (1LL << 31) || (long long)N * K >= (1LL << 31))
    return W4_ERR_SHAPE;
  if (M == 0 || N == 0) return W4_OK;
  if (!X || !W || !Y) return W4_ERR_NULL;
  if (misaligned(X) || misaligned(W) || misaligned(Y)) return W4_ERR_ALIGN;
  return launch_bf16_gemm(X, M, K, N, W, Y, static_cast<hipStream_t>(stream));
}

int awq_grid_loss(const uint16_t* X, int T, int K, int N, const uint16_t* W, const uint16_t* Yref,
                  const float* S, const float* ratios, int C, int symmetric, int group_size, float* losses,
                  void* workspace, size_t* workspace_bytes, void* stream) {
  int st = check_weight_shape(N, K, group_size);
  if (st) return st;
  if (T <= 0 || N <= 0 || C < 0) return W4_ERR_SHAPE;
  if ((st = grid_loss_check_size(T, K, N, C))) return st;
  if (symmetric != 0 && symmetric != 1) return W4_ERR_VALUE;
  const size_t need = grid_loss_workspace_bytes(T, K, N, C, Yref == nullptr);
  if (!workspace) {
    if (!workspace_bytes) return need ? W4_ERR_WORKSPACE : W4_OK;
    *workspace_bytes = need;
    return W4_OK;
  }
  if (!workspace_bytes || *workspace_bytes < need) return W4_ERR_WORKSPACE;
  if (!X || !W || !S || !ratios || !losses) return W4_ERR_NULL;
  if (misaligned(X) || misaligned(W) || misaligned(Yref) || misaligned(S) || misaligned(workspace))
    return W4_ERR_ALIGN;
  if (C == 0) return W4_OK;
  return launch_grid_loss(X, T, K, N, W, Yref, S, ratios, C, symmetric, losses, workspace,
                          static_cast<hipStream_t>(stream));
}

int awq_clip_search(const uint16_t* X, int T, int K, int N, const uint16_t* W, const float* s,
                    const float* ratios, int R, int symmetric, int group_size, float* losses, uint8_t* best,
                    void* workspace, size_t* workspace_bytes, void* stream) {
  int st = check_weight_shape(N, K, group_size);
  if (st) return st;
  if (T < 0) return W4_ERR_SHAPE;
  if (symmetric != 0 && symmetric != 1) return W4_ERR_VALUE;
  if (R < 1 || R > 64) return W4_ERR_VALUE;
  const size_t need = clip_search_workspace_bytes(T, K);
  if (!workspace) {
    if (!workspace_bytes) return W4_ERR_WORKSPACE;
    *workspace_bytes = need;
    return W4_OK;
  }
  if (!workspace_bytes || *workspace_bytes < need) return W4_ERR_WORKSPACE;
  if (N == 0) return W4_OK;
  if ((T > 0 && !X) || !W || !ratios || !best) return W4_ERR_NULL;
  if (misaligned(X) || misaligned(W) || misaligned(s) || misaligned(workspace)) return W4_ERR_ALIGN;
  return launch_clip_search(X, T, K, N, W, s, ratios, R, symmetric, losses, best, workspace,
                            static_cast<hipStream_t>(stream));
}

namespace {
int check_block_shape(int B, int L, int H, int nq, int nkv, int I) {
  if (B < 1 || L < 1 || H < kGroup || H % kGroup || I < kGroup || I % kGroup || nkv < 1 || nq < nkv || nq % nkv)
    return W4_ERR_SHAPE;
  const long long T = (long long)B * L;
  const long long wide = std::max<long long>(std::max<long long>(H, I), 128LL * nq);
  if ((T + 64) * wide >= (1LL << 31) || (long long)I * H >= (1LL << 31) || 128LL * nq * H >= (1LL << 31) ||
      L > 65535LL * 64 || nq > 65535 || B > 65535)
    return W4_ERR_SHAPE;
  return W4_OK;
}
bool block_null(const w4_block* b) {
  return !b || !b->norm1 || !b->wq || !b->wk || !b->wv || !b->wo || !b->norm2 || !b->wgate || !b->wup || !b->wdown;
}
bool block_misaligned(const w4_block* b) {
  return misaligned(b->norm1) || misaligned(b->wq) || misaligned(b->wk) || misaligned(b->wv) || misaligned(b->wo) ||
         misaligned(b->norm2) || misaligned(b->wgate) || misaligned(b->wup) || misaligned(b->wdown);
}
}  // namespace

int w4_block_forward(const uint16_t* X, int B, int L, int hidden, int n_q, int n_kv, int inter,
                     const w4_block* blk, uint16_t* Y, void* workspace, size_t* workspace_bytes, void* stream) {
  int st = check_block_shape(B, L, hidden, n_q, n_kv, inter);
  if (st) return st;
  const size_t need = block_forward_workspace_bytes(B, L, hidden, n_q, n_kv, inter);
  if (!workspace) {
    if (!workspace_bytes) return W4_ERR_WORKSPACE;
    *workspace_bytes = need;
    return W4_OK;
  }
  if (!workspace_bytes || *workspace_bytes < need) return W4_ERR_WORKSPACE;
  if (!X || !Y || block_null(blk)) return W4_ERR_NULL;
  if (misaligned(X) || misaligned(Y) || misaligned(workspace) || block_misaligned(blk)) return W4_ERR_ALIGN;
  return launch_block_forward(X, B, L, hidden, n_q, n_kv, inter, *blk, Y, workspace, static_cast<hipStream_t>(stream));
}

int w4_block_forward_quantized(const uint16_t* X, int B, int L, int hidden, int n_q, int n_kv, int inter,
                               const w4_block* blk, int linear, const float* s, const uint32_t* qweight,
                               const uint16_t* scales, const uint32_t* qzeros, int symmetric, int group_size,
                               uint16_t* Y, void* workspace, size_t* workspace_bytes, void* stream) {
  if (group_size != kGroup) return W4_ERR_UNSUPPORTED;
  int st = check_block_shape(B, L, hidden, n_q, n_kv, inter);
  if (st) return st;
  if (linear < 0 || linear > 6 || (symmetric != 0 && symmetric != 1)) return W4_ERR_VALUE;
  const size_t need = block_quantized_workspace_bytes(B, L, hidden, n_q, n_kv, inter, linear);
  if (!workspace) {
    if (!workspace_bytes) return W4_ERR_WORKSPACE;
    *workspace_bytes = need;
    return W4_OK;
  }
  if (!workspace_bytes || *workspace_bytes < need) return W4_ERR_WORKSPACE;
  if (!X || !Y || !s || block_null(blk)) return W4_ERR_NULL;
  st = check_packed(qweight, scales, qzeros, symmetric);
  if (st) return st;
  if (misaligned(X) || misaligned(Y) || misaligned(s) || misaligned(workspace) || block_misaligned(blk))
    return W4_ERR_ALIGN;
  return launch_block_forward_quantized(X, B, L, hidden, n_q, n_kv, inter, *blk, linear, s, qweight, scales, qzeros,
                                        symmetric, Y, workspace, static_cast<hipStream_t>(stream));
}

int awq_lookahead_loss(const uint16_t* X, int B, int L, int hidden, int n_q, int n_kv, int inter,
                       const w4_block* blk, const w4_block* next, int linear, const float* S,
                       const float* ratios, int C, int symmetric, int group_size, float* losses,
                       float* losses_d0, void* workspace, size_t* workspace_bytes, void* stream) {
  if (group_size != kGroup) return W4_ERR_UNSUPPORTED;
  int st = check_block_shape(B, L, hidden, n_q, n_kv, inter);
  if (st) return st;
  if (linear < 0 || linear > 6 || C < 0 || (symmetric != 0 && symmetric != 1)) return W4_ERR_VALUE;
  const size_t need = lookahead_workspace_bytes(B, L, hidden, n_q, n_kv, inter, linear);
  if (!workspace) {
    if (!workspace_bytes) return W4_ERR_WORKSPACE;
    *workspace_bytes = need;
    return W4_OK;
  }
  if (!workspace_bytes || *workspace_bytes < need) return W4_ERR_WORKSPACE;
  if (C == 0) return W4_OK;
  if (!X || !S || !ratios || !losses || block_null(blk) || (next && block_null(next))) return W4_ERR_NULL;
  if (misaligned(X) || misaligned(workspace) || block_misaligned(blk) || (next && block_misaligned(next)))
    return W4_ERR_ALIGN;
  return launch_lookahead_loss(X, B, L, hidden, n_q, n_kv, inter, *blk, next, linear, S, ratios, C, symmetric,
                               losses, losses_d0, workspace, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

constexpr int kActRows = 64;

struct SearchLayout {
  size_t yref, grid, S, ratios, losses, m, total;
  size_t grid_bytes;
};

SearchLayout search_layout(int T, int K, int N, int C) {
  SearchLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  L.yref = take((size_t)T * N * 2);
  L.grid_bytes = grid_loss_workspace_bytes(T, K, N, C, false);
  L.grid = take(L.grid_bytes);
  L.S = take((size_t)C * K * 4);
  L.ratios = take((size_t)C * 4);
  L.losses = take((size_t)C * 4);
  const int chunks = (T + kActRows - 1) / kActRows;
  L.m = take((size_t)(1 + chunks) * K * 8);
  L.total = off;
  return L;
}

// s(alpha)_k = max(m_k^alpha, 1e-4) / sqrt(max_j p_j min_j p_j) on the host in fp64,
// stored fp32: row i of S for alphas[i].
void alpha_scales(const std::vector<double>& m, const double* alphas, int n_alpha, std::vector<float>& S) {
  const int K = (int)m.size();
  // row i of S from alpha i alone: the rows are independent, so host threads take
  // interleaved rows (same arithmetic per row, whichever thread computes it)
  auto rows = [&](int first, int step) {
    std::vector<double> p(K);
    for (int i = first; i < n_alpha; i += step) {
      double pmax = 0.0, pmin = INFINITY;
      for (int k = 0; k < K; ++k) {
        const double v = pow(m[k], alphas[i]);
        p[k] = v > 1e-4 ? v : 1e-4;
        pmax = p[k] > pmax ? p[k] : pmax;
        pmin = p[k] < pmin ? p[k] : pmin;
      }
      const double d = sqrt(pmax * pmin);
      for (int k = 0; k < K; ++k) S[(size_t)i * K + k] = (float)(p[k] / d);
    }
  };
  const unsigned hw = std::thread::hardware_concurrency();
  const int nt = std::max(1, std::min({n_alpha, 8, (int)(hw > 1 ? hw / 2 : 1)}));
  std::vector<std::thread> pool;
  int started = 1;                     // threads running (this one included)
  try {
    for (; started < nt; ++started) pool.emplace_back(rows, started, nt);
  } catch (...) {
    // a thread that could not start leaves its rows to this one
  }
  rows(0, nt);
  for (int t = started; t < nt; ++t) rows(t, nt);
  for (auto& th : pool) th.join();
}

// An event recorded on a stream, destroyed with its scope.
struct ScopedEvent {
  hipEvent_t ev = nullptr;
  ScopedEvent() {
    if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) ev = nullptr;
  }
  ~ScopedEvent() {
    if (ev) (void)hipEventDestroy(ev);
  }
};

int first_argmin(const std::vector<float>& v) {
  int best = 0;
  for (int i = 1; i < (int)v.size(); ++i)
    if (v[i] < v[best]) best = i;
  return best;
}

int search_impl(const uint16_t* X, int T, int K, int N, const uint16_t* W, const double* alphas, int n_alpha,
                const double* ratios, int n_ratio, int symmetric, float* losses_out, int* alpha_index,
                int* ratio_index, float* s_out, char* ws, const SearchLayout& L, hipStream_t stream) {
  const int C = n_alpha > n_ratio ? n_alpha : n_ratio;
  uint16_t* yref = reinterpret_cast<uint16_t*>(ws + L.yref);
  void* grid_ws = ws + L.grid;
  float* dS = reinterpret_cast<float*>(ws + L.S);
  float* dR = reinterpret_cast<float*>(ws + L.ratios);
  float* dL = reinterpret_cast<float*>(ws + L.losses);
  double* dm = reinterpret_cast<double*>(ws + L.m);

  int st = launch_act_mean_abs(X, T, K, dm, stream);
  if (st) return st;
  std::vector<double> m(K);
  ScopedEvent m_ready;
  if (!m_ready.ev || hipMemcpyAsync(m.data(), dm, (size_t)K * 8, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipEventRecord(m_ready.ev, stream) != hipSuccess)
    return W4_ERR_HIP;
  // Y_ref = bf16(X W^T) once for both phases, through the bf16-weight MFMA path; it
  // runs while the host computes s(alpha) from the statistic
  st = launch_reference_gemm(X, T, K, N, W, yref, stream);
  if (st) return st;
  if (hipEventSynchronize(m_ready.ev) != hipSuccess) return W4_ERR_HIP;

  std::vector<float> S((size_t)C * K), R(C, 1.0f);
  alpha_scales(m, alphas, n_alpha, S);
  if (hipMemcpyAsync(dS, S.data(), (size_t)n_alpha * K * 4, hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipMemcpyAsync(dR, R.data(), (size_t)n_alpha * 4, hipMemcpyHostToDevice, stream) != hipSuccess)
    return W4_ERR_HIP;
  st = launch_grid_loss(X, T, K, N, W, yref, dS, dR, n_alpha, symmetric, dL, grid_ws, stream);
  if (st) return st;
  std::vector<float> la(n_alpha);
  if (hipMemcpyAsync(la.data(), dL, (size_t)n_alpha * 4, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return W4_ERR_HIP;
  const int ia = first_argmin(la);

  // phase 2: every ratio at s(alpha*)
  const std::vector<float> s_star(S.begin() + (size_t)ia * K, S.begin() + (size_t)(ia + 1) * K);
  for (int j = 0; j < n_ratio; ++j) {
    memcpy(&S[(size_t)j * K], s_star.data(), (size_t)K * 4);
    R[j] = (float)ratios[j];
  }
  if (hipMemcpyAsync(dS, S.data(), (size_t)n_ratio * K * 4, hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipMemcpyAsync(dR, R.data(), (size_t)n_ratio * 4, hipMemcpyHostToDevice, stream) != hipSuccess)
    return W4_ERR_HIP;
  st = launch_grid_loss(X, T, K, N, W, yref, dS, dR, n_ratio, symmetric, dL, grid_ws, stream, true);
  if (st) return st;
  std::vector<float> lr(n_ratio);
  if (hipMemcpyAsync(lr.data(), dL, (size_t)n_ratio * 4, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipMemcpyAsync(s_out, dS, (size_t)K * 4, hipMemcpyDeviceToDevice, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return W4_ERR_HIP;
  const int ir = first_argmin(lr);
  memcpy(losses_out, la.data(), (size_t)n_alpha * 4);
  memcpy(losses_out + n_alpha, lr.data(), (size_t)n_ratio * 4);
  *alpha_index = ia;
  *ratio_index = ir;
  return W4_OK;
}

}  // namespace

extern "C" int awq_search(const uint16_t* X, int T, int K, int N, const uint16_t* W, const double* alphas,
                          int n_alpha, const double* ratios, int n_ratio, int symmetric, int group_size,
                          float* losses_out, int* alpha_index, int* ratio_index, float* s_out, void* workspace,
                          size_t* workspace_bytes, void* stream) {
  int st = check_weight_shape(N, K, group_size);
  if (st) return st;
  if (T <= 0 || N <= 0) return W4_ERR_SHAPE;
  if (n_alpha < 1 || n_alpha > 64 || n_ratio < 1 || n_ratio > 64) return W4_ERR_VALUE;
  if (symmetric != 0 && symmetric != 1) return W4_ERR_VALUE;
  if (!alphas || !ratios) return W4_ERR_NULL;
  for (int i = 0; i < n_alpha; ++i)
    if (!(alphas[i] >= 0.0 && alphas[i] <= 16.0)) return W4_ERR_VALUE;
  for (int j = 0; j < n_ratio; ++j)
    if (!(ratios[j] > 0.0 && ratios[j] <= 1.0)) return W4_ERR_VALUE;
  const int C = n_alpha > n_ratio ? n_alpha : n_ratio;
  if ((st = grid_loss_check_size(T, K, N, C))) return st;
  const SearchLayout L = search_layout(T, K, N, C);
  if (!workspace && workspace_bytes) {
    *workspace_bytes = L.total;
    return W4_OK;
  }
  if (!workspace || !workspace_bytes || *workspace_bytes < L.total) return W4_ERR_WORKSPACE;
  if (!X || !W || !losses_out || !alpha_index || !ratio_index || !s_out) return W4_ERR_NULL;
  if (misaligned(X) || misaligned(W) || misaligned(s_out) || misaligned(workspace)) return W4_ERR_ALIGN;
  return search_impl(X, T, K, N, W, alphas, n_alpha, ratios, n_ratio, symmetric, losses_out, alpha_index,
                     ratio_index, s_out, static_cast<char*>(workspace), L, static_cast<hipStream_t>(stream));
}

namespace {

struct LookSearchLayout {
  size_t look, S, R, L, m, total;
};

LookSearchLayout look_search_layout(int B, int L, int H, int nq, int nkv, int I, int linear, int C) {
  LookSearchLayout l{};
  const int K = lookahead_input_size(H, nq, I, linear);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  l.look = take(lookahead_workspace_bytes(B, L, H, nq, nkv, I, linear));
  l.S = take((size_t)C * K * 4);
  l.R = take((size_t)C * 4);
  l.L = take((size_t)C * 4);
  l.m = take((size_t)(1 + ((long long)B * L + kActRows - 1) / kActRows) * K * 8);
  l.total = off;
  return l;
}

int look_search_impl(const uint16_t* X, int B, int L, int H, int nq, int nkv, int I, const w4_block& blk,
                     const w4_block* next, int linear, const double* alphas, int n_alpha, const double* ratios,
                     int n_ratio, int symmetric, float* losses_out, int* alpha_index, int* ratio_index,
                     float* s_out, char* ws, const LookSearchLayout& l, hipStream_t stream) {
  const int K = lookahead_input_size(H, nq, I, linear);
  const int C = std::max(n_alpha, n_ratio);
  void* lw = ws + l.look;
  float* dS = reinterpret_cast<float*>(ws + l.S);
  float* dR = reinterpret_cast<float*>(ws + l.R);
  float* dL = reinterpret_cast<float*>(ws + l.L);
  double* dm = reinterpret_cast<double*>(ws + l.m);
  // the statistic reaches the host right after block i; the host computes s(alpha)
  // while block i + 1 of the reference runs
  std::vector<double> m(K);
  ScopedEvent m_ready;
  if (!m_ready.ev) return W4_ERR_HIP;
  int st = launch_lookahead_reference(X, B, L, H, nq, nkv, I, blk, next, linear, dm, lw, stream, m.data(),
                                      m_ready.ev);
  if (st) return st;
  if (hipEventSynchronize(m_ready.ev) != hipSuccess) return W4_ERR_HIP;
  std::vector<float> S((size_t)C * K), R(C, 1.0f);
  alpha_scales(m, alphas, n_alpha, S);
  if (hipMemcpyAsync(dS, S.data(), (size_t)n_alpha * K * 4, hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipMemcpyAsync(dR, R.data(), (size_t)n_alpha * 4, hipMemcpyHostToDevice, stream) != hipSuccess)
    return W4_ERR_HIP;
  st = launch_lookahead_candidates(X, B, L, H, nq, nkv, I, blk, next, linear, dS, dR, n_alpha, symmetric, dL,
                                   nullptr, lw, stream);
  if (st) return st;
  std::vector<float> la(n_alpha);
  if (hipMemcpyAsync(la.data(), dL, (size_t)n_alpha * 4, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return W4_ERR_HIP;
  const int ia = first_argmin(la);
  const std::vector<float> s_star(S.begin() + (size_t)ia * K, S.begin() + (size_t)(ia + 1) * K);
  for (int j = 0; j < n_ratio; ++j) {
    memcpy(&S[(size_t)j * K], s_star.data(), (size_t)K * 4);
    R[j] = (float)ratios[j];
  }
  if (hipMemcpyAsync(dS, S.data(), (size_t)n_ratio * K * 4, hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipMemcpyAsync(dR, R.data(), (size_t)n_ratio * 4, hipMemcpyHostToDevice, stream) != hipSuccess)
    return W4_ERR_HIP;
  st = launch_lookahead_candidates(X, B, L, H, nq, nkv, I, blk, next, linear, dS, dR, n_ratio, symmetric, dL,
                                   nullptr, lw, stream);
  if (st) return st;
  std::vector<float> lr(n_ratio);
  if (hipMemcpyAsync(lr.data(), dL, (size_t)n_ratio * 4, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipMemcpyAsync(s_out, dS, (size_t)K * 4, hipMemcpyDeviceToDevice, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return W4_ERR_HIP;
  memcpy(losses_out, la.data(), (size_t)n_alpha * 4);
  memcpy(losses_out + n_alpha, lr.data(), (size_t)n_ratio * 4);
  *alpha_index = ia;
  *ratio_index = first_argmin(lr);
  return W4_OK;
}

}  // namespace

extern "C" int awq_search_lookahead(const uint16_t* X, int B, int L, int hidden, int n_q, int n_kv, int inter,
                                    const w4_block* blk, const w4_block* next, int linear, const double* alphas,
                                    int n_alpha, const double* ratios, int n_ratio, int symmetric, int group_size,
                                    float* losses_out, int* alpha_index, int* ratio_index, float* s_out,
                                    void* workspace, size_t* workspace_bytes, void* stream) {
  if (group_size != kGroup) return W4_ERR_UNSUPPORTED;
  int st = check_block_shape(B, L, hidden, n_q, n_kv, inter);
  if (st) return st;
  if (linear < 0 || linear > 6 || (symmetric != 0 && symmetric != 1)) return W4_ERR_VALUE;
  if (n_alpha < 1 || n_alpha > 64 || n_ratio < 1 || n_ratio > 64) return W4_ERR_VALUE;
  if (!alphas || !ratios) return W4_ERR_NULL;
  for (int i = 0; i < n_alpha; ++i)
    if (!(alphas[i] >= 0.0 && alphas[i] <= 16.0)) return W4_ERR_VALUE;
  for (int j = 0; j < n_ratio; ++j)
    if (!(ratios[j] > 0.0 && ratios[j] <= 1.0)) return W4_ERR_VALUE;
  const LookSearchLayout l =
      look_search_layout(B, L, hidden, n_q, n_kv, inter, linear, std::max(n_alpha, n_ratio));
  if (!workspace && workspace_bytes) {
    *workspace_bytes = l.total;
    return W4_OK;
  }
  if (!workspace || !workspace_bytes || *workspace_bytes < l.total) return W4_ERR_WORKSPACE;
  if (!X || !losses_out || !alpha_index || !ratio_index || !s_out || block_null(blk) || (next && block_null(next)))
    return W4_ERR_NULL;
  if (misaligned(X) || misaligned(s_out) || misaligned(workspace) || block_misaligned(blk) ||
      (next && block_misaligned(next)))
    return W4_ERR_ALIGN;
  return look_search_impl(X, B, L, hidden, n_q, n_kv, inter, *blk, next, linear, alphas, n_alpha, ratios, n_ratio,
                          symmetric, losses_out, alpha_index, ratio_index, s_out, static_cast<char*>(workspace), l,
                          static_cast<hipStream_t>(stream));
}
