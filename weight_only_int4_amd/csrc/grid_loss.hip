// Batched fake-quant loss of AWQ candidates, model card "rebuttal_w4g128_awq_w2":
// the scale-rewrite paragraph (a candidate (s, r) is simulated with the weight
// Q(W diag(s)) diag(1/s); the deployed form feeds X diag(1/s) -- the previous
// op's output divided by s, stored in bf16 -- to the int4 weight Q(W diag(s)));
// details-table row "Search" and "Clipping granularity" (s from the scale
// exponent grid; one global shrink ratio per linear).
//
// Steps, all on the caller's stream:
//   1. (Yref == NULL) Y_ref = bf16(X W^T) with the MFMA core and bf16 weights.
//   2. Q_c = quantize_pack(W diag(s_c), r_c) for every candidate (one launch).
//   3. Xs_c = bf16(X / s_c) and the group row sums of Xs_c.
//   4. MFMA core with int4 weights Q_c and a squared-difference epilogue against
//      Y_ref: one fp32 partial sum per 128x128 tile.
//   5. losses[c] = (fixed-order fp64 sum of the tile partials) / (T N).
#include "gemm_core.hpp"

#pragma clang fp contract(off)

namespace w4 {

namespace {

struct LossLayout {
  size_t yref, qw, sc, qz, xs, rsq, szq, part, total;
  int mpad, npad, G, GW, tiles;
};

LossLayout loss_layout(int T, int K, int N, int C, bool need_yref) {
  LossLayout L{};
  L.G = K / kGroup;
  L.GW = (L.G + 7) / 8;
  L.mpad = (int)align_up((size_t)T, kBM);
  L.npad = gemm_npad(N);
  L.tiles = ((N + kBN - 1) / kBN) * ((T + kBM - 1) / kBM);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  L.yref = need_yref ? take((size_t)T * N * 2) : 0;
  L.qw = take((size_t)C * N * (K / 8) * 4);
  L.sc = take((size_t)C * N * L.G * 2);
  L.qz = take((size_t)C * N * L.GW * 4);
  L.xs = take((size_t)C * L.mpad * K * 2);
  L.rsq = take((size_t)C * L.G * L.mpad * 8);
  L.szq = take((size_t)C * L.G * L.npad * 4);
  L.part = take((size_t)C * L.tiles * 4);
  L.total = off;
  return L;
}

// Xs[c][t][k] = bf16(X[t][k] / S[c][k]) (IEEE division, round to nearest even),
// stored pair-arranged for the int4 MFMA path: each 8-channel run as
// (x0,x4)(x1,x5)(x2,x6)(x3,x7); Xs[c] has tpad rows, rows T .. tpad-1 zero.
// Each thread handles 8 consecutive channels of one row.
__global__ __launch_bounds__(256) void scale_activations_kernel(const uint16_t* X, int T, int tpad, int K,
                                                                const float* S, uint16_t* Xs) {
  const int c = blockIdx.z;
  const size_t chunks = (size_t)tpad * (K / 8);
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= chunks) return;
  const size_t t = i / (K / 8);
  const int k0 = (int)(i % (K / 8)) * 8;
  uint4* dst = reinterpret_cast<uint4*>(Xs + (size_t)c * tpad * K + t * K + k0);
  if ((int)t >= T) {
    *dst = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const uint4 v = *reinterpret_cast<const uint4*>(X + t * K + k0);
  const float4 s0 = *reinterpret_cast<const float4*>(S + (size_t)c * K + k0);
  const float4 s1 = *reinterpret_cast<const float4*>(S + (size_t)c * K + k0 + 4);
  const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float lo = __uint_as_float(d[q] << 16) / s[2 * q];
    const float hi = __uint_as_float(d[q] & 0xFFFF0000u) / s[2 * q + 1];
    o[q] = f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
  }
  uint32_t e[4];
  pair_activations(o, e);
  *dst = make_uint4(e[0], e[1], e[2], e[3]);
}

// losses[c] = sum_tiles partials[c][tile] (fp64, tile order) / (T N); one wave per c,
// lane-strided fp64 partial sums combined in a fixed butterfly order.
__global__ __launch_bounds__(64) void loss_reduce_kernel(const float* partials, int tiles, double inv_count,
                                                         float* losses) {
  const int c = blockIdx.x;
  const int lane = threadIdx.x;
  // loads issued 16 at a time, added in the same ascending order
  const float* pc = partials + (size_t)c * tiles;
  double s = 0.0;
  int t = lane;
  for (; t + 64 * 15 < tiles; t += 64 * 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = pc[t + 64 * u];
#pragma unroll
    for (int u = 0; u < 16; ++u) s += (double)v[u];
  }
  for (; t < tiles; t += 64) s += (double)pc[t];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) losses[c] = (float)(s * inv_count);
}

// partial[chunk][k] = sum over rows of chunk of |X[t][k]| (fp64).
__global__ __launch_bounds__(256) void act_abs_partial_kernel(const uint16_t* X, int T, int K, int rows,
                                                              double* partial) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  const int t0 = blockIdx.y * rows;
  const int t1 = min(t0 + rows, T);
  // loads issued 8 at a time, added in the same ascending order
  double s = 0.0;
  int t = t0;
  for (; t + 7 < t1; t += 8) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = X[(size_t)(t + u) * K + k];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += (double)fabsf(bf16_bits_to_f32(v[u]));
  }
  for (; t < t1; ++t) s += (double)fabsf(bf16_bits_to_f32(X[(size_t)t * K + k]));
  partial[(size_t)blockIdx.y * K + k] = s;
}

__global__ __launch_bounds__(256) void act_abs_finish_kernel(const double* partial, int chunks, int K, int T,
                                                             double* m) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  // loads issued 8 at a time, added in the same ascending order
  double s = 0.0;
  int c = 0;
  for (; c + 7 < chunks; c += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = partial[(size_t)(c + u) * K + k];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; c < chunks; ++c) s += partial[(size_t)c * K + k];
  m[k] = s / (double)T;
}

}  // namespace

// 32-bit per-lane byte offsets in the cores: the scaled activations (2 x (T + 64) x K
// bytes) and the bf16 reference weights (2 N K bytes) below 2^32; C candidates on
// grid.z.
int grid_loss_check_size(int T, int K, int N, int C) {
  if (((long long)T + kBM) * K >= (1LL << 31) || (long long)N * K >= (1LL << 31) || C > 65535) return W4_ERR_SHAPE;
  return W4_OK;
}

size_t grid_loss_workspace_bytes(int T, int K, int N, int C, bool need_yref) {
  if (T <= 0 || K <= 0 || N <= 0 || C <= 0) return 0;
  return loss_layout(T, K, N, C, need_yref).total;
}

int launch_grid_loss(const uint16_t* X, int T, int K, int N, const uint16_t* W, const uint16_t* Yref,
                     const float* S, const float* ratios, int C, int symmetric, float* losses,
                     void* workspace, hipStream_t stream, bool shared_s) {
  if (C == 0) return W4_OK;
  if (int st = grid_loss_check_size(T, K, N, C)) return st;
  const LossLayout L = loss_layout(T, K, N, C, Yref == nullptr);
  char* ws = static_cast<char*>(workspace);
  const dim3 tile_grid((unsigned)L.tiles, 1, 1);

  if (Yref == nullptr) {
    uint16_t* yref = reinterpret_cast<uint16_t*>(ws + L.yref);
    const int st0 = launch_reference_gemm(X, T, K, N, W, yref, stream);
    if (st0 != W4_OK) return st0;
    Yref = yref;
  }

  uint32_t* qw = reinterpret_cast<uint32_t*>(ws + L.qw);
  uint16_t* sc = reinterpret_cast<uint16_t*>(ws + L.sc);
  uint32_t* qz = reinterpret_cast<uint32_t*>(ws + L.qz);
  uint16_t* xs = reinterpret_cast<uint16_t*>(ws + L.xs);
  uint16_t* rsq = reinterpret_cast<uint16_t*>(ws + L.rsq);
  uint32_t* szq = reinterpret_cast<uint32_t*>(ws + L.szq);
  float* part = reinterpret_cast<float*>(ws + L.part);

  QuantArgs q{};
  q.W = W;
  q.N = N;
  q.K = K;
  q.s = S;
  q.s_stride = (size_t)K;
  q.ratio = 1.0f;
  q.ratios = ratios;
  q.symmetric = symmetric;
  q.qweight = qw;
  q.qw_stride = (size_t)N * (K / 8);
  q.scales = sc;
  q.sc_stride = (size_t)N * L.G;
  q.qzeros = symmetric ? nullptr : qz;
  q.qz_stride = (size_t)N * L.GW;
  int st = launch_quantize_pack(q, C, stream);
  if (st != W4_OK) return st;

  const size_t chunks = (size_t)L.mpad * (K / 8);
  // one scaled copy of X per candidate, or one for all when they share s
  const int CX = shared_s ? 1 : C;
  hipLaunchKernelGGL(scale_activations_kernel, dim3((unsigned)((chunks + 255) / 256), 1, (unsigned)CX), dim3(256), 0,
                     stream, X, T, L.mpad, K, S, xs);
  W4_CHECK_LAUNCH();
  st = launch_gemm_prep(xs, (size_t)L.mpad * K, T, K, L.mpad, sc, q.sc_stride, symmetric ? nullptr : qz,
                        q.qz_stride, symmetric, N, rsq, (size_t)L.G * L.mpad * 4, szq, (size_t)L.G * L.npad, nullptr,
                        C, stream, CX);
  if (st != W4_OK) return st;

  GemmCoreArgs a{};
  a.X = xs;
  a.x_stride = shared_s ? 0 : (size_t)L.mpad * K;
  a.M = T;
  a.K = K;
  a.N = N;
  a.qweight = qw;
  a.qw_stride = q.qw_stride;
  a.rsq = rsq;
  a.rsq_stride = shared_s ? 0 : (size_t)L.G * L.mpad * 4;
  a.szq = szq;
  a.szq_stride = (size_t)L.G * L.npad;
  a.mpad = L.mpad;
  a.npad = L.npad;
  a.Yref = Yref;
  a.partials = part;
  dim3 grid = tile_grid;
  grid.z = (unsigned)C;
  if (gemm_core_wide((long long)grid.x * grid.y * grid.z))
    hipLaunchKernelGGL((gemm_core_kernel<EPI_SQDIFF, true>), grid, dim3(kGemmWaves * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_core_kernel<EPI_SQDIFF>), grid, dim3(kGemmWaves * 64), 0, stream, a);
  W4_CHECK_LAUNCH();

  hipLaunchKernelGGL(loss_reduce_kernel, dim3((unsigned)C), dim3(64), 0, stream, part, L.tiles,
                     1.0 / ((double)T * (double)N), losses);
  W4_CHECK_LAUNCH();
  return W4_OK;
}

int launch_reference_gemm(const uint16_t* X, int M, int K, int N, const uint16_t* W, uint16_t* Y,
                          hipStream_t stream) {
  return launch_bf16_gemm(X, M, K, N, W, Y, stream);
}

int launch_act_mean_abs(const uint16_t* X, int T, int K, double* m, hipStream_t stream) {
  const int rows = 64;
  const int chunks = (T + rows - 1) / rows;
  double* partial = m + K;
  hipLaunchKernelGGL(act_abs_partial_kernel, dim3((unsigned)((K + 255) / 256), (unsigned)chunks), dim3(256), 0,
                     stream, X, T, K, rows, partial);
  W4_CHECK_LAUNCH();
  hipLaunchKernelGGL(act_abs_finish_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, stream, partial,
                     chunks, K, T, m);
  W4_CHECK_LAUNCH();
  return W4_OK;
}

}  // namespace w4
