// Look-ahead block scoring, model card "rebuttal_w4g128_awq_w2", details table row
// "Search" and the paragraph under it: a candidate for a linear of block i is scored
// at the output of block i + 1, which runs unquantized; the reference runs block i
// unquantized too; the last block is scored at its own output.  The block is the
// base model's decoder block (same card, "Base model": Qwen3-1.7B, hidden 2048;
// model page "qwen3-1.7b_q326_channel", architecture notes: grouped-query attention
// with 16 query heads over 8 key/value heads of size 128, rotary positions with base
// 10^6, SiLU-gated feed-forward of width 6144).
//
// Readings fixed here: pre-norm RMSNorm (eps 1e-6) before attention and before the
// feed-forward, residual adds after each, no biases and no per-head q/k norms;
// rotary embedding on the pairs (j, j + 64) of each head at the token's position in
// its sequence; causal attention within each of B sequences of L tokens, scale
// 1/sqrt(128), query head h reading key/value head h / (n_q / n_kv); every op output
// is stored in bf16 (round to nearest even) and computed in fp32.
//
// Block forward, all on the caller's stream:
//   a = rmsnorm(x, g1); q, k, v = a Wq^T, a Wk^T, a Wv^T; q, k = rope(q), rope(k);
//   o = attention(q, k, v); h = x + o Wo^T; b = rmsnorm(h, g2);
//   m = silu(b Wg^T) * (b Wu^T); y = h + m Wd^T.
// The unquantized projections run on the library's bf16 MFMA kernel (fp32
// accumulation; q, k, v as one launch with the rotary embedding of q and k in its
// epilogue, and gate, up as one launch storing silu(gate) up, since each group reads
// the same input; the epilogues compute exactly what the standalone rope and
// elementwise kernels do); a candidate linear runs as deployed: bf16(input / s)
// against its int4 codes Q(W diag(s), r) on the library's int4 GEMM, with the
// standalone kernels around it.
#include <math.h>

#include <algorithm>

#include "block_ops.hpp"
#include "internal.hpp"

#pragma clang fp contract(off)

namespace w4 {

namespace {

constexpr int kHd = 128;              // head size
constexpr float kEps = 1e-6f;
constexpr double kRopeBase = 1e6;

// ---------------------------------------------------------------------------------------
// y = bf16((x * r) * g), r = 1 / sqrt(mean(x^2) + eps): one wave per row, fp32 sums in a
// fixed order (lane-strided, then a butterfly).
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ X, int T, int H,
                                                      const uint16_t* __restrict__ g, uint16_t* __restrict__ Y) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= T) return;
  const uint16_t* x = X + (size_t)row * H;
  float ss = 0.0f;
  for (int c = lane * 8; c < H; c += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(x + c);
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a = __uint_as_float(d[q] << 16), b = __uint_as_float(d[q] & 0xFFFF0000u);
      ss = ss + a * a;
      ss = ss + b * b;
    }
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)H + kEps);
  for (int c = lane * 8; c < H; c += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(x + c);
    const uint4 gv = *reinterpret_cast<const uint4*>(g + c);
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
    const uint32_t e[4] = {gv.x, gv.y, gv.z, gv.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = (__uint_as_float(d[q] << 16) * r) * __uint_as_float(e[q] << 16);
      const float hi = (__uint_as_float(d[q] & 0xFFFF0000u) * r) * __uint_as_float(e[q] & 0xFFFF0000u);
      o[q] = f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
    }
    *reinterpret_cast<uint4*>(Y + (size_t)row * H + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// cos / sin [L][64] of p * base^(-2j/128), in fp64, stored fp32.
__global__ __launch_bounds__(256) void rope_table_kernel(int L, float* cs, float* sn) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= L * 64) return;
  const int p = i >> 6, j = i & 63;
  const double ang = (double)p * pow(kRopeBase, -(2.0 * j) / kHd);
  cs[i] = (float)cos(ang);
  sn[i] = (float)sin(ang);
}

// In place on x [T][nh * 128] (T = B L, token t at position t % L): per head, pair
// (j, j + 64) -> (x1 c - x2 s, x2 c + x1 s), bf16.  One thread per (token, head, j).
__global__ __launch_bounds__(256) void rope_kernel(uint16_t* __restrict__ x, long long items, int nh, int L,
                                                   const float* __restrict__ cs, const float* __restrict__ sn) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= items) return;
  const int j = (int)(i & 63);
  const long long th = i >> 6;                 // token * nh + head
  const int t = (int)(th / nh);
  const int p = t % L;
  uint16_t* base = x + th * kHd;
  const float x1 = bf16_bits_to_f32(base[j]), x2 = bf16_bits_to_f32(base[j + 64]);
  const float c = cs[p * 64 + j], s = sn[p * 64 + j];
  float y1, y2;
  rope_rotate(x1, x2, c, s, y1, y2);
  base[j] = (uint16_t)f32_to_bf16_bits(y1);
  base[j + 64] = (uint16_t)f32_to_bf16_bits(y2);
}

// Causal grouped-query attention on the matrix cores.  Workgroup (block of 128
// queries, query head, sequence), 4 waves of 32 queries.  Per block of 32 keys a wave
// computes the transposed scores S^T = K Q^T (8 v_mfma_f32_32x32x16_bf16 over the 128
// dims: lane (query l % 32, half h) receives the scores of keys (r % 4) + 4 h + 8 (r / 4),
// r = 0..15), updates its query's running max and sum (the two halves of a query swap
// their partial max and sum), and accumulates O^T += V^T P^T (16 MFMAs: 4 blocks of 32
// dims x 2 steps of 16 keys x p as bf16 hi and lo).  The next key block's K and V
// are loaded into registers while the current one is computed.  The P operand of
// step s, element j is the lane's own
// score register 8 s + j, i.e. key j % 4 + 4 h + 16 s + 8 (j / 4); V^T is staged with its
// keys in that order (key bits 2 and 3 swapped), so no value crosses lanes.  K rows
// (272 B) and V^T rows (80 B) are padded so that 16 lanes' 16-byte reads hit distinct
// banks.  Softmax in fp32: p = exp(s / sqrt(128) - m), entering the products as bf16
// hi + lo (16 bits of p, so rounding p adds no error of its own beyond the output's
// bf16 rounding), the output divided by the sum.
constexpr int kFaQ = 128, kFaK = 32, kFaKRow = 136, kFaVRow = 40;   // rows in bf16 elements
__global__ __launch_bounds__(256) void attention_mfma_kernel(const uint16_t* __restrict__ Q,
                                                             const uint16_t* __restrict__ Kx,
                                                             const uint16_t* __restrict__ V, int L, int n_q,
                                                             int n_kv, uint16_t* __restrict__ O) {
  __shared__ __align__(16) uint16_t ks[kFaK * kFaKRow];
  __shared__ __align__(16) uint16_t vt[kHd * kFaVRow];
  // Workgroup -> (query block, head, sequence).  A query block's work grows with its
  // index (causal), and workgroups go to the 8 XCDs round-robin, so the blocks are
  // ordered by rank, every rank over all heads and sequences: the heavier half first
  // in decreasing order, then the lighter half in increasing order (4 blocks: 3, 2,
  // 0, 1), so that a CU's first and second workgroup tend to pair heavy with light.
  const int nqb = (int)gridDim.x, nhs = (int)(gridDim.y * gridDim.z);
  const int wg = (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
  const int rank = wg / nhs, hs = wg - rank * nhs;
  const int half = (nqb + 1) / 2;
  const int qb = rank < half ? nqb - 1 - rank : rank - half;
  const int hq = hs % n_q, b = hs / n_q;
  const int kvh = hq / (n_q / n_kv);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const size_t qstride = (size_t)n_q * kHd, kstride = (size_t)n_kv * kHd;
  const size_t tok0 = (size_t)b * L;
  const int q0 = qb * kFaQ + wave * 32;                 // this wave's first query
  const int qpos = q0 + l32;                            // this lane's query
  const int qmax = min(q0 + 31, L - 1);                 // the wave's last live query
  bf16x8 qf[8];
  {
    const uint16_t* qp = Q + (tok0 + min(qpos, L - 1)) * qstride + (size_t)hq * kHd + 8 * h;
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qp + 16 * st);
  }
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
  const float scale = 1.0f / sqrtf((float)kHd);
  float mx = -INFINITY, sum = 0.0f;
  const int kend = min(L, qb * kFaQ + kFaQ);            // keys the workgroup needs: 0 .. kend-1
  // staging: thread -> (key tid / 8, dims 16 (tid % 8) .. +15) of K and of V; the
  // next key block is loaded into registers while the current one is computed
  const int kj = tid >> 3, part = tid & 7;
  uint4 k0, k1, v0, v1;
  auto load_kv = [&](int kb) {
    const int key = kb + kj;
    k0 = make_uint4(0u, 0u, 0u, 0u), k1 = k0, v0 = k0, v1 = k0;
    if (key < kend) {
      const size_t src = (tok0 + key) * kstride + (size_t)kvh * kHd + 16 * part;
      k0 = *reinterpret_cast<const uint4*>(Kx + src);
      k1 = *reinterpret_cast<const uint4*>(Kx + src + 8);
      v0 = *reinterpret_cast<const uint4*>(V + src);
      v1 = *reinterpret_cast<const uint4*>(V + src + 8);
    }
  };
  load_kv(0);
  for (int kb = 0; kb < kend; kb += kFaK) {
    __syncthreads();
    {
      *reinterpret_cast<uint4*>(&ks[kj * kFaKRow + 16 * part]) = k0;
      *reinterpret_cast<uint4*>(&ks[kj * kFaKRow + 16 * part + 8]) = k1;
      const int slot = (kj & ~12) | ((kj & 4) << 1) | ((kj & 8) >> 1);    // key bits 2 and 3 swapped
      const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        vt[(16 * part + 2 * e) * kFaVRow + slot] = (uint16_t)(w[e] & 0xFFFFu);
        vt[(16 * part + 2 * e + 1) * kFaVRow + slot] = (uint16_t)(w[e] >> 16);
      }
    }
    __syncthreads();
    if (kb + kFaK < kend) load_kv(kb + kFaK);
    if (kb > qmax) continue;                            // every query of this wave precedes these keys
    f32x16 sc = f32x16{};
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&ks[l32 * kFaKRow + 16 * st + 8 * h]);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[st], sc, 0, 0, 0);
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kb + (r & 3) + 4 * h + 8 * (r >> 2);
      const float v = (key <= qpos && key < L) ? sc[r] * scale : -INFINITY;
      sc[r] = v;
      mloc = fmaxf(mloc, v);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
    const float mnew = fmaxf(mx, mloc);                 // finite: key 0 is in every query's first block
    const float corr = expf(mx - mnew);
    float lsum = 0.0f;
    uint32_t pb[8], pl[8];          // p as bf16 hi + lo (the pair carries 16 bits of p)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = expf(sc[r] - mnew), p1 = expf(sc[r + 1] - mnew);
      lsum = lsum + p0;
      lsum = lsum + p1;
      const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
      pb[r >> 1] = __builtin_bit_cast(uint32_t, pp);
      const bf16x2 pq = {(__bf16)(p0 - __uint_as_float(pb[r >> 1] << 16)),
                         (__bf16)(p1 - __uint_as_float(pb[r >> 1] & 0xFFFF0000u))};
      pl[r >> 1] = __builtin_bit_cast(uint32_t, pq);
    }
    lsum = lsum + __shfl_xor(lsum, 32, kWave);
    sum = sum * corr + lsum;
    mx = mnew;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = acc[db][r] * corr;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(pb[4 * s2], pb[4 * s2 + 1], pb[4 * s2 + 2], pb[4 * s2 + 3]));
      const bf16x8 pg = __builtin_bit_cast(bf16x8, make_uint4(pl[4 * s2], pl[4 * s2 + 1], pl[4 * s2 + 2], pl[4 * s2 + 3]));
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&vt[(32 * db + l32) * kFaVRow + 16 * s2 + 8 * h]);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc[db], 0, 0, 0);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pg, acc[db], 0, 0, 0);
      }
    }
  }
  if (qpos >= L) return;
  const float inv = 1.0f / sum;
  uint16_t* op = O + (tok0 + qpos) * qstride + (size_t)hq * kHd;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * db + 8 * i + 4 * h;          // registers 4 i .. 4 i + 3: dims d0 .. d0 + 3
      const uint32_t lo = f32_to_bf16_bits(acc[db][4 * i] * inv) | (f32_to_bf16_bits(acc[db][4 * i + 1] * inv) << 16);
      const uint32_t hi = f32_to_bf16_bits(acc[db][4 * i + 2] * inv) | (f32_to_bf16_bits(acc[db][4 * i + 3] * inv) << 16);
      *reinterpret_cast<uint2*>(op + d0) = make_uint2(lo, hi);
    }
}

// Elementwise over n bf16 values (n % 8 == 0), 8 per thread.
enum { EW_ADD = 0, EW_SILU_MUL = 1 };
template <int OP>
__global__ __launch_bounds__(256) void elementwise_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                          size_t n, uint16_t* __restrict__ Y) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= n) return;
  const uint4 av = *reinterpret_cast<const uint4*>(A + i);
  const uint4 bv = *reinterpret_cast<const uint4*>(B + i);
  const uint32_t a[4] = {av.x, av.y, av.z, av.w};
  const uint32_t b[4] = {bv.x, bv.y, bv.z, bv.w};
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float r[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float x = e ? __uint_as_float(a[q] & 0xFFFF0000u) : __uint_as_float(a[q] << 16);
      const float y = e ? __uint_as_float(b[q] & 0xFFFF0000u) : __uint_as_float(b[q] << 16);
      r[e] = OP == EW_ADD ? x + y : silu_mul_f32(x, y);
    }
    o[q] = f32_to_bf16_bits(r[0]) | (f32_to_bf16_bits(r[1]) << 16);
  }
  *reinterpret_cast<uint4*>(Y + i) = make_uint4(o[0], o[1], o[2], o[3]);
}

// Y[t][k] = bf16(X[t][k] / s[k]) (IEEE division), 8 per thread, K % 8 == 0.
__global__ __launch_bounds__(256) void divide_columns_kernel(const uint16_t* __restrict__ X, size_t n, int K,
                                                             const float* __restrict__ s, uint16_t* __restrict__ Y) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= n) return;
  const int k0 = (int)(i % (size_t)K);
  const uint4 v = *reinterpret_cast<const uint4*>(X + i);
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float lo = __uint_as_float(d[q] << 16) / s[k0 + 2 * q];
    const float hi = __uint_as_float(d[q] & 0xFFFF0000u) / s[k0 + 2 * q + 1];
    o[q] = f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
  }
  *reinterpret_cast<uint4*>(Y + i) = make_uint4(o[0], o[1], o[2], o[3]);
}

// part[blk] = sum over this block's elements of (a - b)^2 in fp64 (fixed order);
// 2048 elements per 256-thread block.
__global__ __launch_bounds__(256) void sqdiff_partial_kernel(const uint16_t* __restrict__ A,
                                                             const uint16_t* __restrict__ B, size_t n,
                                                             double* __restrict__ part) {
  __shared__ double red[256];
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
  double s = 0.0;
  if (i < n) {
    const uint4 av = *reinterpret_cast<const uint4*>(A + i);
    const uint4 bv = *reinterpret_cast<const uint4*>(B + i);
    const uint32_t a[4] = {av.x, av.y, av.z, av.w};
    const uint32_t b[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const double d0 = (double)__uint_as_float(a[q] << 16) - (double)__uint_as_float(b[q] << 16);
      const double d1 = (double)__uint_as_float(a[q] & 0xFFFF0000u) - (double)__uint_as_float(b[q] & 0xFFFF0000u);
      s += d0 * d0;
      s += d1 * d1;
    }
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

// out[0] = sum of part[0 .. nparts) (fp64, lane-strided then butterfly) / count.
__global__ __launch_bounds__(64) void mean_finish_kernel(const double* __restrict__ part, long long nparts,
                                                         double count, float* __restrict__ out) {
  // loads issued 16 at a time, added in the same ascending order (one memory
  // round trip per 16 terms instead of per term)
  double s = 0.0;
  long long i = threadIdx.x;
  for (; i + 64 * 15 < nparts; i += 64 * 16) {
    double v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = part[i + 64 * u];
#pragma unroll
    for (int u = 0; u < 16; ++u) s += v[u];
  }
  for (; i < nparts; i += 64) s += part[i];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (threadIdx.x == 0) out[0] = (float)(s / count);
}

// ---------------------------------------------------------------------------------------
// host side

struct Dims {
  int B, L, T, H, nq, nkv, I, QD, KD;      // T = B L, QD = 128 nq, KD = 128 nkv
};

// (K, N) of linear i: q k v o gate up down
inline void linear_shape(const Dims& d, int i, int& K, int& N) {
  static const int kin[7] = {0, 0, 0, 1, 0, 0, 2};  // 0: H, 1: QD, 2: I
  const int in = kin[i];
  K = in == 0 ? d.H : in == 1 ? d.QD : d.I;
  N = i == 0 ? d.QD : (i == 1 || i == 2) ? d.KD : (i == 3 || i == 6) ? d.H : d.I;
}

struct BlockLayout {
  size_t a, q, k, v, o, p, h, b2, gt, up, m, dn;      // per-op outputs
  size_t cs, sn;                                      // rope tables
  size_t total;
};

BlockLayout block_layout(const Dims& d, size_t& off) {
  BlockLayout l{};
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  const size_t T = (size_t)d.T;
  l.a = take(T * d.H * 2);
  l.q = take(T * d.QD * 2);
  l.k = take(T * d.KD * 2);
  l.v = take(T * d.KD * 2);
  l.o = take(T * d.QD * 2);
  l.p = take(T * d.H * 2);
  l.h = take(T * d.H * 2);
  l.b2 = take(T * d.H * 2);
  l.gt = take(T * d.I * 2);
  l.up = take(T * d.I * 2);
  l.m = take(T * d.I * 2);
  l.dn = take(T * d.H * 2);
  l.cs = take((size_t)d.L * 64 * 4);
  l.sn = take((size_t)d.L * 64 * 4);
  l.total = off;
  return l;
}

// The deployed int4 form of one linear: codes, scales, zeros and the scaled input.
struct Candidate {
  int linear;
  const float* s;               // [K]
  const uint32_t* qweight;
  const uint16_t* scales;
  const uint32_t* qzeros;       // NULL when symmetric
  int symmetric;
  uint16_t* xs;                 // [T][K] scratch for bf16(input / s)
  void* gemm_ws;                // launch_gemm workspace
};

int ew_launch(int op, const uint16_t* A, const uint16_t* B, size_t n, uint16_t* Y, hipStream_t st) {
  const size_t blocks = (n / 8 + 255) / 256;
  if (op == EW_ADD)
    hipLaunchKernelGGL(elementwise_kernel<EW_ADD>, dim3((unsigned)blocks), dim3(256), 0, st, A, B, n, Y);
  else
    hipLaunchKernelGGL(elementwise_kernel<EW_SILU_MUL>, dim3((unsigned)blocks), dim3(256), 0, st, A, B, n, Y);
  W4_CHECK_LAUNCH();
  return W4_OK;
}

// Y [T][N] = bf16(X W^T) for bf16 X [T][K] and W [N][K] (the unquantized projections).
int bf16_linear(const uint16_t* X, int T, int K, int N, const uint16_t* W, uint16_t* Y, hipStream_t st) {
  return launch_bf16_gemm(X, T, K, N, W, Y, st);
}

// One linear: Y [T][N] = bf16(X W^T), or the candidate's deployed int4 form.
int run_linear(const Dims& d, int i, const uint16_t* X, const uint16_t* W, const Candidate* cand, uint16_t* Y,
               hipStream_t st) {
  int K, N;
  linear_shape(d, i, K, N);
  if (cand && cand->linear == i) {
    const size_t n = (size_t)d.T * K;
    hipLaunchKernelGGL(divide_columns_kernel, dim3((unsigned)((n / 8 + 255) / 256)), dim3(256), 0, st, X, n, K,
                       cand->s, cand->xs);
    W4_CHECK_LAUNCH();
    return launch_gemm(cand->xs, d.T, K, N, cand->qweight, cand->scales, cand->qzeros, cand->symmetric, Y,
                       cand->gemm_ws, st);
  }
  return bf16_linear(X, d.T, K, N, W, Y, st);
}

// The block from a given stage: 0 = from its input X; 1 = from the attention output
// o_in (X still needed for the residual); 2 = from the post-attention residual h_in.
int run_block(const Dims& d, const w4_block& blk, const uint16_t* X, uint16_t* Y, const Candidate* cand,
              char* ws, const BlockLayout& l, hipStream_t st, int stage = 0, const uint16_t* o_in = nullptr,
              const uint16_t* h_in = nullptr) {
  auto buf = [&](size_t off) { return reinterpret_cast<uint16_t*>(ws + off); };
  const size_t T = (size_t)d.T;
  const unsigned nrow = (unsigned)((d.T + 3) / 4);
  int rc;
  const uint16_t* o = stage >= 1 ? o_in : buf(l.o);
  const uint16_t* h = stage >= 2 ? h_in : buf(l.h);
  if (stage == 0) {
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(nrow), dim3(256), 0, st, X, d.T, d.H, blk.norm1, buf(l.a));
    W4_CHECK_LAUNCH();
    const float* cs = reinterpret_cast<const float*>(ws + l.cs);
    const float* sn = reinterpret_cast<const float*>(ws + l.sn);
    if (cand && cand->linear <= 2) {
      if ((rc = run_linear(d, 0, buf(l.a), blk.wq, cand, buf(l.q), st))) return rc;
      if ((rc = run_linear(d, 1, buf(l.a), blk.wk, cand, buf(l.k), st))) return rc;
      if ((rc = run_linear(d, 2, buf(l.a), blk.wv, cand, buf(l.v), st))) return rc;
      const long long qi = (long long)T * d.nq * 64, ki = (long long)T * d.nkv * 64;
      hipLaunchKernelGGL(rope_kernel, dim3((unsigned)((qi + 255) / 256)), dim3(256), 0, st, buf(l.q), qi, d.nq, d.L,
                         cs, sn);
      W4_CHECK_LAUNCH();
      hipLaunchKernelGGL(rope_kernel, dim3((unsigned)((ki + 255) / 256)), dim3(256), 0, st, buf(l.k), ki, d.nkv,
                         d.L, cs, sn);
      W4_CHECK_LAUNCH();
    } else {      // q, k and v read the same normalized input: one launch, q and k rotated in its epilogue
      const uint16_t* Ws[3] = {blk.wq, blk.wk, blk.wv};
      const int Ns[3] = {d.QD, d.KD, d.KD};
      uint16_t* Ys[3] = {buf(l.q), buf(l.k), buf(l.v)};
      if ((rc = launch_bf16_gemm_rope(buf(l.a), d.T, d.H, 3, Ws, Ns, Ys, 0x3, cs, sn, d.L, st))) return rc;
    }
    hipLaunchKernelGGL(attention_mfma_kernel, dim3((unsigned)((d.L + kFaQ - 1) / kFaQ), (unsigned)d.nq, (unsigned)d.B),
                       dim3(256), 0, st, buf(l.q), buf(l.k), buf(l.v), d.L, d.nq, d.nkv, buf(l.o));
    W4_CHECK_LAUNCH();
  }
  if (stage <= 1) {
    if (cand && cand->linear == 3) {
      if ((rc = run_linear(d, 3, o, blk.wo, cand, buf(l.p), st))) return rc;
      if ((rc = ew_launch(EW_ADD, X, buf(l.p), T * d.H, buf(l.h), st))) return rc;
    } else {      // h = x + o Wo^T: the residual added in the GEMM's epilogue
      uint16_t* hy = buf(l.h);
      if ((rc = launch_bf16_gemm_multi(o, d.T, d.QD, 1, &blk.wo, &d.H, &hy, st, &X))) return rc;
    }
  }
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(nrow), dim3(256), 0, st, h, d.T, d.H, blk.norm2, buf(l.b2));
  W4_CHECK_LAUNCH();
  if (cand && (cand->linear == 4 || cand->linear == 5)) {
    if ((rc = run_linear(d, 4, buf(l.b2), blk.wgate, cand, buf(l.gt), st))) return rc;
    if ((rc = run_linear(d, 5, buf(l.b2), blk.wup, cand, buf(l.up), st))) return rc;
    if ((rc = ew_launch(EW_SILU_MUL, buf(l.gt), buf(l.up), T * d.I, buf(l.m), st))) return rc;
  } else {        // gate and up read the same normalized input: one launch, silu(gate) up in its epilogue
    if ((rc = launch_bf16_glu(buf(l.b2), d.T, d.H, d.I, blk.wgate, blk.wup, buf(l.m), st))) return rc;
  }
  if (cand && cand->linear == 6) {
    if ((rc = run_linear(d, 6, buf(l.m), blk.wdown, cand, buf(l.dn), st))) return rc;
    return ew_launch(EW_ADD, h, buf(l.dn), T * d.H, Y, st);
  }
  // y = h + m Wd^T: the residual added in the GEMM's epilogue
  return launch_bf16_gemm_multi(buf(l.m), d.T, d.I, 1, &blk.wdown, &d.H, &Y, st, &h);
}

int rope_tables(const Dims& d, char* ws, const BlockLayout& l, hipStream_t st) {
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((d.L * 64 + 255) / 256)), dim3(256), 0, st, d.L,
                     reinterpret_cast<float*>(ws + l.cs), reinterpret_cast<float*>(ws + l.sn));
  W4_CHECK_LAUNCH();
  return W4_OK;
}

Dims make_dims(int B, int L, int H, int nq, int nkv, int I) {
  Dims d{};
  d.B = B;
  d.L = L;
  d.T = B * L;
  d.H = H;
  d.nq = nq;
  d.nkv = nkv;
  d.I = I;
  d.QD = nq * kHd;
  d.KD = nkv * kHd;
  return d;
}

struct LookLayout {
  BlockLayout blk;
  size_t yref_i, yref_n, yc_i, yc_n, oref, href, xs, qw, sc, qz, gemm, part, total;
  size_t b2ref, ffix;   // feed-forward candidates: the normalized residual and the operand no candidate changes
  size_t nparts;
};

LookLayout look_layout(const Dims& d, int linear) {
  LookLayout l{};
  size_t off = 0;
  l.blk = block_layout(d, off);
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  int K, N;
  linear_shape(d, linear, K, N);
  const size_t T = (size_t)d.T;
  l.yref_i = take(T * d.H * 2);
  l.yref_n = take(T * d.H * 2);
  l.yc_i = take(T * d.H * 2);
  l.yc_n = take(T * d.H * 2);
  l.oref = take(T * d.QD * 2);      // the scored block's reference attention output and
  l.href = take(T * d.H * 2);       // post-attention residual: candidates start from them
  l.xs = take(T * K * 2);
  l.qw = take((size_t)N * (K / 8) * 4);
  l.sc = take((size_t)N * (K / kGroup) * 2);
  l.qz = take((size_t)N * ((K / kGroup + 7) / 8) * 4);
  l.gemm = take(gemm_workspace_bytes(d.T, K, N));
  l.nparts = (T * d.H + 2047) / 2048;
  l.part = take(l.nparts * 8);
  l.b2ref = take(linear >= 4 ? T * d.H * 2 : 0);
  l.ffix = take(linear >= 4 ? T * d.I * 2 : 0);
  l.total = off;
  return l;
}

}  // namespace

size_t block_forward_workspace_bytes(int B, int L, int H, int nq, int nkv, int I) {
  size_t off = 0;
  return block_layout(make_dims(B, L, H, nq, nkv, I), off).total;
}

int launch_block_forward(const uint16_t* X, int B, int L, int H, int nq, int nkv, int I, const w4_block& blk,
                         uint16_t* Y, void* workspace, hipStream_t stream) {
  const Dims d = make_dims(B, L, H, nq, nkv, I);
  size_t off = 0;
  const BlockLayout l = block_layout(d, off);
  char* ws = static_cast<char*>(workspace);
  int rc = rope_tables(d, ws, l, stream);
  if (rc) return rc;
  return run_block(d, blk, X, Y, nullptr, ws, l, stream);
}

// Block layout, then the candidate's scaled input bf16(a / s) and the int4 GEMM's workspace.
size_t block_quantized_layout(const Dims& d, int linear, size_t& xs, size_t& gemm) {
  size_t off = 0;
  block_layout(d, off);
  int K, N;
  linear_shape(d, linear, K, N);
  xs = off;
  off = align_up(off + (size_t)d.T * K * 2, 256);
  gemm = off;
  return align_up(off + gemm_workspace_bytes(d.T, K, N), 256);
}

size_t block_quantized_workspace_bytes(int B, int L, int H, int nq, int nkv, int I, int linear) {
  size_t xs, gemm;
  return block_quantized_layout(make_dims(B, L, H, nq, nkv, I), linear, xs, gemm);
}

int launch_block_forward_quantized(const uint16_t* X, int B, int L, int H, int nq, int nkv, int I,
                                   const w4_block& blk, int linear, const float* s, const uint32_t* qweight,
                                   const uint16_t* scales, const uint32_t* qzeros, int symmetric, uint16_t* Y,
                                   void* workspace, hipStream_t stream) {
  const Dims d = make_dims(B, L, H, nq, nkv, I);
  size_t off = 0;
  const BlockLayout l = block_layout(d, off);
  size_t xs, gemm;
  block_quantized_layout(d, linear, xs, gemm);
  char* ws = static_cast<char*>(workspace);
  int rc = rope_tables(d, ws, l, stream);
  if (rc) return rc;
  Candidate cand{linear, s, qweight, scales, qzeros, symmetric, reinterpret_cast<uint16_t*>(ws + xs), ws + gemm};
  return run_block(d, blk, X, Y, &cand, ws, l, stream);
}

size_t lookahead_workspace_bytes(int B, int L, int H, int nq, int nkv, int I, int linear) {
  return look_layout(make_dims(B, L, H, nq, nkv, I), linear).total;
}

int lookahead_input_size(int H, int nq, int I, int linear) {
  Dims d = make_dims(1, 1, H, nq, 1, I);
  int K, N;
  linear_shape(d, linear, K, N);
  return K;
}

// Reference path: block `blk` (its output kept), then `next` when given.  With m not
// NULL, mean |input| of linear `linear` over the tokens is written to m[0 .. K) (m
// holds (1 + ceil(T / 64)) K doubles, the rest per-chunk partial sums).
int launch_lookahead_reference(const uint16_t* X, int B, int L, int H, int nq, int nkv, int I, const w4_block& blk,
                               const w4_block* next, int linear, double* m, void* workspace, hipStream_t stream,
                               double* m_host, hipEvent_t m_ready) {
  const Dims d = make_dims(B, L, H, nq, nkv, I);
  const LookLayout l = look_layout(d, linear);
  char* ws = static_cast<char*>(workspace);
  auto buf = [&](size_t off) { return reinterpret_cast<uint16_t*>(ws + off); };
  int rc = rope_tables(d, ws, l.blk, stream);
  if (rc) return rc;
  if ((rc = run_block(d, blk, X, buf(l.yref_i), nullptr, ws, l.blk, stream))) return rc;
  if (hipMemcpyAsync(buf(l.oref), buf(l.blk.o), (size_t)d.T * d.QD * 2, hipMemcpyDeviceToDevice, stream) !=
          hipSuccess ||
      hipMemcpyAsync(buf(l.href), buf(l.blk.h), (size_t)d.T * d.H * 2, hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return W4_ERR_HIP;
  if (m) {
    // the block buffers still hold this block's activations: the linear's input
    const size_t in[7] = {l.blk.a, l.blk.a, l.blk.a, l.blk.o, l.blk.b2, l.blk.b2, l.blk.m};
    int K, N;
    linear_shape(d, linear, K, N);
    if ((rc = launch_act_mean_abs(buf(in[linear]), d.T, K, m, stream))) return rc;
    if (m_host && m_ready &&
        (hipMemcpyAsync(m_host, m, (size_t)K * 8, hipMemcpyDeviceToHost, stream) != hipSuccess ||
         hipEventRecord(m_ready, stream) != hipSuccess))
      return W4_ERR_HIP;
  }
  if (next && (rc = run_block(d, *next, buf(l.yref_i), buf(l.yref_n), nullptr, ws, l.blk, stream))) return rc;
  return W4_OK;
}

// The feed-forward half of the block for a candidate of gate, up or down, from the
// reference post-attention residual h: what run_block does from its third stage,
// with the normalized residual b2 = rmsnorm(h) and the operand the candidate does not
// change (up for a gate candidate, gate for an up candidate, silu(gate) up for a
// down candidate) taken as computed once for all candidates.
int run_ffn_candidate(const Dims& d, const w4_block& blk, const uint16_t* h, const uint16_t* b2,
                      const uint16_t* fixed, const Candidate& cand, uint16_t* Y, char* ws, const BlockLayout& l,
                      hipStream_t st) {
  auto buf = [&](size_t off) { return reinterpret_cast<uint16_t*>(ws + off); };
  const size_t T = (size_t)d.T;
  int rc;
  if (cand.linear == 6) {
    if ((rc = run_linear(d, 6, fixed, blk.wdown, &cand, buf(l.dn), st))) return rc;
    return ew_launch(EW_ADD, h, buf(l.dn), T * d.H, Y, st);
  }
  if (cand.linear == 4) {
    if ((rc = run_linear(d, 4, b2, blk.wgate, &cand, buf(l.gt), st))) return rc;
    if ((rc = ew_launch(EW_SILU_MUL, buf(l.gt), fixed, T * d.I, buf(l.m), st))) return rc;
  } else {
    if ((rc = run_linear(d, 5, b2, blk.wup, &cand, buf(l.up), st))) return rc;
    if ((rc = ew_launch(EW_SILU_MUL, fixed, buf(l.up), T * d.I, buf(l.m), st))) return rc;
  }
  return launch_bf16_gemm_multi(buf(l.m), d.T, d.I, 1, &blk.wdown, &d.H, &Y, st, &h);
}

// Candidates against the reference outputs left in the workspace by
// launch_lookahead_reference (same shape, blocks and linear).
int launch_lookahead_candidates(const uint16_t* X, int B, int L, int H, int nq, int nkv, int I, const w4_block& blk,
                                const w4_block* next, int linear, const float* S, const float* ratios, int C,
                                int symmetric, float* losses, float* losses_d0, void* workspace,
                                hipStream_t stream) {
  const Dims d = make_dims(B, L, H, nq, nkv, I);
  const LookLayout l = look_layout(d, linear);
  char* ws = static_cast<char*>(workspace);
  auto buf = [&](size_t off) { return reinterpret_cast<uint16_t*>(ws + off); };
  const uint16_t* ref_n = next ? buf(l.yref_n) : buf(l.yref_i);
  int K, N;
  linear_shape(d, linear, K, N);
  const uint16_t* Wl[7] = {blk.wq, blk.wk, blk.wv, blk.wo, blk.wgate, blk.wup, blk.wdown};
  double* part = reinterpret_cast<double*>(ws + l.part);
  const size_t n = (size_t)d.T * d.H;
  const unsigned pblocks = (unsigned)l.nparts;
  int rc;
  // the block runs from the first op the candidate changes: o from the reference
  // attention output, gate / up / down from the reference post-attention residual
  const int stage = linear <= 2 ? 0 : linear == 3 ? 1 : 2;
  if (stage == 2) {
    // what no feed-forward candidate changes, once: rmsnorm of the residual, then up
    // (gate candidates), gate (up candidates) or silu(gate) up (down candidates)
    hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)((d.T + 3) / 4)), dim3(256), 0, stream, buf(l.href), d.T, d.H,
                       blk.norm2, buf(l.b2ref));
    W4_CHECK_LAUNCH();
    if (linear == 4 && (rc = bf16_linear(buf(l.b2ref), d.T, d.H, d.I, blk.wup, buf(l.ffix), stream))) return rc;
    if (linear == 5 && (rc = bf16_linear(buf(l.b2ref), d.T, d.H, d.I, blk.wgate, buf(l.ffix), stream))) return rc;
    if (linear == 6 &&
        (rc = launch_bf16_glu(buf(l.b2ref), d.T, d.H, d.I, blk.wgate, blk.wup, buf(l.ffix), stream)))
      return rc;
  }
  for (int c = 0; c < C; ++c) {
    QuantArgs q{};
    q.W = Wl[linear];
    q.N = N;
    q.K = K;
    q.s = S + (size_t)c * K;
    q.ratios = ratios + c;
    q.symmetric = symmetric;
    q.qweight = reinterpret_cast<uint32_t*>(ws + l.qw);
    q.scales = buf(l.sc);
    q.qzeros = symmetric ? nullptr : reinterpret_cast<uint32_t*>(ws + l.qz);
    if ((rc = launch_quantize_pack(q, 1, stream))) return rc;
    Candidate cand{linear, S + (size_t)c * K, q.qweight, q.scales, q.qzeros, symmetric, buf(l.xs), ws + l.gemm};
    if (stage == 2)
      rc = run_ffn_candidate(d, blk, buf(l.href), buf(l.b2ref), buf(l.ffix), cand, buf(l.yc_i), ws, l.blk, stream);
    else
      rc = run_block(d, blk, X, buf(l.yc_i), &cand, ws, l.blk, stream, stage, buf(l.oref), buf(l.href));
    if (rc) return rc;
    if (next && (rc = run_block(d, *next, buf(l.yc_i), buf(l.yc_n), nullptr, ws, l.blk, stream))) return rc;
    const uint16_t* yc_n = next ? buf(l.yc_n) : buf(l.yc_i);
    hipLaunchKernelGGL(sqdiff_partial_kernel, dim3(pblocks), dim3(256), 0, stream, yc_n, ref_n, n, part);
    W4_CHECK_LAUNCH();
    hipLaunchKernelGGL(mean_finish_kernel, dim3(1), dim3(64), 0, stream, part, (long long)l.nparts, (double)n,
                       losses + c);
    W4_CHECK_LAUNCH();
    if (losses_d0) {
      hipLaunchKernelGGL(sqdiff_partial_kernel, dim3(pblocks), dim3(256), 0, stream, buf(l.yc_i), buf(l.yref_i), n,
                         part);
      W4_CHECK_LAUNCH();
      hipLaunchKernelGGL(mean_finish_kernel, dim3(1), dim3(64), 0, stream, part, (long long)l.nparts, (double)n,
                         losses_d0 + c);
      W4_CHECK_LAUNCH();
    }
  }
  return W4_OK;
}

int launch_lookahead_loss(const uint16_t* X, int B, int L, int H, int nq, int nkv, int I, const w4_block& blk,
                          const w4_block* next, int linear, const float* S, const float* ratios, int C,
                          int symmetric, float* losses, float* losses_d0, void* workspace, hipStream_t stream) {
  int rc = launch_lookahead_reference(X, B, L, H, nq, nkv, I, blk, next, linear, nullptr, workspace, stream);
  if (rc) return rc;
  return launch_lookahead_candidates(X, B, L, H, nq, nkv, I, blk, next, linear, S, ratios, C, symmetric, losses,
                                     losses_d0, workspace, stream);
}

}  // namespace w4
