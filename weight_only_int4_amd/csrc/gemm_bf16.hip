// Plain bf16 contraction Y = bf16(X W^T) on the matrix cores, for the linears
// that run unquantized: the reference output bf16(X W^T) of the AWQ candidate
// loss (model card "rebuttal_w4g128_awq_w2", scale-rewrite paragraph: the loss
// compares against the unquantized linear) and the decoder block's projections
// in the look-ahead scoring (same card, the paragraph under the details table:
// the reference path and block i + 1 run in original precision).
//
// X [M][K] and W [N][K] are both K-contiguous, so every MFMA operand fragment is
// a 16-byte run of one row.  One launch may cover several weights that read the
// same X (the q, k, v projections; gate and up): their output tiles are laid
// side by side along N, each tile belonging to one weight.  A segment may add a
// residual R [M][N] in its epilogue: Y = bf16(R + bf16(X W^T)), the same roundings
// as a separate add of the rounded product.  Two more epilogues fuse the decoder
// block's elementwise steps (model card "qwen3-1.7b_q326_channel", "Model
// Architecture"), with the arithmetic of the standalone kernels (block_ops.hpp):
//  * GLU: a tile covers 64 columns of the gate weight and the same 64 columns of
//    the up weight (W rows 0-63 and 64-127 of the stage) and stores
//    bf16(silu(gate) up);
//  * RoPE: on the segments it is asked for (q, k: 128-column tiles are heads), the
//    tile stores the rotated pairs of dims (j, j + 64) at position row % L.
// In both, the two waves of a row half hold partner values at the same lane and
// register; they trade their bf16 values through LDS and each finishes one 32-row
// block for both partners.
// Workgroup tile 128 x 128, four waves of 64 x 64
// (2 x 2 blocks of v_mfma_f32_32x32x16_bf16, fp32 accumulation), K in stages of
// 64 channels: per stage and workgroup 16 KB of X and 16 KB of W travel from
// global memory straight into LDS (global_load_lds_dwordx4, no registers), S
// stages deep.  Inside a 128-byte LDS row the 16-byte chunk c is stored at
// position c ^ ((row >> 1) & 7): a 16-lane pass of fragment reads (16 rows, one
// chunk each) then covers all 64 banks once.
#include "block_ops.hpp"
#include "gemm_core.hpp"

namespace w4 {
namespace {

#ifndef W4_BF16_GEMM_STAGES
#define W4_BF16_GEMM_STAGES 2
#endif
#ifndef W4_BF16_GEMM_BK
#define W4_BF16_GEMM_BK 64
#endif

#ifndef W4_BF16_GEMM_BM
#define W4_BF16_GEMM_BM 128
#endif

constexpr int kB16M = W4_BF16_GEMM_BM, kB16N = 128, kB16K = W4_BF16_GEMM_BK;
constexpr int kB16Waves = kB16M / 64 * 2;            // waves of 64 x 64: kB16M / 64 down, 2 across
constexpr int kB16Row = kB16K * 2;                   // bytes of one LDS row (one tile row's stage)
constexpr int kB16Chunks = kB16Row / 16;             // 16-byte chunks per LDS row
constexpr int kB16XPart = kB16M * kB16Row;           // X part of a stage
constexpr int kB16Stage = kB16XPart + kB16N * kB16Row;
constexpr int kB16RowsPerCopy = 1024 / kB16Row;      // LDS rows one 1 KB copy fills
constexpr int kB16CX = kB16M / kB16RowsPerCopy / kB16Waves;   // X copies per wave and stage
constexpr int kB16CW = kB16N / kB16RowsPerCopy / kB16Waves;   // W copies per wave and stage
constexpr int kB16Copies = kB16CX + kB16CW;
constexpr int kB16Blocks = 160 * 1024 / (W4_BF16_GEMM_STAGES * kB16Stage) * kB16Waves / 4;   // waves per SIMD
static_assert(kB16CW >= 1 && kB16CX * kB16Waves * kB16RowsPerCopy == kB16M, "copy split");
static_assert(kB16K == 32 || kB16K == 64, "stage depth");

// Chunk swizzle of an LDS row: a 16-lane pass of fragment reads (16 consecutive
// rows, one logical chunk each) must hit 16 distinct 16-byte bank groups of the
// 64 banks.  64-channel rows (128 bytes, 8 chunks): even and odd rows start on
// opposite halves of the banks, so rows 2 i, 2 i + 1 share the XOR i & 7;
// 32-channel rows (64 bytes, 4 chunks): four rows share a 256-byte bank line, so
// rows 4 i .. 4 i + 3 share the XOR i & 3.
__device__ __forceinline__ int swz(int r) { return kB16K == 64 ? (r >> 1) & 7 : (r >> 2) & 3; }

// Up to three weights reading the same X: segment s has W[s] [N[s]][K] and writes
// Y[s] [M][N[s]] (plus R[s] [M][N[s]] when not NULL); its 128-column tiles are
// tiles t0[s] .. t0[s + 1] - 1 along N.  GLU: one segment, W[0] the gate and W[1]
// the up weight, 64-column tiles.  RoPE: segments whose bit is set in rope_mask
// are rotated with the tables cs, sn [L][64].
enum { B16_PLAIN = 0, B16_GLU = 1, B16_ROPE = 2 };

struct B16Args {
  const uint16_t* X;
  int M, K;
  int nseg;
  const uint16_t* W[3];
  uint16_t* Y[3];
  const uint16_t* R[3];
  int N[3];
  int t0[4];
  const float* cs;
  const float* sn;
  int L;
  int rope_mask;
};

template <int S, int MODE>
__global__ __launch_bounds__(kB16Waves * 64, kB16Blocks) void bf16_gemm_kernel(B16Args g) {
  constexpr int kTN = MODE == B16_GLU ? kB16N / 2 : kB16N;   // output columns per tile
  static_assert(MODE != B16_GLU || kB16CW % 2 == 0, "gate and up copies split evenly");
  constexpr int D = S - 1;                 // stages in flight ahead of the one computed
  __shared__ __attribute__((aligned(1024))) unsigned char smem[S * kB16Stage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % (kB16M / 64), wn = wave / (kB16M / 64);   // this wave's 64 x 64 part of the tile
  const int h = lane >> 5, l32 = lane & 31;
  const int M = g.M, K = g.K;
  int tm, tn;
  tile_coords(blockIdx.x, (M + kB16M - 1) / kB16M, g.t0[g.nseg], tm, tn);
  const int seg = tn >= g.t0[1] ? (tn >= g.t0[2] ? 2 : 1) : 0;     // wave-uniform
  const uint16_t* __restrict__ X = g.X;
  const uint16_t* __restrict__ W = g.W[seg];
  uint16_t* __restrict__ Y = g.Y[seg];
  const uint16_t* __restrict__ R = g.R[seg];
  const int N = g.N[seg];
  const int m0 = tm * kB16M, n0 = (tn - g.t0[seg]) * kTN;
  const int KT = K / kB16K;
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;

  // Copy u of this wave fills LDS rows R (wave + 4 u) .. +R-1 (R = rows per 1 KB)
  // of the X part and the same rows of the W part: lane -> row R (wave + 4 u) +
  // lane / C, position lane % C (C chunks per row), holding logical chunk
  // position ^ swz(row).  Rows past M (columns past N) read the last valid one:
  // finite, never stored.
  uint32_t xoff[kB16CX], woff[kB16CW];
#pragma unroll
  for (int u = 0; u < kB16CX; ++u) {
    const int r = kB16RowsPerCopy * (wave + kB16Waves * u) + lane / kB16Chunks;
    const int c = (lane % kB16Chunks) ^ swz(r);
    xoff[u] = ((uint32_t)min(m0 + r, M - 1) * (uint32_t)K + (uint32_t)(8 * c)) * 2u;
  }
#pragma unroll
  for (int u = 0; u < kB16CW; ++u) {
    const int r = kB16RowsPerCopy * (wave + kB16Waves * u) + lane / kB16Chunks;
    const int c = (lane % kB16Chunks) ^ swz(r);
    // GLU: stage rows 0-63 (copies u < kB16CW / 2) are gate rows n0 .., 64-127 up rows n0 ..
    const int wr = MODE == B16_GLU ? (r & (kTN - 1)) : r;
    woff[u] = ((uint32_t)min(n0 + wr, N - 1) * (uint32_t)K + (uint32_t)(8 * c)) * 2u;
  }
  const unsigned char* xb = reinterpret_cast<const unsigned char*>(X);
  const unsigned char* wb = reinterpret_cast<const unsigned char*>(W);
  const unsigned char* wb2 = reinterpret_cast<const unsigned char*>(g.W[1]);
  auto issue = [&](int kt, int stage) {
    const unsigned char* xs = xb + (size_t)kt * (kB16K * 2);
    const unsigned char* ws = wb + (size_t)kt * (kB16K * 2);
    const uint32_t st = smem_base + stage * kB16Stage;
#pragma unroll
    for (int u = 0; u < kB16CX; ++u) lds_copy16(xoff[u], xs, st + (wave + kB16Waves * u) * 1024);
#pragma unroll
    for (int u = 0; u < kB16CW; ++u) {
      const unsigned char* wsrc =
          MODE == B16_GLU && u >= kB16CW / 2 ? wb2 + (size_t)kt * (kB16K * 2) : ws;
      lds_copy16(woff[u], wsrc, st + kB16XPart + (wave + kB16Waves * u) * 1024);
    }
  };

  // fragment reads: row (or column) 32 b + l32 of this wave's quarter, logical chunk
  // 2 j + h at position (2 j + h) ^ swz(l32) (swz depends only on the row's low bits):
  // byte fbase ^ (32 j)
  const uint32_t fbase = (uint32_t)(l32 * kB16Row + ((h ^ swz(l32)) * 16));
  const uint32_t xq = (uint32_t)(wm * 64 * kB16Row), wq = (uint32_t)(kB16XPart + wn * 64 * kB16Row);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto compute = [&](int stage) {
    const unsigned char* st = smem + stage * kB16Stage;
    const uint32_t fb = opaque_vgpr(fbase);
    bf16x8 a[2][2], b[2][2];
    auto rd = [&](int j, int buf) {
      const uint32_t o = fb ^ (uint32_t)(32 * j);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[buf][i] = *reinterpret_cast<const bf16x8*>(st + xq + i * 32 * kB16Row + o);
        b[buf][i] = *reinterpret_cast<const bf16x8*>(st + wq + i * 32 * kB16Row + o);
      }
    };
    rd(0, 0);
#pragma unroll
    for (int j = 0; j < kB16K / 16; ++j) {
      if (j + 1 < kB16K / 16) rd(j + 1, (j + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
          acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 1][i], b[j & 1][jn], acc[i][jn], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Stage s holds k-tile kt with kt % S == s.  Iteration kt waits for this wave's
  // copies of kt (those of the D - 1 later k-tiles may stay in flight), barriers --
  // after which every wave's copies of kt have landed and every wave is done with
  // kt - 1 -- then refills the stage kt - 1 used with k-tile kt + D (past the last
  // k-tile: the last one again, into a stage nothing reads any more) and computes kt.
#pragma unroll
  for (int p = 0; p < D; ++p) issue(min(p, KT - 1), p);
  for (int kt = 0; kt < KT; ++kt) {
    wait_vmcnt<(D - 1) * kB16Copies>();
    lds_barrier();
    issue(min(kt + D, KT - 1), (kt + D) % S);
    compute(kt % S);
  }
  wait_vmcnt<0>();

  // Fused elementwise step.  The two waves of a row half (wn = 0, 1) hold partner
  // values at the same lane and register: columns c and 64 + c of the tile (RoPE:
  // dims j and j + 64 of a head) or gate and up of column c (GLU).  Each hands all
  // its bf16-rounded values over through LDS (the stage buffers, free after the
  // barrier; pairs of registers per 4-byte word), then wave wn finishes the 32-row
  // block i = wn for both partners: RoPE rotates the pair and stores both dims, GLU
  // stores silu(gate) up.  Afterwards register block acc[s] holds the values for
  // row block rb(s) and column half ch(s) below.
  bool fused = false;
  if constexpr (MODE != B16_PLAIN) {
    if (MODE == B16_GLU || ((g.rope_mask >> seg) & 1)) {      // uniform per workgroup
      fused = true;
      uint32_t* xw = reinterpret_cast<uint32_t*>(smem);
      auto slot = [&](int w_n, int i, int jn, int rp) {
        return ((((wm * 2 + w_n) * 2 + i) * 2 + jn) * 8 + rp) * 64 + lane;
      };
      static_assert(kB16M / 64 * 2 * 2 * 2 * 8 * 64 * 4 <= S * kB16Stage, "exchange fits the stages");
      lds_barrier();                          // every wave is past its last fragment read
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
#pragma unroll
          for (int rp = 0; rp < 8; ++rp)
            xw[slot(wn, i, jn, rp)] =
                f32_to_bf16_bits(acc[i][jn][2 * rp]) | (f32_to_bf16_bits(acc[i][jn][2 * rp + 1]) << 16);
      lds_barrier();
#pragma unroll
      for (int jn = 0; jn < 2; ++jn)
#pragma unroll
        for (int rp = 0; rp < 8; ++rp) {
          const uint32_t pw = xw[slot(1 - wn, wn, jn, rp)];    // the partner's row block i = wn
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int r = 2 * rp + e;
            const float own = bf16_bits_to_f32(f32_to_bf16_bits(wn ? acc[1][jn][r] : acc[0][jn][r]));
            const float other = bf16_bits_to_f32(e ? pw >> 16 : pw & 0xFFFFu);
            const float lo = wn ? other : own;      // column c (dim j) or gate
            const float hi = wn ? own : other;      // column 64 + c (dim j + 64) or up
            if constexpr (MODE == B16_GLU) {
              acc[0][jn][r] = silu_mul_f32(lo, hi);
            } else {
              const int row = m0 + 64 * wm + 32 * wn + 8 * (r >> 2) + 4 * h + (r & 3);
              const int j = 32 * jn + l32;
              const int p = row % g.L;
              float y1, y2;
              rope_rotate(lo, hi, g.cs[p * 64 + j], g.sn[p * 64 + j], y1, y2);
              acc[0][jn][r] = y1;
              acc[1][jn][r] = y2;
            }
          }
        }
    }
  }

  // Epilogue.  A lane holds column l32 and rows 8 i + 4 h + jj (register 4 i + jj)
  // of a block.  Neighbouring lanes (columns c, c + 1) trade values so that the
  // even lane holds both columns of the even registers' rows and the odd lane of
  // the odd registers' rows: one 4-byte store of a bf16 pair per two values.
  const bool odd = l32 & 1;
  const bool pair_ok = (N & 1) == 0;       // 4-byte aligned pairs; otherwise one bf16 per store
  // register block s: row block rb and column half ch (GLU tiles have no column half)
#pragma unroll
  for (int jn = 0; jn < 2; ++jn) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      if (MODE == B16_GLU && sb == 1) continue;
      const int rblk = fused ? wn : sb;
      const int ch = MODE == B16_GLU ? 0 : (fused ? sb : wn);
      const int col = n0 + 64 * ch + 32 * jn + l32;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float v0 = acc[sb][jn][r], v1 = acc[sb][jn][r + 1];
        const float send = odd ? v0 : v1;
        const float recv = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), 0xB1, 0xF, 0xF, true));
        const int row0 = m0 + 64 * wm + 32 * rblk + 8 * (r >> 2) + 4 * h + (r & 3);   // register r + 1: row0 + 1
        if (pair_ok) {
          const int row = odd ? row0 + 1 : row0;
          const int c0 = col & ~1;
          if (row < M && c0 < N) {      // N even: c0 < N implies c0 + 1 < N
            bf16x2 pr = {(__bf16)(odd ? recv : v0), (__bf16)(odd ? v1 : recv)};
            const size_t o = (size_t)row * N + c0;
            if (R) {
              const uint32_t rb = *reinterpret_cast<const uint32_t*>(R + o);
              const uint32_t pb = __builtin_bit_cast(uint32_t, pr);
              pr = bf16x2{(__bf16)(__uint_as_float(rb << 16) + __uint_as_float(pb << 16)),
                          (__bf16)(__uint_as_float(rb & 0xFFFF0000u) + __uint_as_float(pb & 0xFFFF0000u))};
            }
            *reinterpret_cast<bf16x2*>(Y + o) = pr;
          }
        } else if (col < N) {
          auto put = [&](int row, float v) {
            const size_t o = (size_t)row * N + col;
            uint32_t b = f32_to_bf16_bits(v);
            if (R) b = f32_to_bf16_bits(bf16_bits_to_f32(R[o]) + bf16_bits_to_f32(b));
            Y[o] = (uint16_t)b;
          };
          if (row0 < M) put(row0, v0);
          if (row0 + 1 < M) put(row0 + 1, v1);
        }
      }
    }
  }
}

}  // namespace

namespace {

template <int MODE>
int launch_b16(const B16Args& g, long long tiles, hipStream_t stream) {
  if (tiles == 0) return W4_OK;
  if (tiles > 0x7FFFFFFFLL) return W4_ERR_SHAPE;
  hipLaunchKernelGGL((bf16_gemm_kernel<W4_BF16_GEMM_STAGES, MODE>), dim3((unsigned)tiles), dim3(kB16Waves * 64), 0,
                     stream, g);
  W4_CHECK_LAUNCH();
  return W4_OK;
}

// Arguments of a launch over nseg weights reading X; the tile count through `tiles`.
int b16_args(const uint16_t* X, int M, int K, int nseg, const uint16_t* const* W, const int* N, uint16_t* const* Y,
             const uint16_t* const* R, B16Args& g, long long& tiles) {
  if (nseg < 1 || nseg > 3 || K <= 0 || K % kB16K) return W4_ERR_SHAPE;
  g = B16Args{};
  g.X = X;
  g.M = M;
  g.K = K;
  g.nseg = nseg;
  long long t = 0;
  for (int s = 0; s < nseg; ++s) {
    // 32-bit per-lane byte offsets: 2 M K and 2 N K below 2^32
    if (N[s] < 0 || (long long)M * K >= (1LL << 31) || (long long)N[s] * K >= (1LL << 31)) return W4_ERR_SHAPE;
    g.W[s] = W[s];
    g.Y[s] = Y[s];
    g.R[s] = R ? R[s] : nullptr;
    g.N[s] = N[s];
    g.t0[s] = (int)t;
    t += (N[s] + kB16N - 1) / kB16N;
  }
  for (int s = nseg; s < 4; ++s) g.t0[s] = (int)t;
  for (int s = nseg; s < 3; ++s) {
    g.W[s] = W[0];
    g.Y[s] = Y[0];
    g.R[s] = nullptr;
    g.N[s] = 0;
  }
  tiles = (long long)((M + kB16M - 1) / kB16M) * t;
  return W4_OK;
}

}  // namespace

int launch_bf16_gemm_multi(const uint16_t* X, int M, int K, int nseg, const uint16_t* const* W, const int* N,
                           uint16_t* const* Y, hipStream_t stream, const uint16_t* const* R) {
  B16Args g;
  long long tiles = 0;
  if (int st = b16_args(X, M, K, nseg, W, N, Y, R, g, tiles)) return st;
  return launch_b16<B16_PLAIN>(g, tiles, stream);
}

int launch_bf16_gemm_rope(const uint16_t* X, int M, int K, int nseg, const uint16_t* const* W, const int* N,
                          uint16_t* const* Y, int rope_mask, const float* cs, const float* sn, int L,
                          hipStream_t stream) {
  B16Args g;
  long long tiles = 0;
  if (int st = b16_args(X, M, K, nseg, W, N, Y, nullptr, g, tiles)) return st;
  if (L < 1) return W4_ERR_SHAPE;
  for (int s = 0; s < nseg; ++s)
    if (((rope_mask >> s) & 1) && N[s] % 128) return W4_ERR_SHAPE;     // whole heads per tile
  g.cs = cs;
  g.sn = sn;
  g.L = L;
  g.rope_mask = rope_mask;
  return launch_b16<B16_ROPE>(g, tiles, stream);
}

int launch_bf16_glu(const uint16_t* X, int M, int K, int N, const uint16_t* Wg, const uint16_t* Wu, uint16_t* Y,
                    hipStream_t stream) {
  B16Args g;
  long long tiles = 0;
  if (int st = b16_args(X, M, K, 1, &Wg, &N, &Y, nullptr, g, tiles)) return st;
  g.W[1] = Wu;
  const long long t = (N + kB16N / 2 - 1) / (kB16N / 2);
  for (int s = 1; s < 4; ++s) g.t0[s] = (int)t;
  tiles = (long long)((M + kB16M - 1) / kB16M) * t;
  return launch_b16<B16_GLU>(g, tiles, stream);
}

int launch_bf16_gemm(const uint16_t* X, int M, int K, int N, const uint16_t* W, uint16_t* Y, hipStream_t stream) {
  return launch_bf16_gemm_multi(X, M, K, 1, &W, &N, &Y, stream);
}

}  // namespace w4
