"""CPU oracle for weight-only int4, group-128 linears (W4A16) and the AWQ grid loss.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously-correct
statement of what the GPU path computes.  Only the tests, the smoke check and
the benchmark's CPU-baseline leg may import it; the product path never does.
It shares no code with the HIP kernels or their host library.

Sources (web pages, cited by title and section):

* [AWQ-W4 card]  model card "rebuttal_w4g128_awq_w2" (ghostchoir) -- details
  table rows "Scheme" (weight-only, 4-bit, group 128, asymmetric zero point)
  and "Search" (20-point scale-exponent grid + 10-point global shrink grid);
  the scale-rewrite paragraph (prev_op /= s, W *= s  ==  Q(W diag(s)) diag(1/s));
  the "Clipping granularity" paragraph (one shrink ratio per linear);
  the note under the perplexity table (RTN = round-to-nearest group quantization).
* [27B card]  model card "Qwen3.6-27B-W4A16" (GotoAI-Inc) -- opening
  paragraph: int4, group 128, symmetric, weight-only, activations 16-bit,
  data-free round-to-nearest.
* [AWQ ppl record] benchmark record "AWQ INT4-g128 WikiText-2 perplexity delta
  vs fp16, Llama-2 7B" -- "Methodology" field: group 128, grid size 20 for the
  alpha search.

Where the pages leave a step open, the reading taken is stated at the function
(bf16 scale; codes against the stored bf16 scale; round half to even; IEEE fp32
division; symmetric codes in [-8, 7] stored with offset 8; sequential nibble
packing along K; the alpha grid i/20 and shrink grid 1 - j/20; clipping as a
clamp at r * group absmax; s normalised by sqrt(max * min)).

Arithmetic conventions: bf16 values travel as uint16 bit patterns; elementwise
steps are NumPy fp32 (IEEE, round-to-nearest-even, no fused multiply-add);
sums and contractions are fp64.
"""
from __future__ import annotations

import numpy as np

GROUP = 128          # [AWQ-W4 card] "Scheme": group size 128; [27B card] opening paragraph
ASYM_LEVELS = 15     # 4-bit codes 0..15 -> 15 steps between min and max
SYM_MAX = 7          # symmetric codes -8..7 with the scale set by absmax / 7
SYM_OFFSET = 8       # stored nibble = code + 8 (offset binary)
RANGE_FLOOR = np.float32(1e-5)   # guard for constant groups (reading: the pages are silent)
S_FLOOR = 1e-4                   # floor on mean|X|^alpha before normalising (reading)


# --------------------------------------------------------------------------- bf16

def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> fp32 value (exact: bf16 is the top half of fp32)."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


# --------------------------------------------------------------------------- quantize

def quantize_rtn(W_bf16: np.ndarray, s: np.ndarray | None = None, clip_ratio: float = 1.0,
                 symmetric: bool = False):
    """Round-to-nearest group-128 quantization of v = W * diag(s).

    [AWQ-W4 card] "Scheme" row: weight-only, 4-bit, group 128, asymmetric with a
    zero point; the note under its perplexity table: RTN is round-to-nearest group
    quantization.  [27B card] opening paragraph: the symmetric, data-free form.
    [AWQ-W4 card] scale-rewrite paragraph: the candidate weight is Q(W diag(s)),
    so s multiplies input channel k of every row.  [AWQ-W4 card] "Clipping
    granularity": one shrink ratio r per linear, applied here as a clamp of each
    group of W diag(s) to +-r * (group absmax) before the scale is chosen.

    Per row n and group g (128 consecutive k), with v fp32:
      asymmetric: sc = bf16(max(hi - lo, 1e-5) / 15),  z = clamp(rint(-lo / sc), 0, 15),
                  q  = clamp(rint(v / sc) + z, 0, 15)
      symmetric : sc = bf16(max(absmax, 1e-5) / 7),    q = clamp(rint(v / sc), -8, 7) + 8
    rint is round-half-to-even; "/" is IEEE fp32 division by the stored bf16 scale.

    W_bf16: uint16 [N][K] (output channels x input channels, K contiguous), K % 128 == 0.
    Returns (codes uint8 [N][K] in 0..15, scales bf16 bits uint16 [N][K/128],
             zeros uint8 [N][K/128] or None when symmetric).
    """
    W_bf16 = np.asarray(W_bf16, dtype=np.uint16)
    N, K = W_bf16.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    G = K // GROUP
    v = bf16_to_f32(W_bf16)
    if s is not None:
        v = v * np.asarray(s, dtype=np.float32)[None, :]          # fp32 multiply, RNE
    v = v.reshape(N, G, GROUP)
    absmax = np.abs(v).max(axis=2, keepdims=True)
    r = np.float32(clip_ratio)
    if r < np.float32(1.0):
        t = r * absmax                                             # fp32
        v = np.minimum(np.maximum(v, -t), t)
        absmax = np.abs(v).max(axis=2, keepdims=True)
    if symmetric:
        sc_bits = f32_to_bf16(np.maximum(absmax, RANGE_FLOOR) / np.float32(SYM_MAX))
        sc = bf16_to_f32(sc_bits)
        q = np.clip(np.rint(v / sc), -SYM_OFFSET, SYM_MAX) + SYM_OFFSET
        zeros = None
    else:
        lo = v.min(axis=2, keepdims=True)
        hi = v.max(axis=2, keepdims=True)
        sc_bits = f32_to_bf16(np.maximum(hi - lo, RANGE_FLOOR) / np.float32(ASYM_LEVELS))
        sc = bf16_to_f32(sc_bits)
        z = np.clip(np.rint(-lo / sc), 0, ASYM_LEVELS)
        q = np.clip(np.rint(v / sc) + z, 0, ASYM_LEVELS)
        zeros = z.reshape(N, G).astype(np.uint8)
    codes = q.reshape(N, K).astype(np.uint8)
    return codes, sc_bits.reshape(N, G), zeros


# --------------------------------------------------------------------------- packing

def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """8 consecutive 4-bit values along the last axis -> one uint32.

    Layout (reading; the pages only say int4): nibble j (bits 4j..4j+3) of word i
    holds element 8i + j.  A last axis that is not a multiple of 8 is padded with 0.
    """
    codes = np.asarray(codes, dtype=np.uint32)
    n = codes.shape[-1]
    words = -(-n // 8)
    padded = np.zeros(codes.shape[:-1] + (words * 8,), dtype=np.uint32)
    padded[..., :n] = codes & np.uint32(0xF)
    padded = padded.reshape(codes.shape[:-1] + (words, 8))
    out = np.zeros(codes.shape[:-1] + (words,), dtype=np.uint32)
    for j in range(8):
        out |= padded[..., j] << np.uint32(4 * j)
    return out


def unpack_nibbles(words: np.ndarray, n: int) -> np.ndarray:
    """Inverse of pack_nibbles: uint32 [..., W] -> uint8 [..., n]."""
    words = np.asarray(words, dtype=np.uint32)
    out = np.empty(words.shape + (8,), dtype=np.uint8)
    for j in range(8):
        out[..., j] = (words >> np.uint32(4 * j)) & np.uint32(0xF)
    return out.reshape(words.shape[:-1] + (words.shape[-1] * 8,))[..., :n]


def quantize_pack(W_bf16, s=None, clip_ratio=1.0, symmetric=False):
    """Quantize and pack: returns (qweight uint32 [N][K/8], scales uint16 [N][K/128],
    qzeros uint32 [N][ceil(K/1024)] or None when symmetric)."""
    codes, scales, zeros = quantize_rtn(W_bf16, s, clip_ratio, symmetric)
    qzeros = None if zeros is None else pack_nibbles(zeros)
    return pack_nibbles(codes), scales, qzeros


def dequantize(qweight, scales, qzeros, K: int, symmetric: bool) -> np.ndarray:
    """W_hat[n][k] = (q - z) * sc as fp32 ([AWQ-W4 card] the Q(.) of the rewrite).

    The product of a 4-bit integer difference and a bf16 scale has at most 12
    significant bits, so it is exact in fp32.
    """
    codes = unpack_nibbles(qweight, K).astype(np.float32)
    N = codes.shape[0]
    G = K // GROUP
    sc = bf16_to_f32(scales).reshape(N, G, 1)
    if symmetric:
        z = np.float32(SYM_OFFSET)
    else:
        z = unpack_nibbles(qzeros, G).astype(np.float32).reshape(N, G, 1)
    return ((codes.reshape(N, G, GROUP) - z) * sc).reshape(N, K)


# --------------------------------------------------------------------------- contraction

def linear(X_bf16: np.ndarray, W_hat: np.ndarray) -> np.ndarray:
    """Y[m][n] = sum_k X[m][k] * W_hat[n][k] in fp64 (the W4A16 linear, bf16 activations).

    [27B card] opening paragraph: weights int4, activations stay 16-bit.
    """
    return bf16_to_f32(X_bf16).astype(np.float64) @ np.asarray(W_hat, dtype=np.float64).T


# --------------------------------------------------------------------------- per-channel clipping

def clip_search_per_channel(X_bf16, W_bf16, s, ratios, symmetric=False, rows=None):
    """Stock per-output-channel clipping: a shrink ratio per (output channel, group).

    [AWQ-W4 card] "Clipping granularity" and the comparability caveat: the d = 0
    arm searches a clipping threshold per output channel, where each channel's
    loss is its own; the look-ahead arm replaces it with one global ratio.
    Reading: for row n, group g and every ratio r of the grid,
      w_hat = dequantize(Q(clip_r(v))) of that group alone (quantize_rtn with clip r),
      e = v - w_hat with v = W diag(s) (fp32 values, difference in fp64),
      L[g][n][r] = sum_t (sum_{k in g} x'_tk e_k)^2 with x' = bf16(X / s), the
      deployed activations (IEEE fp32 division, then RNE to bf16);
    best[n][g] = the first ratio index with the least loss.
    rows: optional subset of output channels (the result covers only those).
    Returns (L float64 [G][len(rows)][R], best int64 [len(rows)][G]).
    """
    W_bf16 = np.asarray(W_bf16, dtype=np.uint16)
    if rows is not None:
        W_bf16 = W_bf16[np.asarray(rows)]
    N, K = W_bf16.shape
    G = K // GROUP
    s32 = np.asarray(s, dtype=np.float32)
    xs = bf16_to_f32(f32_to_bf16(bf16_to_f32(X_bf16) / s32[None, :])).astype(np.float64)   # [T][K]
    v = (bf16_to_f32(W_bf16) * s32[None, :]).astype(np.float64)                               # [N][K]
    R = len(ratios)
    L = np.zeros((G, N, R))
    for ir, r in enumerate(ratios):
        qw, sc, qz = quantize_pack(W_bf16, s32, float(np.float32(r)), symmetric)
        e = v - dequantize(qw, sc, qz, K, symmetric).astype(np.float64)
        for g in range(G):
            sl = slice(GROUP * g, GROUP * (g + 1))
            P = xs[:, sl] @ e[:, sl].T                        # [T][N] partial outputs of group g
            L[g, :, ir] = (P * P).sum(axis=0)
    best = np.argmin(L, axis=2).T                               # first minimum
    return L, best


# --------------------------------------------------------------------------- W4A8 decode

INT8_MAX = 127       # symmetric int8 activation codes in [-127, 127] (reading)


def quantize_activations_int8(X_bf16: np.ndarray):
    """Per-row symmetric int8 activations for the W4A8 decode path.

    [QSRT card] "What is included" / "Size and memory": W4A8 decode runs on the
    same stored int4 weights; the pages do not define the 8-bit activation format.
    Reading: per row m, sx = max_k |x| / 127 in fp32 (IEEE division; 1 for an
    all-zero row), xq = clamp(rint(x / sx), -127, 127) with the IEEE fp32 quotient,
    ties to even.  Returns (Xq int8 [M][K], sx fp32 [M], xsum int64 [M][K/128]:
    the code sum of every group).
    """
    x = bf16_to_f32(X_bf16)
    M, K = x.shape
    amax = np.abs(x).max(axis=1)
    sx = np.where(amax > 0, amax / np.float32(INT8_MAX), np.float32(1.0)).astype(np.float32)
    q = np.rint(x / sx[:, None])
    xq = np.clip(q, -INT8_MAX, INT8_MAX).astype(np.int8)
    xsum = xq.astype(np.int64).reshape(M, K // GROUP, GROUP).sum(axis=2)
    return xq, sx, xsum


def w4a8_linear(Xq, sx, qweight, scales, qzeros, K: int, symmetric: bool) -> np.ndarray:
    """Y[m][n] = sx[m] * sum_g sc[n][g] * sum_{k in g} xq[m][k] (q[n][k] - z[n][g]).

    [QSRT card] "Reproducible runtime": the W4A8 decode contraction.  The group
    sums are exact integers; the scaling and the sum over groups are fp64.
    """
    codes = unpack_nibbles(qweight, K).astype(np.int64)
    N = codes.shape[0]
    G = K // GROUP
    z = (np.full((N, G), SYM_OFFSET, dtype=np.int64) if symmetric
         else unpack_nibbles(qzeros, G).astype(np.int64))
    d = codes.reshape(N, G, GROUP) - z[:, :, None]                                # q - z
    xq = np.asarray(Xq, dtype=np.int64).reshape(-1, G, GROUP)
    isum = np.einsum("mgk,ngk->mng", xq, d)                                       # exact int64
    sc = bf16_to_f32(scales).astype(np.float64)                                   # [N][G]
    y = (isum.astype(np.float64) * sc[None, :, :]).sum(axis=2)
    return y * np.asarray(sx, dtype=np.float64)[:, None]


# --------------------------------------------------------------------------- AWQ search

def act_mean_abs(X_bf16: np.ndarray) -> np.ndarray:
    """m_k = (1/T) sum_t |X[t][k]| in fp64: the per-input-channel activation statistic."""
    return np.abs(bf16_to_f32(X_bf16).astype(np.float64)).mean(axis=0)


def awq_scales(m: np.ndarray, alpha: float) -> np.ndarray:
    """s = max(m^alpha, 1e-4) / sqrt(max * min), computed in fp64 and stored fp32.

    [AWQ-W4 card] "Search": the AWQ scale exponent; [AWQ ppl record]
    "Methodology": a 20-point grid over alpha.  The normalisation keeps s
    centred on 1 (reading: the pages do not fix it).  0^0 = 1, so alpha = 0
    gives s = 1 exactly.
    """
    p = np.maximum(np.power(np.asarray(m, dtype=np.float64), float(alpha)), S_FLOOR)
    return (p / np.sqrt(p.max() * p.min())).astype(np.float32)


def alpha_grid(n: int = 20) -> np.ndarray:
    """alpha_i = i / n, i = 0..n-1 (reading of the 20-point grid; includes alpha = 0)."""
    return np.arange(n, dtype=np.float64) / n


def shrink_grid(n: int = 10) -> np.ndarray:
    """r_j = 1 - j / 20, j = 0..n-1: 1.0 down to 0.55 (reading of the 10-point grid in [0.5, 1])."""
    return 1.0 - np.arange(n, dtype=np.float64) / 20.0


def reference_output(X_bf16, W_bf16) -> np.ndarray:
    """Y_ref = bf16(fp32(X W^T)) as fp64: the unquantized bf16 linear's output."""
    y = linear(X_bf16, bf16_to_f32(W_bf16))
    return bf16_to_f32(f32_to_bf16(y.astype(np.float32))).astype(np.float64)


def candidate_loss(X_bf16, W_bf16, s, clip_ratio, symmetric=False, Y_ref=None) -> float:
    """Loss of one (s, r) candidate: mean over T x N of (Y_hat - Y_ref)^2 in fp64.

    [AWQ-W4 card] scale-rewrite paragraph: the candidate is simulated by using the
    weight Q(W diag(s)) diag(1/s) with the activations left alone, so
    Y_hat = X (W_hat diag(1/s))^T, with W_hat = dequantize(Q(W diag(s), r)).
    The loss scope is the linear's own output (reading; the card's look-ahead
    scope, which also runs the next block, is a different loss).
    """
    if Y_ref is None:
        Y_ref = reference_output(X_bf16, W_bf16)
    N, K = np.asarray(W_bf16).shape
    qw, sc, qz = quantize_pack(W_bf16, s, clip_ratio, symmetric)
    W_hat = dequantize(qw, sc, qz, K, symmetric).astype(np.float64)
    W_eff = W_hat / np.asarray(s, dtype=np.float32).astype(np.float64)[None, :]
    Y_hat = linear(X_bf16, W_eff)
    d = Y_hat - Y_ref
    return float(np.mean(d * d))


def grid_loss(X_bf16, W_bf16, S: np.ndarray, ratios, symmetric=False, Y_ref=None) -> np.ndarray:
    """Losses of C candidates: row c of S is s_c [K], ratios[c] its clip ratio."""
    if Y_ref is None:
        Y_ref = reference_output(X_bf16, W_bf16)
    S = np.asarray(S, dtype=np.float32)
    return np.array([candidate_loss(X_bf16, W_bf16, S[c], float(np.float32(ratios[c])),
                                    symmetric, Y_ref) for c in range(S.shape[0])])


def search(X_bf16, W_bf16, alphas=None, ratios=None, symmetric=False):
    """Two-phase AWQ search ([AWQ-W4 card] "Search": scale-exponent grid, then
    the global shrink grid).  Phase 1 scores every alpha at r = 1 and keeps the
    first minimum; phase 2 scores every r at s(alpha*) and keeps the first minimum.

    Returns dict(alpha_losses, ratio_losses, alpha_index, ratio_index, s).
    """
    alphas = alpha_grid() if alphas is None else np.asarray(alphas, dtype=np.float64)
    ratios = shrink_grid() if ratios is None else np.asarray(ratios, dtype=np.float64)
    m = act_mean_abs(X_bf16)
    Y_ref = reference_output(X_bf16, W_bf16)
    S = np.stack([awq_scales(m, a) for a in alphas])
    la = grid_loss(X_bf16, W_bf16, S, np.ones(len(alphas)), symmetric, Y_ref)
    ia = int(np.argmin(la))
    s_star = S[ia]
    lr = grid_loss(X_bf16, W_bf16, np.broadcast_to(s_star, (len(ratios), s_star.size)),
                   ratios, symmetric, Y_ref)
    ir = int(np.argmin(lr))
    return dict(alpha_losses=la, ratio_losses=lr, alpha_index=ia, ratio_index=ir, s=s_star)


# --------------------------------------------------------------------------- look-ahead block scoring
#
# [AWQ-W4 card] details table "Search" and the paragraph under it: the candidate
# for block i is scored at the output of block i + 1, which runs unquantized; the
# reference is the same path with block i unquantized too; the last block falls
# back to its own output.  The block is the base model's decoder block ([AWQ-W4
# card] "Base model": Qwen3-1.7B, hidden 2048; [q326 page] architecture notes:
# grouped-query attention with 16 query heads over 8 key/value heads, head size
# 128, rotary positions with base 10^6, SiLU-gated feed-forward of width 6144).
# Readings: pre-norm RMSNorm (eps 1e-6) before attention and before the
# feed-forward, residual adds after each; no biases and no per-head q/k norms
# (the pages name neither); rotary embedding on the pairs (j, j + 64) of each
# head at the token's position within its sequence; causal attention within each
# sequence with scale 1/sqrt(128), query head h reading key/value head
# h // (n_q / n_kv); every op output is rounded to bf16 ("in bf16"), the
# arithmetic inside an op is fp64.  The loss is the mean over tokens and hidden
# units of the squared difference of the two bf16 outputs.

HEAD_DIM = 128
LINEARS = ("q", "k", "v", "o", "gate", "up", "down")
RMS_EPS = 1e-6
ROPE_BASE = 1e6


def _bf16_round(x) -> np.ndarray:
    """fp64 values -> nearest bf16 value (via fp32, as the kernels store), as fp64."""
    return bf16_to_f32(f32_to_bf16(np.asarray(x, dtype=np.float64).astype(np.float32))).astype(np.float64)


def rmsnorm(x, g, eps=RMS_EPS) -> np.ndarray:
    """x [T][H] and g [H] bf16 values (fp64): bf16(x / sqrt(mean_k x^2 + eps) * g)."""
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps)
    return _bf16_round(x * r[:, None] * g[None, :])


def rope_tables(L: int, base: float = ROPE_BASE):
    """cos and sin [L][64] of position p times base^(-2j/128), fp64."""
    inv = base ** (-(2.0 * np.arange(HEAD_DIM // 2)) / HEAD_DIM)
    ang = np.arange(L, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def rope_raw(x, B: int, L: int, n_heads: int, base: float = ROPE_BASE) -> np.ndarray:
    """Rotary embedding of x [B*L][n_heads*128] in fp64: per head, the pair (j, j + 64)
    at position p (within its sequence) rotates by the angle p * base^(-2j/128)."""
    c, s = rope_tables(L, base)
    xr = x.reshape(B, L, n_heads, HEAD_DIM)
    x1, x2 = xr[..., :64], xr[..., 64:]
    c, s = c[None, :, None, :], s[None, :, None, :]
    out = np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
    return out.reshape(B * L, n_heads * HEAD_DIM)


def rope(x, B: int, L: int, n_heads: int, base: float = ROPE_BASE) -> np.ndarray:
    """rope_raw rounded to bf16."""
    return _bf16_round(rope_raw(x, B, L, n_heads, base))


def attention(q, k, v, B: int, L: int, n_q: int, n_kv: int) -> np.ndarray:
    """attention_raw rounded to bf16."""
    return _bf16_round(attention_raw(q, k, v, B, L, n_q, n_kv))


def attention_raw(q, k, v, B: int, L: int, n_q: int, n_kv: int) -> np.ndarray:
    """Causal grouped-query attention per sequence in fp64: softmax(q k^T / sqrt(128)) v
    with query head h reading key/value head h // (n_q / n_kv)."""
    rep = n_q // n_kv
    qh = q.reshape(B, L, n_q, HEAD_DIM)
    kh = k.reshape(B, L, n_kv, HEAD_DIM)
    vh = v.reshape(B, L, n_kv, HEAD_DIM)
    out = np.zeros_like(qh)
    mask = np.triu(np.ones((L, L), dtype=bool), 1)            # key after query
    for b in range(B):
        for h in range(n_q):
            kv = h // rep
            sc = qh[b, :, h, :] @ kh[b, :, kv, :].T / np.sqrt(HEAD_DIM)
            sc[mask] = -np.inf
            sc = sc - sc.max(axis=1, keepdims=True)
            p = np.exp(sc)
            p = p / p.sum(axis=1, keepdims=True)
            out[b, :, h, :] = p @ vh[b, :, kv, :]
    return out.reshape(B * L, n_q * HEAD_DIM)


def silu_mul(g, u) -> np.ndarray:
    """bf16(silu(g) * u), silu(g) = g / (1 + exp(-g))."""
    return _bf16_round(g / (1.0 + np.exp(-g)) * u)


def block_forward(x_bf16, B: int, L: int, blk: dict, n_q: int, n_kv: int, candidate=None, inputs=None):
    """One decoder block on x [B*L][H] (uint16 bf16).  blk maps "norm1", "norm2" to
    bf16 [H] and each name of LINEARS to its bf16 weight [out][in].  candidate =
    (name, s fp32 [in], packed (qweight, scales, qzeros), symmetric) replaces that
    linear by its deployed int4 form: input bf16(in / s) against the dequantized
    codes.  Returns the block output as bf16 bits [B*L][H]; a dict passed as
    `inputs` receives each linear's input (bf16 values, fp64)."""
    val = lambda bits: bf16_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)

    def lin(name, a):
        if inputs is not None:
            inputs[name] = a
        if candidate is not None and candidate[0] == name:
            _, s, (qw, sc, qz), sym = candidate
            K = a.shape[1]
            s32 = np.asarray(s, dtype=np.float32)
            xs = bf16_to_f32(f32_to_bf16(a.astype(np.float32) / s32[None, :])).astype(np.float64)
            w = dequantize(qw, sc, qz, K, sym).astype(np.float64)
        else:
            xs, w = a, val(blk[name])
        return _bf16_round(xs @ w.T)

    x = val(x_bf16)
    a = rmsnorm(x, val(blk["norm1"]))
    q = rope(lin("q", a), B, L, n_q)
    k = rope(lin("k", a), B, L, n_kv)
    v = lin("v", a)
    o = attention(q, k, v, B, L, n_q, n_kv)
    h = _bf16_round(x + lin("o", o))
    b2 = rmsnorm(h, val(blk["norm2"]))
    m = silu_mul(lin("gate", b2), lin("up", b2))
    y = _bf16_round(h + lin("down", m))
    return f32_to_bf16(y.astype(np.float32))


def lookahead_losses(x_bf16, B, L, blk, nxt, n_q, n_kv, name, S, ratios, symmetric=False):
    """Look-ahead (d = 1) and block-output (d = 0) losses of C candidates (S[c], ratios[c])
    for linear `name` of block blk, nxt the next block or None (last block: the d = 1
    loss falls back to the block's own output).  Returns (d1 [C], d0 [C]) fp64."""
    val = lambda bits: bf16_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)
    ref_i = block_forward(x_bf16, B, L, blk, n_q, n_kv)
    ref_n = block_forward(ref_i, B, L, nxt, n_q, n_kv) if nxt is not None else ref_i
    d1, d0 = [], []
    for c in range(len(ratios)):
        packed = quantize_pack(blk[name], S[c], float(np.float32(ratios[c])), symmetric)
        yi = block_forward(x_bf16, B, L, blk, n_q, n_kv, candidate=(name, S[c], packed, symmetric))
        yn = block_forward(yi, B, L, nxt, n_q, n_kv) if nxt is not None else yi
        d0.append(float(np.mean((val(yi) - val(ref_i)) ** 2)))
        d1.append(float(np.mean((val(yn) - val(ref_n)) ** 2)))
    return np.array(d1), np.array(d0)


def search_lookahead(x_bf16, B, L, blk, nxt, n_q, n_kv, name, alphas=None, ratios=None, symmetric=False):
    """Two-phase search of [AWQ-W4 card] "Search" with the look-ahead loss: the
    statistic m = mean |input of the linear| over the tokens of the reference pass,
    every alpha at r = 1 (first minimum alpha*), then every ratio at s(alpha*).
    Returns dict(alpha_losses, ratio_losses, alpha_index, ratio_index, s)."""
    alphas = alpha_grid() if alphas is None else np.asarray(alphas, dtype=np.float64)
    ratios = shrink_grid() if ratios is None else np.asarray(ratios, dtype=np.float64)
    ins = {}
    block_forward(x_bf16, B, L, blk, n_q, n_kv, inputs=ins)
    m = np.abs(ins[name]).mean(axis=0)
    S = np.stack([awq_scales(m, a) for a in alphas])
    la, _ = lookahead_losses(x_bf16, B, L, blk, nxt, n_q, n_kv, name, S, np.ones(len(alphas)), symmetric)
    ia = int(np.argmin(la))
    s_star = S[ia]
    lr, _ = lookahead_losses(x_bf16, B, L, blk, nxt, n_q, n_kv, name,
                             np.broadcast_to(s_star, (len(ratios), s_star.size)), ratios, symmetric)
    ir = int(np.argmin(lr))
    return dict(alpha_losses=la, ratio_losses=lr, alpha_index=ia, ratio_index=ir, s=s_star)
