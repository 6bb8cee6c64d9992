"""Pure-Python scalar restatement of the group-128 RTN quantizer and the AWQ
candidate loss, for brute-force checks of the vectorised oracle on tiny inputs.

It is written independently of ``oracle/``: one element at a time, Python
floats (fp64) with every fp32 step rounded back to fp32 through ``struct``
(rounding a correctly rounded fp64 sum, product or quotient of two fp32 values to
fp32 gives the correctly rounded fp32 result, because 53 >= 2*24 + 2), bf16
rounding by exponent/mantissa arithmetic (not bit tricks), and Python's
``round`` (ties to even) as rint.  Definitions: model card
"rebuttal_w4g128_awq_w2", details table rows "Scheme" and "Search", the
scale-rewrite paragraph and "Clipping granularity"; model card
"Qwen3.6-27B-W4A16", opening paragraph (symmetric form).
"""
from __future__ import annotations

import math
import struct


def f32(x: float) -> float:
    return struct.unpack("f", struct.pack("f", x))[0]


def bf16_value(bits: int) -> float:
    return struct.unpack(">f", struct.pack(">I", (bits & 0xFFFF) << 16))[0]


def round_bf16(x: float) -> float:
    """Nearest value with 8 significant bits, ties to even (finite, normal inputs)."""
    if x == 0.0:
        return 0.0
    m, e = math.frexp(x)            # x = m * 2**e, 0.5 <= |m| < 1
    scaled = m * 256.0              # 8 significant bits before the point
    return math.ldexp(float(round(scaled)), e - 8)


def quantize_group(v: list[float], symmetric: bool):
    """One group of 128 fp32 values -> (codes 0..15, scale value, zero)."""
    floor = f32(1e-5)
    if symmetric:
        amax = max(abs(x) for x in v)
        sc = round_bf16(f32(max(amax, floor) / 7.0))
        codes = [min(max(round(f32(x / sc)), -8), 7) + 8 for x in v]
        return codes, sc, 8
    lo, hi = min(v), max(v)
    sc = round_bf16(f32(max(f32(hi - lo), floor) / 15.0))
    z = min(max(round(f32(-lo / sc)), 0), 15)
    codes = [min(max(round(f32(x / sc)) + z, 0), 15) for x in v]
    return codes, sc, z


def quantize_dequant(W_rows: list[list[float]], s: list[float] | None, r: float, symmetric: bool):
    """Fake-quantized weights W_hat (list of rows) of Q(W diag(s)) with clip ratio r."""
    out = []
    r = f32(r)
    for row in W_rows:
        K = len(row)
        v = [f32(row[k] * s[k]) if s is not None else row[k] for k in range(K)]
        what = []
        for g0 in range(0, K, 128):
            grp = v[g0:g0 + 128]
            if r < 1.0:
                t = f32(r * max(abs(x) for x in grp))
                grp = [min(max(x, -t), t) for x in grp]
            codes, sc, z = quantize_group(grp, symmetric)
            what.extend((c - z) * sc for c in codes)
        out.append(what)
    return out


def mean_abs(X_rows):
    T = len(X_rows)
    K = len(X_rows[0])
    return [sum(abs(X_rows[t][k]) for t in range(T)) / T for k in range(K)]


def scales_for(m: list[float], alpha: float) -> list[float]:
    p = [max(math.pow(x, alpha), 1e-4) for x in m]
    d = math.sqrt(max(p) * min(p))
    return [f32(x / d) for x in p]


def loss(X_rows, W_rows, s, r, symmetric, Y_ref):
    what = quantize_dequant(W_rows, s, r, symmetric)
    T, N, K = len(X_rows), len(W_rows), len(W_rows[0])
    acc = 0.0
    for t in range(T):
        for n in range(N):
            y = 0.0
            for k in range(K):
                y += X_rows[t][k] * (what[n][k] / s[k])
            d = y - Y_ref[t][n]
            acc += d * d
    return acc / (T * N)


def reference(X_rows, W_rows):
    """bf16(fp32(sum_k x w)) for every (t, n)."""
    return [[round_bf16(f32(sum(x * w for x, w in zip(xr, wr)))) for wr in W_rows] for xr in X_rows]


def search(X_rows, W_rows, alphas, ratios, symmetric=False):
    m = mean_abs(X_rows)
    Y_ref = reference(X_rows, W_rows)
    la = [loss(X_rows, W_rows, scales_for(m, a), 1.0, symmetric, Y_ref) for a in alphas]
    ia = min(range(len(la)), key=lambda i: (la[i], i))
    s_star = scales_for(m, alphas[ia])
    lr = [loss(X_rows, W_rows, s_star, r, symmetric, Y_ref) for r in ratios]
    ir = min(range(len(lr)), key=lambda i: (lr[i], i))
    return la, lr, ia, ir


def per_channel_clip_losses(X_rows, W_rows, s, ratios, symmetric=False):
    """Per (group g, output channel n, ratio index j): the squared partial output
    error of group g over the tokens, sum_t (sum_{k in g} x'[t][k] e[n][k])^2 with
    x' = bf16(fp32(x / s)) and e = fp32(w s) - w_hat(ratio j); and per (n, g) the
    first ratio index of least loss.  Returns (L[g][n][j], best[n][g])."""
    T, N, K = len(X_rows), len(W_rows), len(W_rows[0])
    xs = [[round_bf16(f32(X_rows[t][k] / s[k])) for k in range(K)] for t in range(T)]
    v = [[f32(W_rows[n][k] * s[k]) for k in range(K)] for n in range(N)]
    G = K // 128
    L = [[[0.0] * len(ratios) for _ in range(N)] for _ in range(G)]
    for j, r in enumerate(ratios):
        what = quantize_dequant(W_rows, s, r, symmetric)
        for n in range(N):
            for g in range(G):
                tot = 0.0
                for t in range(T):
                    p = 0.0
                    for k in range(128 * g, 128 * g + 128):
                        p += xs[t][k] * (v[n][k] - what[n][k])
                    tot += p * p
                L[g][n][j] = tot
    best = [[min(range(len(ratios)), key=lambda j: (L[g][n][j], j)) for g in range(G)] for n in range(N)]
    return L, best


def causal_attention(q, k, v, L, n_q, n_kv, hd=128):
    """One sequence, pure Python: q [L][n_q*hd], k, v [L][n_kv*hd] (lists of floats).
    Query head h reads key/value head h // (n_q // n_kv); token t attends to 0..t."""
    rep = n_q // n_kv
    out = [[0.0] * (n_q * hd) for _ in range(L)]
    for t in range(L):
        for h in range(n_q):
            kv = h // rep
            sc = []
            for j in range(t + 1):
                d = 0.0
                for e in range(hd):
                    d += q[t][h * hd + e] * k[j][kv * hd + e]
                sc.append(d / math.sqrt(hd))
            mx = max(sc)
            ex = [math.exp(x - mx) for x in sc]
            z = sum(ex)
            for e in range(hd):
                acc = 0.0
                for j in range(t + 1):
                    acc += ex[j] / z * v[j][kv * hd + e]
                out[t][h * hd + e] = acc
    return out


def rotate_pairs(x, p, base=1e6, hd=128):
    """Rotary embedding of one head vector x (list of hd floats) at position p."""
    half = hd // 2
    out = [0.0] * hd
    for j in range(half):
        a = p * base ** (-(2.0 * j) / hd)
        c, s = math.cos(a), math.sin(a)
        out[j] = x[j] * c - x[j + half] * s
        out[j + half] = x[j + half] * c + x[j] * s
    return out


# ----------------------------------------------------------------------------- one decoder block
#
# The block of the look-ahead scoring (model card "rebuttal_w4g128_awq_w2",
# "Search" row and the paragraph under the details table; model page
# "qwen3-1.7b_q326_channel", "Model Architecture": grouped-query attention,
# rotary positions with base 10^6, SiLU-gated feed-forward), restated token by
# token with the readings the oracle takes where the pages are silent:
# pre-norm RMSNorm with eps 1e-6 and a per-channel weight before attention and
# before the feed-forward, the second norm reading the post-attention residual;
# SiLU on the gate projection, multiplied by the up projection; residual adds
# after attention and after the feed-forward; every op output rounded to bf16
# (through fp32, as the GPU stores it).

RMS_EPS_READING = 1e-6


def rb(x: float) -> float:
    """An op output as stored: fp64 value -> fp32 -> bf16 (nearest even both times)."""
    return round_bf16(f32(x))


def rms_row(x: list[float], g: list[float]) -> list[float]:
    ms = sum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + RMS_EPS_READING)
    return [rb(x[c] * r * g[c]) for c in range(len(x))]


def matvec(W: list[list[float]], a: list[float]) -> list[float]:
    """One token through a linear with weight W [out][in]: rounded outputs."""
    return [rb(sum(W[o][c] * a[c] for c in range(len(a)))) for o in range(len(W))]


def block_tokens(x_rows, blk, n_q, n_kv, candidate=None):
    """One sequence x [L][H] (bf16 values) through the block.  blk holds "norm1",
    "norm2" ([H] values) and "q", "k", "v", "o", "gate", "up", "down" (weights
    [out][in] as lists of values).  candidate = (name, s, W_hat) runs that
    linear in its deployed form: input bf16(fp32(a / s)) against the dequantized
    weights W_hat (values).  Returns the block output [L][H] (values)."""
    L = len(x_rows)

    def lin(name, a):
        if candidate is not None and candidate[0] == name:
            _, s, what = candidate
            xs = [round_bf16(f32(a[c] / s[c])) for c in range(len(a))]
            return matvec(what, xs)
        return matvec(blk[name], a)

    a = [rms_row(x, blk["norm1"]) for x in x_rows]
    q, k, v = [], [], []
    for t in range(L):
        qt, kt = lin("q", a[t]), lin("k", a[t])
        q.append([rb(e) for h in range(n_q) for e in rotate_pairs(qt[128 * h:128 * h + 128], t)])
        k.append([rb(e) for h in range(n_kv) for e in rotate_pairs(kt[128 * h:128 * h + 128], t)])
        v.append(lin("v", a[t]))
    att = [[rb(e) for e in row] for row in causal_attention(q, k, v, L, n_q, n_kv)]
    out = []
    for t in range(L):
        ot = lin("o", att[t])
        h1 = [rb(x_rows[t][c] + ot[c]) for c in range(len(ot))]
        b = rms_row(h1, blk["norm2"])
        gt, ut = lin("gate", b), lin("up", b)
        m = [rb(gt[i] / (1.0 + math.exp(-gt[i])) * ut[i]) for i in range(len(gt))]
        dt = lin("down", m)
        out.append([rb(h1[c] + dt[c]) for c in range(len(dt))])
    return out
