"""Pins of the CPU oracle against things other than itself.

Each ``check_*`` function raises AssertionError when the oracle disagrees with:
hand-computed worked groups (``tests/golden/worked_groups.json``), bf16
conversion by a library routine (torch), closed forms, algebraic invariants of
the definitions, special cases, or a scalar brute-force restatement
(``tests/scalar_reference.py``) on tiny inputs.  The checks are plain functions
so that ``test_oracle_mutants.py`` can re-run them against planted mistakes.

Definitions pinned: model card "rebuttal_w4g128_awq_w2" (details table rows
"Scheme" and "Search"; the scale-rewrite paragraph; "Clipping granularity";
the RTN note under the perplexity table); model card "Qwen3.6-27B-W4A16"
(opening paragraph: symmetric int4 g128, activations 16-bit); benchmark record
"AWQ INT4-g128 WikiText-2 perplexity delta vs fp16, Llama-2 7B" ("Methodology":
group 128, alpha grid of 20).
"""
from __future__ import annotations

import json
import os

import numpy as np

from oracle import w4a16_oracle as O
from tests import scalar_reference as S
from workloads import round_to_bf16_bits, small_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_groups.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _group_values(g):
    fill = g.get("fill", 0.0)
    vals = np.full(128, fill, dtype=np.float32)
    for k, v in g.get("listed", g.get("listed_all", {})).items():
        vals[int(k)] = v
    return vals


def _bits(vals):
    bits = round_to_bf16_bits(np.asarray(vals, dtype=np.float32))
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), vals), "fixture not bf16-exact"
    return bits


# ----------------------------------------------------------------------------- bf16

def check_bf16_golden():
    for src, dst in _golden()["bf16"]["cases"]:
        x = np.array([int(src, 16)], dtype=np.uint32).view(np.float32)
        assert int(O.f32_to_bf16(x)[0]) == int(dst, 16), (src, dst)


def check_bf16_against_torch():
    import torch
    rng = np.random.default_rng(7)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(3.0)
    u = x.view(np.uint32)
    u[:5000] = (u[:5000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)   # exact ties
    x = u.view(np.float32)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16(x), want)
    back = torch.from_numpy(want.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(O.bf16_to_f32(want), back)


# ----------------------------------------------------------------------------- worked groups

def check_worked_groups():
    for g in _golden()["groups"]:
        vals = _group_values(g)
        W = _bits(vals)[None, :]
        sym = g["symmetric"]
        codes, scales, zeros = O.quantize_rtn(W, symmetric=sym)
        assert int(scales[0, 0]) == int(g["scale_bits"], 16), (g["name"], hex(int(scales[0, 0])))
        if not sym:
            assert int(zeros[0, 0]) == g["zero"], g["name"]
        want = np.full(128, g["code_unlisted"], dtype=np.int64)
        for k, c in g["codes_listed"].items():
            want[int(k)] = c
        assert np.array_equal(codes[0].astype(np.int64), want), (g["name"], codes[0][:12])
        qw, sc, qz = O.quantize_pack(W, symmetric=sym)
        deq = O.dequantize(qw, sc, qz, 128, sym)
        for k, d in g["dequant_listed"].items():
            assert deq[0, int(k)] == np.float32(d), (g["name"], k, deq[0, int(k)], d)
        for i, word in g.get("qweight_words", {}).items():
            assert int(qw[0, int(i)]) == int(word, 16), (g["name"], i, hex(int(qw[0, int(i)])))
        if "qzeros_word0" in g:
            assert int(qz[0, 0]) == int(g["qzeros_word0"], 16)


def check_pack_golden():
    p = _golden()["pack"]
    w = O.pack_nibbles(np.array([p["codes"]], dtype=np.uint8))
    assert int(w[0, 0]) == int(p["word"], 16)


# ----------------------------------------------------------------------------- invariants

def _rand_w(N=24, K=512, seed=3, std=0.02):
    _, W = small_case(1, K, N, seed, w_std=std)
    return W


def check_pack_roundtrip():
    rng = np.random.default_rng(11)
    for n in (8, 16, 24, 40, 136, 5):
        c = rng.integers(0, 16, size=(7, n)).astype(np.uint8)
        assert np.array_equal(O.unpack_nibbles(O.pack_nibbles(c), n), c)
    # padding nibbles are zero
    w = O.pack_nibbles(np.full((1, 5), 15, dtype=np.uint8))
    assert int(w[0, 0]) == 0x000FFFFF


def check_ranges_and_error_bound():
    W = _rand_w()
    for sym in (False, True):
        codes, scales, zeros = O.quantize_rtn(W, symmetric=sym)
        assert codes.max() <= 15
        if zeros is not None:
            assert zeros.max() <= 15
        v = O.bf16_to_f32(W).reshape(W.shape[0], -1, 128)
        sc = O.bf16_to_f32(scales)[..., None]
        z = 8.0 if sym else zeros.astype(np.float64)[..., None]
        deq = (codes.reshape(v.shape).astype(np.float64) - z) * sc
        err = np.abs(deq - v)
        c = codes.reshape(v.shape)
        if sym:
            # absmax / sc <= 7 (1 + 2^-8) < 7.5, so no code is clamped: every value is
            # within half a step of its reconstruction, and |code| <= 7
            assert np.all(err <= sc / 2 + 1e-12), float((err - sc / 2).max())
            assert codes.min() >= 1
        else:
            # the bf16 scale can sit up to 2^-8 below (hi - lo)/15, so only the top code
            # may be clamped, by at most 15 * 2^-8 of a step
            top = c == 15
            assert np.all(err[~top] <= np.broadcast_to(sc / 2 + 1e-12, err.shape)[~top])
            assert np.all(err <= sc * (0.5 + 15 * 2.0 ** -8) + 1e-12)


def check_asym_range_covers_group():
    """Asymmetric: sc >= (hi - lo)/15 up to bf16 rounding, so 15 steps span the group."""
    W = _rand_w(N=16, K=1024, seed=5)
    codes, scales, zeros = O.quantize_rtn(W)
    v = O.bf16_to_f32(W).astype(np.float64).reshape(16, -1, 128)
    rng_ = v.max(-1) - v.min(-1)
    sc = O.bf16_to_f32(scales).astype(np.float64)
    assert np.all(np.abs(sc * 15 - rng_) <= rng_ * 2.0 ** -8 + 1e-12)
    # the minimum of each group maps to a code <= 1 and the maximum to >= 14
    c = codes.reshape(16, -1, 128)
    idx_lo = v.argmin(-1)
    idx_hi = v.argmax(-1)
    clo = np.take_along_axis(c, idx_lo[..., None], -1)
    chi = np.take_along_axis(c, idx_hi[..., None], -1)
    assert clo.max() <= 1 and chi.min() >= 14


def check_symmetric_oddness():
    W = _rand_w(seed=9)
    Wneg = W ^ np.uint16(0x8000)
    qa, sa, _ = O.quantize_pack(W, symmetric=True)
    qb, sb, _ = O.quantize_pack(Wneg, symmetric=True)
    assert np.array_equal(sa, sb)
    da = O.dequantize(qa, sa, None, W.shape[1], True)
    db = O.dequantize(qb, sb, None, W.shape[1], True)
    assert np.array_equal(da, -db)


def check_power_of_two_equivariance():
    W = _rand_w(seed=13)
    for sym in (False, True):
        for j in (-3, 2):
            f = np.float32(2.0 ** j)
            qa, sa, za = O.quantize_pack(W, symmetric=sym)
            s = np.full(W.shape[1], f, dtype=np.float32)
            qb, sb, zb = O.quantize_pack(W, s=s, symmetric=sym)
            da = O.dequantize(qa, sa, za, W.shape[1], sym)
            db = O.dequantize(qb, sb, zb, W.shape[1], sym)
            assert np.array_equal(da * f, db), (sym, j)
            assert np.array_equal(qa, qb)


def check_scale_multiplies_input_channels():
    """W diag(s): s_k scales column k (input channel) of every row, not row n."""
    W = _rand_w(N=8, K=256, seed=21)
    s = np.ones(256, dtype=np.float32)
    s[:128] = 4.0                       # first group scaled by a power of two
    qa, sa, za = O.quantize_pack(W)
    qb, sb, zb = O.quantize_pack(W, s=s)
    da = O.dequantize(qa, sa, za, 256, False)
    db = O.dequantize(qb, sb, zb, 256, False)
    assert np.array_equal(db[:, :128], 4 * da[:, :128])
    assert np.array_equal(db[:, 128:], da[:, 128:])


def check_clip_is_clamp():
    """r < 1 clamps each group of W diag(s) at +-r*absmax; r = 1 is the identity."""
    g = np.zeros(128, dtype=np.float32)
    g[0], g[1], g[2] = -1.0, 2.0, 0.5
    W = _bits(g)[None, :]
    # r = 0.5: t = 1.0 -> group becomes {-1, 1, 0.5, 0...}: lo=-1, hi=1, sc = bf16(2/15)
    codes, scales, zeros = O.quantize_rtn(W, clip_ratio=0.5)
    sc = O.bf16_to_f32(scales)[0, 0]
    assert sc == O.bf16_to_f32(O.f32_to_bf16(np.float32(2.0) / np.float32(15.0)))
    d = O.dequantize(O.pack_nibbles(codes), scales, O.pack_nibbles(zeros), 128, False)[0]
    assert abs(d[1] - 1.0) <= sc / 2 and abs(d[0] + 1.0) <= sc / 2
    q1 = O.quantize_pack(W, clip_ratio=1.0)
    q0 = O.quantize_pack(W)
    assert all(np.array_equal(a, b) for a, b in zip(q1, q0))


def check_dequant_exact():
    W = _rand_w(seed=17)
    qw, sc, qz = O.quantize_pack(W)
    d = O.dequantize(qw, sc, qz, W.shape[1], False).astype(np.float64)
    codes = O.unpack_nibbles(qw, W.shape[1]).astype(np.float64).reshape(W.shape[0], -1, 128)
    z = O.unpack_nibbles(qz, W.shape[1] // 128).astype(np.float64)[..., None]
    exact = ((codes - z) * O.bf16_to_f32(sc).astype(np.float64)[..., None]).reshape(W.shape)
    assert np.array_equal(d, exact)


# ----------------------------------------------------------------------------- contraction

def check_linear_special_cases():
    X, W = small_case(3, 256, 12, 23)
    qw, sc, qz = O.quantize_pack(W)
    What = O.dequantize(qw, sc, qz, 256, False)
    # one-hot activations pick out one input channel of every row exactly
    for k in (0, 127, 128, 255):
        onehot = np.zeros((1, 256), dtype=np.uint16)
        onehot[0, k] = 0x3F80          # 1.0 in bf16
        y = O.linear(onehot, What)
        assert np.array_equal(y[0], What[:, k].astype(np.float64))
    assert not O.linear(np.zeros((2, 256), dtype=np.uint16), What).any()
    # brute force on a tiny product
    Xf = O.bf16_to_f32(X).astype(np.float64)
    bf = [[sum(float(Xf[m, k]) * float(What[n, k]) for k in range(256)) for n in range(12)] for m in range(3)]
    assert np.allclose(O.linear(X, What), np.array(bf), rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------------------- AWQ search

def check_grids():
    a = O.alpha_grid()
    assert a.size == 20 and a[0] == 0.0 and np.allclose(np.diff(a), 0.05) and a[-1] < 1.0
    r = O.shrink_grid()
    assert r.size == 10 and r[0] == 1.0 and r.min() >= 0.5 and np.all(np.diff(r) < 0)


def check_act_stat_closed_form():
    X = np.zeros((4, 256), dtype=np.float32)
    X[:, :128] = [[1.0], [-1.0], [3.0], [-3.0]]       # mean |x| = 2 on the first 128 channels
    X[:, 128:] = 0.5
    m = O.act_mean_abs(round_to_bf16_bits(X))
    assert np.all(m[:128] == 2.0) and np.all(m[128:] == 0.5)


def check_scales_closed_form():
    m = np.array([0.25, 1.0, 4.0, 16.0])
    s1 = O.awq_scales(m, 1.0)                       # p = m; sqrt(16 * 0.25) = 2
    assert np.array_equal(s1, np.array([0.125, 0.5, 2.0, 8.0], dtype=np.float32))
    s0 = O.awq_scales(m, 0.0)
    assert np.array_equal(s0, np.ones(4, dtype=np.float32))
    s5 = O.awq_scales(m, 0.5)                       # p = sqrt(m) = .5,1,2,4; sqrt(4*.5) = sqrt 2
    assert np.allclose(s5, np.array([0.5, 1, 2, 4]) / np.sqrt(2.0), rtol=1e-7)
    # a zero statistic is floored at 1e-4 before normalising: p = (1e-4, 1), sqrt(1e-4) = 0.01
    assert np.allclose(O.awq_scales(np.array([0.0, 1.0]), 0.5), [0.01, 100.0], rtol=1e-6)


def check_rewrite_identity():
    """X (Q(W diag s) diag(1/s))^T == (X diag(1/s)) Q(W diag s)^T; bit-exact for power-of-two s."""
    X, W = small_case(6, 256, 8, 31)
    rng = np.random.default_rng(3)
    for pow2 in (True, False):
        if pow2:
            s = (2.0 ** rng.integers(-2, 3, size=256)).astype(np.float32)
        else:
            s = np.exp(rng.standard_normal(256) * 0.5).astype(np.float32)
        qw, sc, qz = O.quantize_pack(W, s=s)
        What = O.dequantize(qw, sc, qz, 256, False).astype(np.float64)
        Xf = O.bf16_to_f32(X).astype(np.float64)
        lhs = Xf @ (What / s.astype(np.float64)).T
        rhs = (Xf / s.astype(np.float64)) @ What.T
        if pow2:
            assert np.array_equal(lhs, rhs)
        else:
            assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-14)
        Yref = O.reference_output(X, W)
        want = float(np.mean((rhs - Yref) ** 2))
        got = O.candidate_loss(X, W, s, 1.0)
        assert abs(got - want) <= 1e-12 * want, (got, want)


def check_alpha_zero_is_rtn():
    X, W = small_case(16, 256, 8, 37)
    m = O.act_mean_abs(X)
    s0 = O.awq_scales(m, 0.0)
    assert np.array_equal(s0, np.ones(256, dtype=np.float32))
    rtn = O.candidate_loss(X, W, s0, 1.0)
    qw, sc, qz = O.quantize_pack(W)
    What = O.dequantize(qw, sc, qz, 256, False)
    d = O.linear(X, What) - O.reference_output(X, W)
    assert O.candidate_loss(X, W, s0, 1.0) == float(np.mean(d * d)) == rtn
    res = O.search(X, W)
    assert res["alpha_losses"][0] == rtn
    assert min(res["alpha_losses"]) <= rtn


def check_loss_closed_form_reference():
    """Y_ref is the bf16-rounded unquantized output; a weight with exact 4-bit
    structure (every group already on its grid) has loss equal to the squared
    bf16 rounding of the reference alone."""
    rng = np.random.default_rng(41)
    N, K = 4, 256
    codes = rng.integers(0, 16, size=(N, K)).astype(np.float32)
    codes[:, ::128] = 0.0
    codes[:, 1::128] = 15.0                        # every group spans 0..15 exactly
    Wf = (codes - 8.0) * np.float32(0.0625)        # sc = 15*0.0625/15, z = 8: exact on the grid
    W = round_to_bf16_bits(Wf)
    X = round_to_bf16_bits(rng.standard_normal((5, K)).astype(np.float32))
    qw, sc, qz = O.quantize_pack(W)
    assert np.array_equal(O.dequantize(qw, sc, qz, K, False), Wf)
    y = O.linear(X, Wf.astype(np.float64))
    yref = O.bf16_to_f32(O.f32_to_bf16(y.astype(np.float32))).astype(np.float64)
    want = float(np.mean((y - yref) ** 2))
    got = O.candidate_loss(X, W, np.ones(K, np.float32), 1.0)
    assert abs(got - want) <= 1e-15 + 1e-12 * want


def check_bruteforce_search():
    """K=256, N=4, T=8, all 30 candidates: the scalar restatement agrees to 1e-10."""
    X, W = small_case(8, 256, 4, 43)
    rng = np.random.default_rng(43)
    mag = np.exp(rng.standard_normal(256)).astype(np.float32)
    X = round_to_bf16_bits(O.bf16_to_f32(X) * mag)
    Xr = O.bf16_to_f32(X).astype(np.float64).tolist()
    Wr = O.bf16_to_f32(W).astype(np.float64).tolist()
    alphas = O.alpha_grid().tolist()
    ratios = O.shrink_grid().tolist()
    for sym in (False, True):
        la, lr, ia, ir = S.search(Xr, Wr, alphas, ratios, sym)
        res = O.search(X, W, symmetric=sym)
        assert np.allclose(res["alpha_losses"], la, rtol=1e-10, atol=0), sym
        assert np.allclose(res["ratio_losses"], lr, rtol=1e-10, atol=0), sym
        assert res["alpha_index"] == ia and res["ratio_index"] == ir


def check_bruteforce_quantizer_random():
    """Scalar restatement vs vectorised quantizer, bit-exact, with s and clipping."""
    rng = np.random.default_rng(47)
    for sym in (False, True):
        for r in (1.0, 0.85):
            _, W = small_case(1, 256, 6, int(1000 * r) + sym)
            s = np.exp(rng.standard_normal(256) * 0.7).astype(np.float32)
            qw, sc, qz = O.quantize_pack(W, s=s, clip_ratio=r, symmetric=sym)
            d = O.dequantize(qw, sc, qz, 256, sym).astype(np.float64)
            ref = S.quantize_dequant(O.bf16_to_f32(W).astype(np.float64).tolist(),
                                     s.astype(np.float64).tolist(), r, sym)
            assert np.array_equal(d, np.array(ref)), (sym, r)


def check_division_ties():
    """Codes are rint of the IEEE fp32 quotient v / sc, ties to even.

    Group 0 is {0, 1, t...}: sc = bf16(1/15) = 137/2048, z = 0.  Group 1 is
    {0, 1.203125, t...}: sc = bf16(1.203125/15) = 164/2048, z = 0.  Each
    t = (k + 1/2) sc is exact in fp32, so v / sc is exactly k + 1/2 and the code is
    the even neighbour (for sc = 164/2048, multiplying by a rounded reciprocal
    instead of dividing misses the ties at k = 3, 7 and 13).  The fp32 neighbours
    of each tie are checked against the scalar restatement, which forms the
    correctly rounded quotient independently.
    """
    s = np.ones(256, dtype=np.float32)
    Wf = np.zeros(256, dtype=np.float32)
    for g, (hi, num) in enumerate(((1.0, 137.0), (1.203125, 164.0))):
        sc = num / 2048.0
        ties = [(k + 0.5) * sc for k in range(14)]
        below = [float(np.nextafter(np.float32(t), np.float32(0))) for t in ties]
        above = [float(np.nextafter(np.float32(t), np.float32(2))) for t in ties]
        vals = [0.0, hi] + ties + below + above
        base = 128 * g
        Wf[base + 1] = hi
        Wf[base + 2: base + len(vals)] = 1.0          # v = 1.0 * s_k
        s[base + 2: base + len(vals)] = np.array(vals[2:], dtype=np.float32)
    W = round_to_bf16_bits(Wf)[None, :]
    codes, scales, zeros = O.quantize_rtn(W, s=s)
    assert int(scales[0, 0]) == 0x3D89 and int(scales[0, 1]) == 0x3DA4
    assert int(zeros[0, 0]) == 0 and int(zeros[0, 1]) == 0
    for g in range(2):
        for k in range(14):
            assert int(codes[0, 128 * g + 2 + k]) == (k if k % 2 == 0 else k + 1), (g, k)
    ref = S.quantize_dequant([Wf.astype(np.float64).tolist()], s.astype(np.float64).tolist(), 1.0, False)
    d = O.dequantize(O.pack_nibbles(codes), scales, O.pack_nibbles(zeros), 256, False)
    assert np.array_equal(d[0].astype(np.float64), np.array(ref[0]))


def check_w4a8_activation_codes():
    """Per-row int8 activations: codes in [-127, 127], the absmax element of every
    nonzero row maps to +-127 exactly, an all-zero row gives scale 1 and codes 0,
    integer rows containing +-127 come back unchanged (scale 1), quotients at
    k + 1/2 round to the even neighbour, and xsum is the per-group code sum
    (pure-Python loop)."""
    rng = np.random.default_rng(7)
    X = round_to_bf16_bits(rng.standard_normal((5, 384)).astype(np.float32) * 3)
    X[3] = 0
    xq, sx, xs = O.quantize_activations_int8(X)
    assert xq.dtype == np.int8 and xq.min() >= -127 and xq.max() <= 127
    x = O.bf16_to_f32(X)
    for m in (0, 1, 2, 4):
        j = int(np.argmax(np.abs(x[m])))
        assert abs(int(xq[m, j])) == 127 and np.sign(xq[m, j]) == np.sign(x[m, j])
        assert sx[m] == np.float32(np.abs(x[m]).max()) / np.float32(127)
    assert sx[3] == 1.0 and not xq[3].any()
    ints = np.array([[127, -3, 5, 0] * 32, [-127, 126, 1, -1] * 32], dtype=np.float32)
    q2, s2, _ = O.quantize_activations_int8(round_to_bf16_bits(ints))
    assert np.all(s2 == 1.0) and np.array_equal(q2.astype(np.float32), ints)
    # ties: row absmax 127 * 2 -> sx = 2, values 2k + 1 divide to k + 1/2 exactly
    half = np.array([[254.0] + [2 * k + 1.0 for k in range(127)]], dtype=np.float32)
    q3, s3, _ = O.quantize_activations_int8(round_to_bf16_bits(half))
    assert s3[0] == 2.0
    for k in range(127):
        want = k if k % 2 == 0 else k + 1
        assert int(q3[0, 1 + k]) == min(want, 127), k
    for m in range(5):
        for g in range(3):
            tot = 0
            for k in range(128 * g, 128 * g + 128):
                tot += int(xq[m, k])
            assert xs[m, g] == tot


def check_w4a8_linear_reduces_to_dequant_matmul():
    """The W4A8 contraction equals a library fp64 matmul of the dequantized codes:
    Y = diag(sx) (Xq W_hat^T) with W_hat the W4A16 dequantization, asymmetric and
    symmetric, and a one-hot code row picks sx * W_hat[n][k] * 127."""
    W = _rand_w(N=9, K=384, seed=11)
    rng = np.random.default_rng(12)
    X = round_to_bf16_bits(rng.standard_normal((3, 384)).astype(np.float32))
    xq, sx, _ = O.quantize_activations_int8(X)
    for sym in (False, True):
        qw, sc, qz = O.quantize_pack(W, None, 1.0, sym)
        Wh = O.dequantize(qw, sc, qz, 384, sym).astype(np.float64)
        y = O.w4a8_linear(xq, sx, qw, sc, qz, 384, sym)
        ref = sx.astype(np.float64)[:, None] * (xq.astype(np.float64) @ Wh.T)
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-12), sym
        onehot = np.zeros((1, 384), dtype=np.int8)
        onehot[0, 200] = 127
        y1 = O.w4a8_linear(onehot, np.array([0.5], np.float32), qw, sc, qz, 384, sym)
        assert np.array_equal(y1[0], 0.5 * 127 * Wh[:, 200])


def check_clip_channel_bruteforce():
    """Per-channel clipping losses and choices: the scalar restatement agrees to
    1e-10 on K=256, N=3, T=6 with a non-trivial s, both quantizer forms."""
    X, W = small_case(6, 256, 3, 53)
    rng = np.random.default_rng(53)
    s = np.exp(rng.standard_normal(256) * 0.5).astype(np.float32)
    ratios = O.shrink_grid()
    Xr = O.bf16_to_f32(X).astype(np.float64).tolist()
    Wr = O.bf16_to_f32(W).astype(np.float64).tolist()
    for sym in (False, True):
        Ls, bs = S.per_channel_clip_losses(Xr, Wr, s.astype(np.float64).tolist(), ratios.tolist(), sym)
        L, best = O.clip_search_per_channel(X, W, s, ratios, sym)
        assert np.allclose(L, np.array(Ls), rtol=1e-10, atol=0), sym
        assert np.array_equal(best, np.array(bs)), sym


def check_clip_channel_special_cases():
    """One-hot deployed activations (x' = unit vectors) make each loss the plain
    squared quantization error of the group; scaling X by 2 scales every loss by 4
    exactly with the same choices; a row subset is the same slice of the full
    result; an all-zero weight row has zero loss everywhere and picks ratio 0."""
    K, N = 256, 4
    W = _rand_w(N=N, K=K, seed=59)
    W[2] = 0
    s = np.exp2(np.random.default_rng(59).integers(-2, 3, size=K)).astype(np.float32)
    X = round_to_bf16_bits(np.diag(s))                     # bf16(X / s) = identity exactly
    ratios = O.shrink_grid()
    for sym in (False, True):
        L, best = O.clip_search_per_channel(X, W, s, ratios, sym)
        v = O.bf16_to_f32(W).astype(np.float64) * s.astype(np.float64)
        for j, r in enumerate(ratios):
            qw, sc, qz = O.quantize_pack(W, s, float(r), sym)
            e = v - O.dequantize(qw, sc, qz, K, sym)
            sq = (e.reshape(N, 2, 128) ** 2).sum(axis=2)   # [N][G]
            assert np.allclose(L[:, :, j], sq.T, rtol=1e-12, atol=0), (sym, j)
        assert not L[:, 2, :].any() and not best[2].any()
        X2, W2 = small_case(5, K, N, 61)
        La, ba = O.clip_search_per_channel(X2, W2, s, ratios, sym)
        Xd = round_to_bf16_bits(O.bf16_to_f32(X2) * np.float32(2))
        Lb, bb = O.clip_search_per_channel(Xd, W2, s, ratios, sym)
        assert np.array_equal(Lb, 4 * La) and np.array_equal(ba, bb)
        Lr, br = O.clip_search_per_channel(X2, W2, s, ratios, sym, rows=[3, 1])
        assert np.array_equal(Lr, La[:, [3, 1], :]) and np.array_equal(br, ba[[3, 1]])


# ----------------------------------------------------------------------------- look-ahead block

def _block(rng, H=256, I=384, n_q=2, n_kv=1, std=0.05):
    w = lambda o, i: round_to_bf16_bits((rng.standard_normal((o, i)) * std).astype(np.float32))
    g = lambda: round_to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    return dict(norm1=g(), norm2=g(), q=w(n_q * 128, H), k=w(n_kv * 128, H), v=w(n_kv * 128, H),
                o=w(H, n_q * 128), gate=w(I, H), up=w(I, H), down=w(H, I))


def check_rope_rotation():
    """Rotary embedding: position 0 is the identity; each (j, j + 64) pair keeps its
    length; q.k after rotation depends only on the position difference; the pure-Python
    rotation agrees; rope() is rope_raw rounded to bf16."""
    rng = np.random.default_rng(71)
    B, L, nh = 2, 6, 2
    x = O.bf16_to_f32(round_to_bf16_bits(rng.standard_normal((B * L, nh * 128)).astype(np.float32)))
    x = x.astype(np.float64)
    r = O.rope_raw(x, B, L, nh)
    xr, rr = x.reshape(B, L, nh, 128), r.reshape(B, L, nh, 128)
    assert np.array_equal(rr[:, 0], xr[:, 0])
    assert np.allclose(rr[..., :64] ** 2 + rr[..., 64:] ** 2, xr[..., :64] ** 2 + xr[..., 64:] ** 2, rtol=1e-12)
    # q at position m, k at n: same vectors placed at every position of a sequence
    qv, kv = x[0, :128], x[1, :128]
    seq = np.zeros((1 * L, 2 * 128))
    seq[:, :128], seq[:, 128:] = qv, kv
    rs = O.rope_raw(seq, 1, L, 2)
    dots = np.array([[rs[m, :128] @ rs[n, 128:] for n in range(L)] for m in range(L)])
    for d in range(-(L - 1), L):
        diag = np.diagonal(dots, offset=d)
        assert np.allclose(diag, diag[0], rtol=1e-10, atol=1e-10), d
    for t in range(L):
        want = S.rotate_pairs(xr[1, t, 1].tolist(), t)
        assert np.allclose(rr[1, t, 1], want, rtol=1e-12, atol=1e-12)
    assert np.array_equal(O.rope(x, B, L, nh), O.bf16_to_f32(O.f32_to_bf16(r.astype(np.float32))).astype(np.float64))


def check_attention():
    """Causal grouped-query attention: the pure-Python loop agrees to 1e-12 (2 query heads
    over 1 key/value head, and 4 over 2); the first token returns its own value; zero
    queries average the values seen so far; a key/value head that is all zero gives
    zero output exactly for the query heads that read it."""
    rng = np.random.default_rng(73)
    for n_q, n_kv in ((2, 1), (4, 2)):
        L = 5
        q = rng.standard_normal((L, n_q * 128))
        k = rng.standard_normal((L, n_kv * 128))
        v = rng.standard_normal((L, n_kv * 128))
        o = O.attention_raw(q, k, v, 1, L, n_q, n_kv)
        want = np.array(S.causal_attention(q.tolist(), k.tolist(), v.tolist(), L, n_q, n_kv))
        assert np.allclose(o, want, rtol=1e-12, atol=1e-12), (n_q, n_kv)
        rep = n_q // n_kv
        for h in range(n_q):
            assert np.allclose(o[0, 128 * h:128 * h + 128], v[0, 128 * (h // rep):128 * (h // rep) + 128], rtol=1e-14)
        oz = O.attention_raw(np.zeros_like(q), k, v, 1, L, n_q, n_kv)
        for t in range(L):
            for h in range(n_q):
                kv = h // rep
                assert np.allclose(oz[t, 128 * h:128 * h + 128], v[:t + 1, 128 * kv:128 * kv + 128].mean(axis=0))
        v2 = v.copy()
        v2[:, :128] = 0
        o2 = O.attention_raw(q, k, v2, 1, L, n_q, n_kv)
        assert not o2[:, :128 * rep].any() and (n_kv == 1 or o2[:, 128 * rep:].all())


def check_rmsnorm_and_silu():
    """RMSNorm of a +-c row with eps 0 is sign * g exactly; of a zero row is zero; silu(0)
    = 0 and silu(g) * 1 matches g sigmoid(g) closed values."""
    g = O.bf16_to_f32(round_to_bf16_bits(np.linspace(0.5, 2, 256).astype(np.float32))).astype(np.float64)
    x = np.where(np.arange(256) % 3 == 0, -3.0, 3.0)[None, :]
    y = O.rmsnorm(x, g, eps=0.0)
    assert np.array_equal(y[0], O._bf16_round(np.sign(x[0]) * g))
    assert not O.rmsnorm(np.zeros((1, 256)), g).any()
    gv = np.array([0.0, 1.0, -2.0, 4.0])
    got = O.silu_mul(gv, np.ones(4))
    want = O._bf16_round(gv / (1 + np.exp(-gv)))
    assert np.array_equal(got, want) and got[0] == 0.0
    assert abs(got[1] - 0.7310585786) < 4e-3 and abs(got[2] + 0.2384058440) < 2e-3


def check_block_and_lookahead():
    """Block with zero o- and down-projections returns its input; a candidate whose
    weights are already on the int4 grid (s = 1, r = 1) reproduces the reference, so
    both losses are 0; without a next block the d = 1 loss equals the d = 0 loss;
    a coarser clip gives a larger loss than none on this block."""
    rng = np.random.default_rng(79)
    B, L, H = 2, 6, 256
    blk = _block(rng, H=H)
    x = round_to_bf16_bits(rng.standard_normal((B * L, H)).astype(np.float32))
    z = dict(blk)
    z["o"] = np.zeros_like(blk["o"])
    z["down"] = np.zeros_like(blk["down"])
    assert np.array_equal(O.block_forward(x, B, L, z, 2, 1), x)
    # weights on the grid: codes 0..15 spanning each group, scale 1/64, zero 8
    for name in ("q", "down"):
        on = dict(blk)
        N, K = blk[name].shape
        codes = rng.integers(0, 16, size=(N, K)).astype(np.float32)
        codes[:, ::128], codes[:, 1::128] = 0.0, 15.0
        on[name] = round_to_bf16_bits((codes - 8.0) * np.float32(1 / 64))
        S1 = np.ones((2, K), np.float32)
        d1, d0 = O.lookahead_losses(x, B, L, on, blk, 2, 1, name, S1, np.array([1.0, 0.6]))
        assert d1[0] == 0.0 and d0[0] == 0.0 and d1[1] > 0 and d0[1] > 0, (name, d1, d0)
    # scale rewrite: per-group powers of two keep the grid, so Q(W diag(s)) diag(1/s) = W
    on = dict(blk)
    N, K = blk["up"].shape
    codes = rng.integers(0, 16, size=(N, K)).astype(np.float32)
    codes[:, ::128], codes[:, 1::128] = 0.0, 15.0
    on["up"] = round_to_bf16_bits((codes - 8.0) * np.float32(1 / 64))
    sg = np.repeat(np.exp2(rng.integers(-2, 3, size=K // 128)).astype(np.float32), 128)
    d1, d0 = O.lookahead_losses(x, B, L, on, blk, 2, 1, "up", sg[None, :], np.array([1.0]))
    assert d1[0] == 0.0 and d0[0] == 0.0
    nxt = _block(rng, H=H)
    S2 = np.ones((2, H), np.float32)
    e1, e0 = O.lookahead_losses(x, B, L, blk, None, 2, 1, "gate", S2, np.array([1.0, 0.5]))
    assert np.array_equal(e1, e0)
    f1, f0 = O.lookahead_losses(x, B, L, blk, nxt, 2, 1, "gate", S2, np.array([1.0, 0.5]))
    assert np.array_equal(f0, e0) and f1[1] > f1[0] > 0


def check_search_lookahead_statistic_and_ties():
    """The look-ahead search takes m from the linear's own input (for gate: the second
    RMSNorm's output) and keeps the first of equal minima: with equal-magnitude inputs
    every alpha gives the same s, so all alpha losses tie and alpha 0 is chosen."""
    rng = np.random.default_rng(83)
    B, L, H = 1, 8, 256
    blk = _block(rng, H=H)
    blk["norm2"] = round_to_bf16_bits(np.ones(H, np.float32))
    x = round_to_bf16_bits(np.where(rng.random((B * L, H)) < 0.5, -1.0, 1.0).astype(np.float32))
    blk["o"] = np.zeros_like(blk["o"])              # h = x, so the gate input is rmsnorm(x) = x
    ins = {}
    O.block_forward(x, B, L, blk, 2, 1, inputs=ins)
    assert np.array_equal(ins["gate"], O.bf16_to_f32(x).astype(np.float64))
    res = O.search_lookahead(x, B, L, blk, None, 2, 1, "gate", alphas=[0.0, 0.3, 0.7], ratios=[1.0, 0.9])
    assert np.all(res["alpha_losses"] == res["alpha_losses"][0]) and res["alpha_index"] == 0
    assert np.array_equal(res["s"], np.ones(H, np.float32))


def check_block_scalar_restatement():
    """The oracle's block, op by op, against the pure-Python token loop of
    tests/scalar_reference.py on a tiny block (H = 128, feed-forward 256, two query
    heads over one key/value head, two sequences of three tokens): bit-identical
    outputs, with every linear unquantized and with the gate projection replaced
    by its deployed int4 candidate (non-trivial s and a clip ratio).  The first
    token of each sequence is scaled by 2^-10, so its mean square (about 1e-6) is
    of the order of the norm's epsilon and the epsilon reading shows in the output;
    the weights of the two norms differ, and the gate and up weights differ, so the
    norm each op reads and the projection that carries the SiLU are visible."""
    rng = np.random.default_rng(97)
    B, L, H, I, n_q, n_kv = 2, 3, 128, 256, 2, 1
    blk = _block(rng, H=H, I=I, n_q=n_q, n_kv=n_kv, std=0.08)
    x = rng.standard_normal((B * L, H)).astype(np.float32)
    x[0::L] *= np.float32(2.0 ** -10)
    x = round_to_bf16_bits(x)
    val = lambda b: O.bf16_to_f32(b).astype(np.float64)
    sblk = {k: (val(v).tolist()) for k, v in blk.items()}
    s = np.exp(rng.standard_normal(H) * 0.4).astype(np.float32)
    packed = O.quantize_pack(blk["gate"], s, 0.9, False)
    what = S.quantize_dequant(sblk["gate"], s.astype(np.float64).tolist(), 0.9, False)
    for cand in (None, ("gate", s, packed, False)):
        y = val(O.block_forward(x, B, L, blk, n_q, n_kv, candidate=cand))
        for b in range(B):
            rows = val(x[b * L:(b + 1) * L]).tolist()
            sc = None if cand is None else ("gate", s.astype(np.float64).tolist(), what)
            want = np.array(S.block_tokens(rows, sblk, n_q, n_kv, candidate=sc))
            got = y[b * L:(b + 1) * L]
            assert np.array_equal(got, want), (cand is None, b, np.argwhere(got != want)[:4])


def check_rmsnorm_epsilon_closed_form():
    """RMSNorm of a constant row c with unit weight is bf16(c / sqrt(c^2 + eps)):
    with c = 2^-10 (mean square 2^-20, about 1e-6) and c = 2^-7, eps = 1e-6 (the
    reading; the pages name no value) gives the closed values below, which any
    other eps of the same order misses."""
    g = np.ones(256)
    for c in (2.0 ** -10, 2.0 ** -7):
        y = O.rmsnorm(np.full((1, 256), c), g)
        want = S.rb(c / np.sqrt(c * c + 1e-6))
        assert np.all(y == want), (c, y[0, 0], want)
    y = O.rmsnorm(np.full((1, 256), 2.0 ** -10), g)
    assert abs(y[0, 0] - 0.6987) < 4e-3


ALL_CHECKS = [
    check_search_lookahead_statistic_and_ties, check_rope_rotation, check_attention, check_rmsnorm_and_silu, check_block_and_lookahead,
    check_clip_channel_bruteforce, check_clip_channel_special_cases,
    check_w4a8_activation_codes, check_w4a8_linear_reduces_to_dequant_matmul,
    check_division_ties,
    check_bf16_golden, check_bf16_against_torch, check_worked_groups, check_pack_golden,
    check_pack_roundtrip, check_ranges_and_error_bound, check_asym_range_covers_group,
    check_symmetric_oddness, check_power_of_two_equivariance, check_scale_multiplies_input_channels,
    check_clip_is_clamp, check_dequant_exact, check_linear_special_cases, check_grids,
    check_act_stat_closed_form, check_scales_closed_form, check_rewrite_identity,
    check_alpha_zero_is_rtn, check_loss_closed_form_reference, check_bruteforce_search,
    check_bruteforce_quantizer_random,
    check_rmsnorm_epsilon_closed_form, check_block_scalar_restatement,
]
