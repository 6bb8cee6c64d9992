"""GPU path (through the C ABI) against the CPU oracle, on the same seeded inputs.

Bars:
* quantize + pack: bit-exact (qweight, scales, qzeros).
* GEMV / GEMM: relative Frobenius error <= 2e-3 against the fp64 oracle on the
  same dequantized weights, and elementwise within half a bf16 ulp of the exact
  value plus 1e-4 of the output RMS (the kernels keep every group sum exact in
  integer weights and round once, at the store).
* grid loss: every loss within 2e-3 relative of the oracle's; the chosen index
  equals the oracle's or the oracle's losses at the two indices are within 2e-3.
"""
import numpy as np
import pytest
import torch

import weight_only_int4_amd as w4
import workloads as wl
from oracle import w4a16_oracle as O
from tests.gpu_util import (bf16_values, bits16, bits32, gpu_available, rel_fro, say, to_bf16, to_f32,
                            to_i32)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

FRO_TOL = 2e-3


def _quant_gpu(W, s=None, r=1.0, sym=False):
    qw, sc, qz = w4.awq_quantize_pack(to_bf16(W), None if s is None else to_f32(s), r, sym)
    torch.cuda.synchronize()
    return bits32(qw), bits16(sc), None if qz is None else bits32(qz)


def _assert_quant_equal(W, s=None, r=1.0, sym=False):
    gq, gs, gz = _quant_gpu(W, s, r, sym)
    oq, os_, oz = O.quantize_pack(W, s, r, sym)
    assert np.array_equal(gs, os_), f"scales differ at {np.argwhere(gs != os_)[:5]}"
    if not sym:
        assert np.array_equal(gz, oz), f"zeros differ at {np.argwhere(gz != oz)[:5]}"
    assert np.array_equal(gq, oq), f"codes differ at {np.argwhere(gq != oq)[:5]}"


def _fro_ok(y, ref):
    """Relative Frobenius error <= 2e-3; for outputs so few that the bf16 rounding of
    the exact result alone exceeds that, <= that rounding floor + 2e-4."""
    floor = rel_fro(bf16_values(O.f32_to_bf16(np.asarray(ref, dtype=np.float32))), ref)
    err = rel_fro(y, ref)
    assert err <= max(FRO_TOL, floor + 2e-4), (err, floor)
    return err, floor


def _elementwise_ok(y_gpu, y_ref):
    y_ref = np.asarray(y_ref, dtype=np.float64)
    mag = np.abs(y_ref)
    ulp = np.where(mag > 0, 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-300))) - 7), 0.0)
    rms = np.sqrt(np.mean(y_ref ** 2)) if y_ref.size else 0.0
    bound = 0.5 * ulp + 1e-4 * rms + 1e-30
    bad = np.abs(y_gpu - y_ref) > bound
    return int(bad.sum())


# ----------------------------------------------------------------------------- quantize

@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("N,K", [(24, 512), (37, 384), (5, 128), (64, 1152), (3, 8320)])
def test_quantize_small(sym, N, K):
    say("quantize", N, K, sym)
    _, W = wl.small_case(1, K, N, 1000 + N + K)
    _assert_quant_equal(W, sym=sym)


@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("r", [1.0, 0.9, 0.55])
def test_quantize_with_scales_and_clip(sym, r):
    say("quantize s/clip", sym, r)
    _, W = wl.small_case(1, 1024, 48, 77)
    rng = np.random.default_rng(5)
    s = np.exp(rng.standard_normal(1024) * 0.8).astype(np.float32)
    _assert_quant_equal(W, s, r, sym)


def test_quantize_golden_groups():
    """The hand-computed worked groups go through the GPU quantizer unchanged."""
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_groups.json")))
    for grp in g["groups"]:
        vals = np.full(128, grp.get("fill", 0.0), dtype=np.float32)
        for k, v in grp.get("listed", grp.get("listed_all", {})).items():
            vals[int(k)] = v
        W = wl.round_to_bf16_bits(vals)[None, :]
        say("golden", grp["name"])
        gq, gs, gz = _quant_gpu(W, sym=grp["symmetric"])
        assert int(gs[0, 0]) == int(grp["scale_bits"], 16)
        for i, word in grp.get("qweight_words", {}).items():
            assert int(gq[0, int(i)]) == int(word, 16)
        _assert_quant_equal(W, sym=grp["symmetric"])


def test_quantize_division_ties():
    """Exact half-integer quotients and their fp32 neighbours (IEEE division, ties to even)."""
    sc = 164.0 / 2048.0
    ties = [(k + 0.5) * sc for k in range(14)]
    vals = ties + [float(np.nextafter(np.float32(t), np.float32(0))) for t in ties] + \
        [float(np.nextafter(np.float32(t), np.float32(2))) for t in ties]
    s = np.ones(128, dtype=np.float32)
    s[2:2 + len(vals)] = vals
    Wf = np.zeros(128, dtype=np.float32)
    Wf[1] = 1.203125
    Wf[2:2 + len(vals)] = 1.0
    W = wl.round_to_bf16_bits(Wf)[None, :]
    say("division ties")
    _assert_quant_equal(W, s)


def test_quantize_near_ties():
    """Quotients a few dozen ulps from half-integers, in groups of known scale (an
    anchor fixes sc = 5/64 exactly): codes equal to the IEEE-division oracle's on
    either side of every half-integer, whichever way the kernel takes them."""
    c = 5.0 / 64.0
    vals = []
    for k in range(7):
        t = np.float32((k + 0.5) * c)
        for d in (12, 16, 20, 24, 32, 64):
            up, dn = t, t
            for _ in range(d):
                up = np.nextafter(up, np.float32(8))
                dn = np.nextafter(dn, np.float32(0))
            vals += [float(up), float(dn)]
    for sym in (False, True):
        G = (len(vals) + 125) // 126
        s = np.ones(128 * G, dtype=np.float32)
        Wf = np.zeros(128 * G, dtype=np.float32)
        for g in range(G):
            chunk = vals[126 * g:126 * (g + 1)]
            # anchors: symmetric absmax 7c (sc = c); asymmetric min 0, max 15c (sc = c, z = 0)
            Wf[128 * g] = 7.0 * c if sym else 15.0 * c
            Wf[128 * g + 1] = 0.0
            s[128 * g + 2:128 * g + 2 + len(chunk)] = chunk
            Wf[128 * g + 2:128 * g + 2 + len(chunk)] = 1.0
        W = wl.round_to_bf16_bits(Wf)[None, :]
        say("near ties", sym)
        _assert_quant_equal(W, s, sym=sym)


def test_quantize_degenerate_groups():
    """Constant and all-zero groups hit the 1e-5 range floor; a lone outlier clamps."""
    W = np.zeros((4, 256), dtype=np.float32)
    W[1, :] = 0.5
    W[2, :128] = -3.0
    W[3, 5] = 100.0
    W = wl.round_to_bf16_bits(W)
    say("degenerate groups")
    for sym in (False, True):
        for r in (1.0, 0.5):
            _assert_quant_equal(W, None, r, sym)


@pytest.mark.parametrize("shape", [0, 1])
def test_quantize_full_size_large(shape):
    """27B-shaped linears (symmetric): every row of a 1/16 sample, full rows."""
    W = wl.large_weight(shape)
    rows = np.arange(0, W.shape[0], 16)
    say("quantize large", shape, W.shape)
    gq, gs, _ = _quant_gpu(W, sym=True)
    oq, os_, _ = O.quantize_pack(W[rows], None, 1.0, True)
    assert np.array_equal(gs[rows], os_)
    assert np.array_equal(gq[rows], oq)


def test_quantize_full_size_decode_block():
    """The seven linears of one hidden-2048 block, asymmetric, all rows."""
    for layer in range(len(wl.BLOCK_LINEARS)):
        W = wl.decode_weight(0, layer)
        say("quantize block linear", layer, W.shape)
        _assert_quant_equal(W)


# ----------------------------------------------------------------------------- GEMV

def _packed(W, sym, s=None):
    qw, sc, qz = O.quantize_pack(W, s, 1.0, sym)
    return qw, sc, qz


def _gemv_case(X, W, sym):
    qw, sc, qz = _packed(W, sym)
    Y = w4.w4a16_gemv(to_bf16(X), to_i32(qw), to_bf16(sc), None if sym else to_i32(qz), sym)
    torch.cuda.synchronize()
    y = bf16_values(bits16(Y))
    ref = O.linear(X, O.dequantize(qw, sc, qz, W.shape[1], sym))
    return y, ref


@pytest.mark.parametrize("M", list(range(1, 17)))
@pytest.mark.parametrize("sym", [False, True])
def test_gemv_all_m(M, sym):
    say("gemv", M, sym)
    X, W = wl.small_case(M, 2048, 300, 11 + M)
    y, ref = _gemv_case(X, W, sym)
    _fro_ok(y, ref)
    assert _elementwise_ok(y, ref) == 0


@pytest.mark.parametrize("M,K,N", [(1, 128, 1), (1, 384, 37), (3, 1152, 129), (8, 6144, 200), (16, 17408, 70),
                                   (5, 5120, 64), (1, 17408, 33), (9, 8320, 17), (2, 16384, 8), (4, 24576, 5),
                                   (1, 4096, 77), (1, 5120, 65), (1, 8192, 9), (1, 9216, 40), (1, 33792, 12),
                                   (5, 128, 1), (16, 128, 17), (7, 256, 33), (12, 384, 5), (6, 640, 4100),
                                   (16, 8192, 3), (3, 1024, 4097), (3, 17408, 37)])
def test_gemv_ragged(M, K, N):
    say("gemv ragged", M, K, N)
    X, W = wl.small_case(M, K, N, 21)
    for sym in (False, True):
        y, ref = _gemv_case(X, W, sym)
        _fro_ok(y, ref)
        assert _elementwise_ok(y, ref) == 0


def test_gemv_one_hot_and_zero():
    """One-hot activations reproduce bf16 dequantized weights bit-exactly; X = 0 gives 0."""
    _, W = wl.small_case(1, 512, 64, 3)
    qw, sc, qz = _packed(W, False)
    What = O.dequantize(qw, sc, qz, 512, False)
    X = np.zeros((4, 512), dtype=np.uint16)
    for i, k in enumerate((0, 127, 300, 511)):
        X[i, k] = 0x3F80
    say("gemv one-hot")
    Y = w4.w4a16_gemv(to_bf16(X), to_i32(qw), to_bf16(sc), to_i32(qz), False)
    torch.cuda.synchronize()
    got = bits16(Y)
    want = O.f32_to_bf16(What[:, [0, 127, 300, 511]].T.astype(np.float32))
    assert np.array_equal(got, want)
    Y0 = w4.w4a16_gemv(to_bf16(np.zeros((2, 512), np.uint16)), to_i32(qw), to_bf16(sc), to_i32(qz), False)
    torch.cuda.synchronize()
    assert not bf16_values(bits16(Y0)).any()


def test_gemv_decode_block_full_size():
    """All seven linears of block 0 at M in {1, 4, 16}, full size."""
    for layer in range(len(wl.BLOCK_LINEARS)):
        W = wl.decode_weight(0, layer)
        for M in wl.DECODE_MS:
            X = wl.decode_act(0, layer, M)
            say("gemv block", layer, M)
            y, ref = _gemv_case(X, W, False)
            _fro_ok(y, ref)
            assert _elementwise_ok(y, ref) == 0


@pytest.mark.parametrize("shape", [0, 1])
@pytest.mark.parametrize("M", [1, 8])
def test_gemv_large_full_size(shape, M):
    """27B-shaped symmetric linears at M in {1, 8}; oracle on a 1/8 sample of the rows of W."""
    W = wl.large_weight(shape)
    X = wl.large_act(shape, M)
    qw, sc, _ = O.quantize_pack(W, None, 1.0, True)
    say("gemv large", shape, M)
    Y = w4.w4a16_gemv(to_bf16(X), to_i32(qw), to_bf16(sc), None, True)
    torch.cuda.synchronize()
    y = bf16_values(bits16(Y))
    cols = np.arange(0, W.shape[0], 8)
    ref = O.linear(X, O.dequantize(qw[cols], sc[cols], None, W.shape[1], True))
    _fro_ok(y[:, cols], ref)
    assert _elementwise_ok(y[:, cols], ref) == 0


@pytest.mark.parametrize("M,K,N", [(1, 2048, 40000), (2, 2048, 40000), (4, 2048, 36000), (16, 2048, 30000),
                                   (16, 2048, 4104), (8, 2048, 4104), (4, 2048, 8211), (8, 2048, 17942),
                                   (1, 5120, 25601), (3, 2048, 36000), (5, 4096, 4104), (12, 8192, 1000),
                                   (6, 6144, 4100), (10, 2048, 2000), (16, 4096, 600)])
def test_gemv_tall_random_codes(M, K, N):
    """Tall linears: enough rows that every workgroup gets several row batches
    (and, for the larger M, several rounds of workgroups), on both forms of the
    GEMV: the VALU form (M <= 4 on narrow outputs; several row-batch counts per
    workgroup) and the matrix-core form (1 to 8 column blocks per slab; 2 groups
    per wave up to K = 4096 and 4 above, with a K split at K = 8192; entered at
    M = 3 from N = 4096 and at M = 5 otherwise; K = 4096 at M = 16 takes more than
    64 KB of LDS per workgroup).  The packed operands are drawn directly (random
    codes, scales and zero words);
    oracle on every 16th row."""
    rng = np.random.default_rng(1000 + M + N)
    qw = rng.integers(0, 2 ** 32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    sc = O.f32_to_bf16((np.abs(rng.standard_normal((N, K // 128))) * 2e-3 + 1e-4).astype(np.float32))
    qz = rng.integers(0, 2 ** 32, size=(N, (K // 128 + 7) // 8), dtype=np.uint64).astype(np.uint32)
    X = O.f32_to_bf16(rng.standard_normal((M, K)).astype(np.float32))
    rows = np.arange(0, N, 16)
    for sym in (False, True):
        say("gemv tall", M, K, N, sym)
        Y = w4.w4a16_gemv(to_bf16(X), to_i32(qw), to_bf16(sc), None if sym else to_i32(qz), sym)
        torch.cuda.synchronize()
        y = bf16_values(bits16(Y))[:, rows]
        ref = O.linear(X, O.dequantize(qw[rows], sc[rows], None if sym else qz[rows], K, sym))
        _fro_ok(y, ref)
        assert _elementwise_ok(y, ref) == 0


@pytest.mark.parametrize("M,K,N", [(1, 33792, 96), (16, 17408, 200), (1, 2048, 4096), (4, 6144, 2048),
                                   (12, 2048, 4096), (16, 256, 300)])
def test_gemv_deterministic_and_overwrites(M, K, N):
    """Y prefilled with NaN is fully overwritten and two calls agree bit for bit, on
    the direct store (K = 2048 at M = 1; the matrix-core form with one wave per
    slab at K = 256), the cross-wave LDS sums (K = 6144 at M = 4; the matrix-core
    form at K = 2048, M = 12) and the K split with its second reduction kernel
    (K = 33792 at M = 1, K = 17408 at M = 16)."""
    X, W = wl.small_case(M, K, N, 91)
    qw, sc, qz = _packed(W, False)
    args = (to_bf16(X), to_i32(qw), to_bf16(sc), to_i32(qz), False)
    say("gemv determinism", M, K, N)
    Y1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    w4.w4a16_gemv(*args, Y=Y1)
    Y2 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    w4.w4a16_gemv(*args, Y=Y2)
    torch.cuda.synchronize()
    assert not torch.isnan(Y1.float()).any()
    assert np.array_equal(bits16(Y1), bits16(Y2))
    ref = O.linear(X, O.dequantize(qw, sc, qz, K, False))
    _fro_ok(bf16_values(bits16(Y1)), ref)


def test_gemv_rejects_m17():
    _, W = wl.small_case(1, 256, 8, 1)
    qw, sc, qz = _packed(W, False)
    X = np.zeros((17, 256), dtype=np.uint16)
    with pytest.raises(w4.W4Error):
        w4.w4a16_gemv(to_bf16(X), to_i32(qw), to_bf16(sc), to_i32(qz), False)


# ----------------------------------------------------------------------------- GEMM

def _gemm_case(X, W, sym, rows=None):
    qw, sc, qz = _packed(W, sym)
    Y = w4.w4a16_gemm(to_bf16(X), to_i32(qw), to_bf16(sc), None if sym else to_i32(qz), sym)
    torch.cuda.synchronize()
    y = bf16_values(bits16(Y))
    Xr = X if rows is None else X[rows]
    ref = O.linear(Xr, O.dequantize(qw, sc, qz, W.shape[1], sym))
    return (y if rows is None else y[rows]), ref


@pytest.mark.parametrize("M,K,N", [(1, 128, 1), (64, 2048, 128), (200, 384, 200), (256, 1152, 1000),
                                   (129, 2048, 257), (37, 5120, 64), (512, 256, 96), (130, 17408, 130),
                                   (70, 640, 90)])
@pytest.mark.parametrize("sym", [False, True])
def test_gemm_shapes(M, K, N, sym):
    say("gemm", M, K, N, sym)
    X, W = wl.small_case(M, K, N, 31)
    y, ref = _gemm_case(X, W, sym)
    _fro_ok(y, ref)
    assert _elementwise_ok(y, ref) == 0


@pytest.mark.parametrize("M,N", [(2048, 2048), (2048, 2056), (2050, 2048)])
def test_gemm_core_layout_boundary(M, N):
    """Either side of the grid size at which the MFMA core switches from three
    stages and two workgroups per CU to two stages and three: 512 tiles of 64 x 128
    (three stages) and 544 / 528 tiles (two stages) with a ragged column or row
    tail; K = 640 (five groups: both stage parities and an odd count).  Oracle on
    every 16th row."""
    X, W = wl.small_case(M, 640, N, 51)
    rows = np.arange(0, M, 16)
    say("gemm core layout", M, N)
    y, ref = _gemm_case(X, W, False, rows)
    _fro_ok(y, ref)
    assert _elementwise_ok(y, ref) == 0


@pytest.mark.parametrize("M,N", [(1024, 4096), (1025, 4096), (1024, 3968), (2048, 6144)])
def test_gemm_row_tail_and_rounds(M, N):
    """The MFMA core at 512 tiles of 64 x 128 (one round of two workgroups per CU,
    three stages), 544 with a one-row tail (two stages), 496 (three stages, a short
    round) and the prefill width (1536 tiles, two stages); K = 640 (five groups:
    every stage of the ring and an odd count).  Oracle on every 8th row and the
    last one."""
    X, W = wl.small_case(M, 640, N, 57)
    rows = np.unique(np.concatenate([np.arange(0, M, 8), [M - 1]]))
    say("gemm tall boundary", M, N)
    y, ref = _gemm_case(X, W, False, rows)
    _fro_ok(y, ref)
    assert _elementwise_ok(y, ref) == 0


def test_gemm_one_hot_and_zero():
    _, W = wl.small_case(1, 384, 160, 9)
    qw, sc, qz = _packed(W, False)
    What = O.dequantize(qw, sc, qz, 384, False)
    X = np.zeros((130, 384), dtype=np.uint16)
    ks = np.arange(130) * 3 % 384
    X[np.arange(130), ks] = 0x3F80
    say("gemm one-hot")
    Y = w4.w4a16_gemm(to_bf16(X), to_i32(qw), to_bf16(sc), to_i32(qz), False)
    torch.cuda.synchronize()
    assert np.array_equal(bits16(Y), O.f32_to_bf16(What[:, ks].T.astype(np.float32)))


@pytest.mark.parametrize("shape", [0, 1])
def test_gemm_prefill_full_size(shape):
    """M=2048 prefill shapes with x20 outlier channels, full size, all outputs."""
    X, W = wl.prefill(shape)
    say("gemm prefill", shape)
    y, ref = _gemm_case(X, W, False)
    _fro_ok(y, ref)
    assert _elementwise_ok(y, ref) == 0


@pytest.mark.parametrize("M,K,N,sym", [(1, 128, 1, False), (5, 384, 70, True), (16, 4096, 64, False),
                                       (17, 2048, 300, False), (31, 640, 129, True), (33, 17408, 40, False),
                                       (48, 2176, 257, True), (40, 33792, 24, True), (48, 128, 16, False),
                                       (47, 2304, 1000, False), (48, 2048, 17, True), (49, 2048, 130, False),
                                       (17, 2304, 33, False)])
def test_gemm_short_m(M, K, N, sym):
    """The one-pass form for up to 48 rows: one to three row blocks with a ragged
    row tail, ragged column tails, a single group, K within one workgroup's 16
    groups (no split), K splits with a short last range (17 groups: 16 + 1; 18: 16 +
    2; 264: 17 ranges; 17 x 33 outputs, a count the split reduction cannot take
    four at a time), and 49 rows on the tiled core beside it."""
    say("gemm short M", M, K, N, sym)
    X, W = wl.small_case(M, K, N, 77)
    y, ref = _gemm_case(X, W, sym)
    _fro_ok(y, ref)
    assert _elementwise_ok(y, ref) == 0


@pytest.mark.parametrize("M,K,N", [(48, 4096, 300), (20, 2048, 33)])
def test_gemm_short_m_deterministic_and_overwrites(M, K, N):
    """Y prefilled with NaN is fully overwritten and two calls agree bit for bit,
    through the split reduction (32 groups: 2 ranges) and without a split."""
    X, W = wl.small_case(M, K, N, 5)
    qw, sc, qz = _packed(W, False)
    args = (to_bf16(X), to_i32(qw), to_bf16(sc), to_i32(qz), False)
    say("gemm short M determinism", M, K, N)
    Y1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    w4.w4a16_gemm(*args, Y=Y1)
    Y2 = w4.w4a16_gemm(*args)
    torch.cuda.synchronize()
    assert not torch.isnan(Y1.float()).any()
    assert np.array_equal(bits16(Y1), bits16(Y2))


@pytest.mark.parametrize("shape", [0, 1])
@pytest.mark.parametrize("M", [48, 64, 512])
def test_gemm_large_full_size(shape, M):
    W = wl.large_weight(shape)
    X = wl.large_act(shape, M)
    rows = np.arange(0, M, 8)
    say("gemm large", shape, M)
    y, ref = _gemm_case(X, W, True, rows)
    _fro_ok(y, ref)
    assert _elementwise_ok(y, ref) == 0


@pytest.mark.parametrize("M,K,N", [(300, 1024, 300), (64, 17408, 256)])
def test_gemm_deterministic_and_overwrites(M, K, N):
    """Y prefilled with NaN is fully overwritten and two calls agree bit for bit:
    a 2-way K split (300 x 1024 x 300) and a 34-way one (two column tiles of
    136 groups), both through the split reduction; the second also against the
    oracle."""
    X, W = wl.small_case(M, K, N, 5)
    qw, sc, qz = _packed(W, False)
    args = (to_bf16(X), to_i32(qw), to_bf16(sc), to_i32(qz), False)
    say("gemm determinism", M, K, N)
    Y1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    w4.w4a16_gemm(*args, Y=Y1)
    Y2 = w4.w4a16_gemm(*args)
    torch.cuda.synchronize()
    assert not torch.isnan(Y1.float()).any()
    assert np.array_equal(bits16(Y1), bits16(Y2))
    if M == 64:
        y = bf16_values(bits16(Y1))
        ref = O.linear(X, O.dequantize(qw, sc, qz, K, False))
        _fro_ok(y, ref)
        assert _elementwise_ok(y, ref) == 0


# ----------------------------------------------------------------------------- unquantized bf16 linear

@pytest.mark.parametrize("M,K,N", [(1, 64, 1), (130, 192, 257), (64, 2048, 128), (257, 6144, 200), (1000, 128, 129),
                                   (2, 4096, 3000)])
def test_bf16_linear_shapes(M, K, N):
    """Y = bf16(X W^T): within half a bf16 ulp of the fp64 value plus the fp32
    accumulation slack, ragged tiles on both sides."""
    X, W = wl.small_case(M, K, N, 61)
    say("bf16 linear", M, K, N)
    Y = w4.bf16_linear(to_bf16(X), to_bf16(W))
    torch.cuda.synchronize()
    y = bf16_values(bits16(Y))
    ref = O.linear(X, O.bf16_to_f32(W))
    _fro_ok(y, ref)
    assert _elementwise_ok(y, ref) == 0


@pytest.mark.parametrize("M,K,N", [(4096, 2048, 6144), (4096, 6144, 2048), (4096, 2048, 1024)])
def test_bf16_linear_full_size(M, K, N):
    """The search's reference output (T=4096, K=2048, N=6144) and the decoder block's
    down and k/v projections at 8 x 512 tokens; oracle on every 16th row; bit-identical rerun."""
    rng = np.random.default_rng(M + K + N)
    X = wl.round_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    W = wl.round_to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    say("bf16 linear full", M, K, N)
    Xd, Wd = to_bf16(X), to_bf16(W)
    Y = w4.bf16_linear(Xd, Wd)
    Y2 = w4.bf16_linear(Xd, Wd)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)
    rows = np.arange(0, M, 16)
    y = bf16_values(bits16(Y))[rows]
    ref = O.linear(X[rows], O.bf16_to_f32(W))
    _fro_ok(y, ref)
    assert _elementwise_ok(y, ref) == 0


# ----------------------------------------------------------------------------- grid loss

def _grid_inputs(T, K, N, seed):
    X, W = wl.awq_calibration(T, K, N, seed_block=seed)
    m = O.act_mean_abs(X)
    S = np.stack([O.awq_scales(m, a) for a in O.alpha_grid()])
    return X, W, S


@pytest.mark.parametrize("sym", [False, True])
def test_grid_loss_small(sym):
    X, W, S = _grid_inputs(256, 384, 200, 1)
    S = np.concatenate([S, np.repeat(S[6:7], 10, axis=0)])          # 20 alphas + 10 ratios at alpha_6
    ratios = np.concatenate([np.ones(20, np.float32), O.shrink_grid().astype(np.float32)])
    say("grid loss small", sym)
    L = w4.awq_grid_loss(to_bf16(X), to_bf16(W), to_f32(S), to_f32(ratios), sym)
    L2 = w4.awq_grid_loss(to_bf16(X), to_bf16(W), to_f32(S), to_f32(ratios), sym)
    torch.cuda.synchronize()
    got = L.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, L2.cpu().numpy().astype(np.float64)), "grid loss not deterministic"
    want = O.grid_loss(X, W, S, ratios, sym)
    rel = np.abs(got - want) / want
    assert rel.max() <= 2e-3, rel.max()


def test_grid_loss_full_size():
    """The search workload at full size (T=4096, K=2048, N=6144): three candidates in the
    launch configuration the search uses (alpha 0 and 0.3 at r = 1, alpha 0.3 at r = 0.85)."""
    X, W = wl.awq_calibration()
    m = O.act_mean_abs(X)
    S = np.stack([O.awq_scales(m, 0.0), O.awq_scales(m, 0.3), O.awq_scales(m, 0.3)])
    ratios = np.array([1.0, 1.0, 0.85], dtype=np.float32)
    say("grid loss full size", X.shape, W.shape)
    L = w4.awq_grid_loss(to_bf16(X), to_bf16(W), to_f32(S), to_f32(ratios), False)
    torch.cuda.synchronize()
    got = L.cpu().numpy().astype(np.float64)
    want = O.grid_loss(X, W, S, ratios, False)
    assert np.max(np.abs(got - want) / want) <= 2e-3, (got, want)


def test_grid_loss_given_yref():
    X, W, S = _grid_inputs(200, 256, 130, 2)
    ratios = np.ones(S.shape[0], dtype=np.float32)
    Yref = O.f32_to_bf16(O.linear(X, O.bf16_to_f32(W)).astype(np.float32))
    say("grid loss yref")
    L = w4.awq_grid_loss(to_bf16(X), to_bf16(W), to_f32(S), to_f32(ratios), False, Yref=to_bf16(Yref))
    torch.cuda.synchronize()
    want = O.grid_loss(X, W, S, ratios, False)
    assert np.max(np.abs(L.cpu().numpy() - want) / want) <= 2e-3


def _argmin_ok(i_gpu, i_or, losses_or):
    return i_gpu == i_or or abs(losses_or[i_gpu] - losses_or[i_or]) <= 2e-3 * losses_or[i_or]


def test_search_small():
    """Both phases against the oracle.  The second phase is checked at the GPU's own
    alpha*: when a near-tie made it differ from the oracle's, the oracle scores the
    ratio grid at that alpha too."""
    X, W = wl.awq_calibration(512, 256, 192, seed_block=3)
    say("search small")
    res = w4.awq_search(to_bf16(X), to_bf16(W), O.alpha_grid(), O.shrink_grid())
    ref = O.search(X, W)
    la, lr = np.array(res["alpha_losses"]), np.array(res["ratio_losses"])
    assert np.max(np.abs(la - ref["alpha_losses"]) / ref["alpha_losses"]) <= 2e-3
    ia = res["alpha_index"]
    assert _argmin_ok(ia, ref["alpha_index"], ref["alpha_losses"])
    s_gpu = O.awq_scales(O.act_mean_abs(X), O.alpha_grid()[ia])
    assert np.array_equal(res["s"].cpu().numpy(), s_gpu)
    want_r = ref["ratio_losses"] if ia == ref["alpha_index"] else O.grid_loss(
        X, W, np.broadcast_to(s_gpu, (10, s_gpu.size)), O.shrink_grid(), False)
    assert np.max(np.abs(lr - want_r) / want_r) <= 2e-3
    assert _argmin_ok(res["ratio_index"], int(np.argmin(want_r)), want_r)


def test_search_full_size():
    """The 30-candidate two-phase search on the full search workload (T=4096, K=2048,
    N=6144) in the launch configuration the benchmark times, against the oracle's
    search stored by tests/golden/make_search_c5.py: all 30 losses within 2e-3,
    alpha* and r* the oracle's or a near-tie, s(alpha*) bit-identical."""
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "search_c5.json")))
    X, W = wl.awq_calibration()
    assert list(X.shape) == [g["shape"]["T"], g["shape"]["K"]] and W.shape[0] == g["shape"]["N"]
    say("search full size", X.shape, W.shape)
    res = w4.awq_search(to_bf16(X), to_bf16(W), np.array(g["alphas"]), np.array(g["ratios"]))
    la, lr = np.array(res["alpha_losses"]), np.array(res["ratio_losses"])
    oa = np.array(g["alpha_losses"])
    assert np.max(np.abs(la - oa) / oa) <= 2e-3, np.abs(la - oa) / oa
    ia = res["alpha_index"]
    assert _argmin_ok(ia, g["alpha_index"], oa), (ia, g["alpha_index"])
    near = g["ratio_losses_near_tied_alphas"]
    assert str(ia) in near, f"GPU alpha* {ia} is not among the oracle's near-tied alphas {list(near)}"
    orr = np.array(near[str(ia)])
    assert np.max(np.abs(lr - orr) / orr) <= 2e-3, np.abs(lr - orr) / orr
    assert _argmin_ok(res["ratio_index"], int(np.argmin(orr)), orr)
    if ia == g["alpha_index"]:
        want = np.array([int(g["s_bits"][8 * i:8 * i + 8], 16) for i in range(len(g["s_bits"]) // 8)], np.uint32)
        assert np.array_equal(res["s"].cpu().numpy().view(np.uint32), want)


# ----------------------------------------------------------------------------- W4A8 decode

def _w4a8_inputs(X):
    xq, sx, xs = O.quantize_activations_int8(X)
    return (torch.from_numpy(xq).cuda(), torch.from_numpy(sx).cuda(),
            torch.from_numpy(xs.astype(np.int32)).cuda(), xq, sx, xs)


@pytest.mark.parametrize("M,K", [(1, 128), (5, 2048), (16, 5120), (3, 17408)])
def test_w4a8_quantize_activations_bit_exact(M, K):
    say("w4a8 quantize", M, K)
    X, _ = wl.small_case(M, K, 1, 31)
    X[M - 1, : K // 2] = 0                                  # a half-zero row
    if M > 1:
        X[0] = 0                                            # an all-zero row
    Xq, sx, xs = w4.w4a8_quantize_activations(to_bf16(X))
    torch.cuda.synchronize()
    oq, osx, oxs = O.quantize_activations_int8(X)
    assert np.array_equal(Xq.cpu().numpy(), oq)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), osx.view(np.uint32))
    assert np.array_equal(xs.cpu().numpy(), oxs.astype(np.int32))


@pytest.mark.parametrize("M,K,N", [(1, 2048, 300), (4, 2048, 129), (16, 2048, 64), (7, 128, 33), (2, 6144, 17),
                                   (16, 17408, 40), (1, 5120, 1000), (9, 4224, 31), (3, 51200, 20), (5, 9344, 100),
                                   (3, 8064, 40), (3, 8192, 40)])
@pytest.mark.parametrize("sym", [False, True])
def test_w4a8_gemv(M, K, N, sym):
    say("w4a8 gemv", M, K, N, sym)
    X, W = wl.small_case(M, K, N, 41)
    qw, sc, qz = _packed(W, sym)
    gq, gsx, gxs, xq, sx, _ = _w4a8_inputs(X)
    Y = w4.w4a8_gemv(gq, gsx, gxs, to_i32(qw), to_bf16(sc), None if sym else to_i32(qz), sym)
    torch.cuda.synchronize()
    y = bf16_values(bits16(Y))
    ref = O.w4a8_linear(xq, sx, qw, sc, qz, K, sym)
    _fro_ok(y, ref)
    assert _elementwise_ok(y, ref) == 0


@pytest.mark.parametrize("shape", [0, 1])
@pytest.mark.parametrize("M", [1, 16])
def test_w4a8_gemv_large_full_size(shape, M):
    """27B-shaped symmetric linears; activations quantized on the GPU (bit-exact
    with the oracle's); oracle on every 8th output channel."""
    W = wl.large_weight(shape)
    X = wl.large_act(shape, M)
    qw, sc, _ = O.quantize_pack(W, None, 1.0, True)
    say("w4a8 large", shape, M)
    Xq, sx, xs = w4.w4a8_quantize_activations(to_bf16(X))
    Y = w4.w4a8_gemv(Xq, sx, xs, to_i32(qw), to_bf16(sc), None, True)
    torch.cuda.synchronize()
    oq, osx, _ = O.quantize_activations_int8(X)
    assert np.array_equal(Xq.cpu().numpy(), oq)
    y = bf16_values(bits16(Y))
    cols = np.arange(0, W.shape[0], 8)
    ref = O.w4a8_linear(oq, osx, qw[cols], sc[cols], None, W.shape[1], True)
    _fro_ok(y[:, cols], ref)
    assert _elementwise_ok(y[:, cols], ref) == 0


@pytest.mark.parametrize("M,K,N", [(1, 2048, 300), (16, 17408, 40), (3, 51200, 20)])
def test_w4a8_gemv_deterministic_and_overwrites(M, K, N):
    """Y prefilled with NaN is fully overwritten and two calls agree bit for bit:
    one workgroup per 16-channel tile (K = 2048) and the split over K with the
    fp32 partials added in split order (K = 17408 and 51200 on narrow N)."""
    say("w4a8 determinism", M, K, N)
    X, W = wl.small_case(M, K, N, 43)
    qw, sc, qz = _packed(W, False)
    gq, gsx, gxs, _, _, _ = _w4a8_inputs(X)
    args = (gq, gsx, gxs, to_i32(qw), to_bf16(sc), to_i32(qz), False)
    Y1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    w4.w4a8_gemv(*args, Y=Y1)
    Y2 = w4.w4a8_gemv(*args)
    torch.cuda.synchronize()
    assert not torch.isnan(Y1.float()).any()
    assert np.array_equal(bits16(Y1), bits16(Y2))


def test_w4a8_rejects_m17():
    _, W = wl.small_case(1, 256, 8, 1)
    qw, sc, qz = _packed(W, False)
    X = np.zeros((17, 256), dtype=np.uint16)
    with pytest.raises(w4.W4Error):
        w4.w4a8_quantize_activations(to_bf16(X))


# ----------------------------------------------------------------------------- per-channel clipping

# Error bound of the GPU loss e^T H_g e: e and H_g enter the matrix cores as bf16
# hi + lo (residue <= 2^-17 of each entry, the lo x lo product dropped: <= 2^-18),
# H_g and H_g e accumulate in fp32 over at most 256 tokens per slice and 384
# products; all of it is below 2^-13 of the same expression with every term taken
# in absolute value, e^T (|X'|^T |X'|) e with |e|.  The test allows 2^-12 of that.
CLIP_TOL = 2.0 ** -12


def _clip_reference(X, W, s, ratios, sym, rows):
    s32 = np.ones(X.shape[1], np.float32) if s is None else s
    L, best = O.clip_search_per_channel(X, W, s32, ratios, sym, rows=rows)
    xs = np.abs(O.bf16_to_f32(O.f32_to_bf16(O.bf16_to_f32(X) / s32[None, :])).astype(np.float64))
    Wr = W[np.asarray(rows)]
    v = O.bf16_to_f32(Wr).astype(np.float64) * s32.astype(np.float64)
    K = X.shape[1]
    bound = np.zeros_like(L)
    for j, r in enumerate(ratios):
        qw, sc, qz = O.quantize_pack(Wr, s32, float(r), sym)
        e = np.abs(v - O.dequantize(qw, sc, qz, K, sym))
        for g in range(K // 128):
            sl = slice(128 * g, 128 * g + 128)
            bound[g, :, j] = ((xs[:, sl] @ e[:, sl].T) ** 2).sum(axis=0)
    return L, best, bound


def _clip_check(X, W, s, ratios, sym, rows=None, repeat=False):
    N, K = W.shape
    rows = list(range(N)) if rows is None else rows
    args = (to_bf16(X), to_bf16(W), to_f32(ratios))
    kw = dict(s=None if s is None else to_f32(s), symmetric=sym)
    L, best = w4.awq_clip_search(*args, **kw)
    torch.cuda.synchronize()
    if repeat:
        L2, best2 = w4.awq_clip_search(*args, **kw)
        torch.cuda.synchronize()
        assert torch.equal(L, L2) and torch.equal(best, best2), "clip search not deterministic"
    got = L.cpu().numpy().astype(np.float64)[:, rows, :]
    gbest = best.cpu().numpy().astype(np.int64)[rows]
    want, wbest, bound = _clip_reference(X, W, s, ratios, sym, rows)
    tol = CLIP_TOL * bound + 1e-30
    bad = np.abs(got - want) > tol
    assert not bad.any(), (f"{int(bad.sum())} losses off; worst excess "
                           f"{np.max((np.abs(got - want) - tol))}, at {np.argwhere(bad)[:4]}")
    G = K // 128
    n_idx = np.arange(len(rows))[:, None]
    g_idx = np.arange(G)[None, :]
    pick = want[g_idx, n_idx, gbest]             # [rows][G] oracle loss at the GPU's choice
    low = want[g_idx, n_idx, wbest]
    slack = tol[g_idx, n_idx, gbest] + tol[g_idx, n_idx, wbest]
    assert np.all(pick <= low + slack), np.argwhere(pick > low + slack)[:4]
    return float(np.mean(gbest == wbest))


@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("with_s", [False, True])
def test_clip_search_small(sym, with_s):
    X, W = wl.awq_calibration(256, 384, 200, seed_block=4)
    s = O.awq_scales(O.act_mean_abs(X), 0.5) if with_s else None
    say("clip search small", sym, with_s)
    agree = _clip_check(X, W, s, O.shrink_grid().astype(np.float32), sym, repeat=True)
    assert agree >= 0.9, agree


@pytest.mark.parametrize("T,K,N", [(77, 128, 37), (1, 256, 5), (130, 1152, 131), (64, 640, 129)])
def test_clip_search_ragged(T, K, N):
    X, W = wl.awq_calibration(T, K, N, seed_block=5)
    s = O.awq_scales(O.act_mean_abs(X), 0.35)
    ratios = np.array([1.0, 0.9, 0.8, 0.7, 0.6, 0.55, 0.5], dtype=np.float32)
    for sym in (False, True):
        say("clip search ragged", T, K, N, sym)
        _clip_check(X, W, s, ratios, sym)


def test_clip_search_degenerate():
    """No tokens: every loss 0 and ratio 0 chosen; all-zero weight rows: losses 0,
    ratio 0; a single ratio; N = 0 is a no-op."""
    X, W = wl.awq_calibration(64, 256, 40, seed_block=6)
    W = W.copy()
    W[[0, 17, 39]] = 0
    ratios = O.shrink_grid().astype(np.float32)
    say("clip search degenerate")
    L, best = w4.awq_clip_search(to_bf16(X[:0]), to_bf16(W), to_f32(ratios))
    torch.cuda.synchronize()
    assert not L.any() and not best.any()
    L, best = w4.awq_clip_search(to_bf16(X), to_bf16(W), to_f32(ratios))
    torch.cuda.synchronize()
    assert not L[:, [0, 17, 39], :].any() and not best[[0, 17, 39]].any()
    _clip_check(X, W, None, ratios[:1], False)
    L, best = w4.awq_clip_search(to_bf16(X), to_bf16(W[:0]), to_f32(ratios))
    torch.cuda.synchronize()
    assert L.numel() == 0 and best.numel() == 0


def test_clip_search_rounding_ties_and_degenerate_groups():
    """Row 0 holds exact half-integer quotients and their fp32 neighbours at ratio 1
    (the codes come from the division itself there); rows 1-4 hold constant, zero and
    single-outlier groups."""
    sc = 164.0 / 2048.0
    ties = [(k + 0.5) * sc for k in range(14)]
    vals = ties + [float(np.nextafter(np.float32(t), np.float32(0))) for t in ties] + \
        [float(np.nextafter(np.float32(t), np.float32(2))) for t in ties]
    s = np.ones(256, dtype=np.float32)
    s[2:2 + len(vals)] = vals
    Wf = np.zeros((5, 256), dtype=np.float32)
    Wf[0, 1] = 1.203125
    Wf[0, 2:2 + len(vals)] = 1.0
    Wf[0, 128:] = np.linspace(-1, 1, 128, dtype=np.float32)
    Wf[1, :] = 0.5
    Wf[2, :128] = -3.0
    Wf[3, 5] = 100.0
    W = wl.round_to_bf16_bits(Wf)
    X = wl.round_to_bf16_bits(np.random.default_rng(12).standard_normal((64, 256)).astype(np.float32))
    ratios = np.array([1.0, 0.9, 0.5], dtype=np.float32)
    for sym in (False, True):
        say("clip search ties and degenerate groups", sym)
        _clip_check(X, W, s, ratios, sym)


@pytest.mark.parametrize("sym", [False, True])
def test_clip_search_full_size(sym):
    """4096 calibration tokens, K = 2048, N = 6144 at s(alpha = 0.5); 48 sampled
    channels (first, last, tile edges, random) against the oracle."""
    X, W = wl.awq_calibration(seed_block=0)
    s = O.awq_scales(O.act_mean_abs(X), 0.5)
    N = W.shape[0]
    rng = np.random.default_rng(11)
    rows = sorted(set([0, 31, 32, 127, 128, N - 129, N - 1] + rng.choice(N, 41, replace=False).tolist()))
    say("clip search full size", sym, X.shape, W.shape)
    _clip_check(X, W, s, O.shrink_grid().astype(np.float32), sym, rows=rows)
