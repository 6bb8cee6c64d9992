"""Decoder block forward and look-ahead (d = 1) candidate losses through the C ABI,
against the CPU oracle on the same seeded inputs.

Bars (the pages fix only "in bf16"):
* block output: relative Frobenius error <= 2^-8 against the oracle.  Both sides
  round every op output to bf16 (2^-9 relative at most) but from fp32 (GPU) and
  fp64 (oracle) values, so a small fraction of roundings land on the other
  neighbour (one ulp, 2^-8 relative) and later ops carry those flips along with
  gains of order one: the RMS difference stays within one ulp of the RMS output.
* losses: |gpu - oracle| <= 1e-2 oracle + 2 sqrt(oracle n) + n, where n is the
  mean square of the noise in the difference of two block outputs: twice the mean
  square difference between the GPU's and the oracle's reference outputs of the
  scored block (measured in the test with w4_block_forward).  The loss is the mean
  square of d = y_c - y_ref; each side's d carries its own rounding flips e, and
  mean((d + e)^2) - mean(d^2) = 2 mean(d e) + mean(e^2) is bounded by the last two
  terms; the 1e-2 covers the rest of the arithmetic (the measured disagreement of
  losses well above the noise is below 2e-3).
* choices: the GPU's first minimum over the candidates has an oracle loss within
  the two candidates' bars of the oracle's minimum.
"""
import numpy as np
import pytest
import torch

import weight_only_int4_amd as w4
from oracle import w4a16_oracle as O
from tests.gpu_util import bf16_values, bits16, gpu_available, rel_fro, say, to_bf16, to_f32
from workloads import block_input, round_to_bf16_bits, synthetic_block

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

BLOCK_TOL = 2.0 ** -8
LOSS_TOL = 1e-2


def _dev(blk):
    return {k: to_bf16(v) for k, v in blk.items()}


def _block_case(H, I, n_q, n_kv, B, L, seed):
    blk = synthetic_block(H, I, n_q, n_kv, seed)
    return blk, block_input(B * L, H, seed)


@pytest.mark.parametrize("H,I,n_q,n_kv,B,L", [(256, 384, 2, 1, 2, 70), (128, 256, 1, 1, 1, 1), (384, 128, 4, 2, 3, 33),
                                              (2048, 6144, 16, 8, 1, 64), (2048, 6144, 16, 8, 2, 130)])
def test_block_forward(H, I, n_q, n_kv, B, L):
    blk, x = _block_case(H, I, n_q, n_kv, B, L, 3)
    say("block forward", H, I, n_q, n_kv, B, L)
    Y = w4.block_forward(to_bf16(x), B, L, _dev(blk), n_q, n_kv)
    Y2 = w4.block_forward(to_bf16(x), B, L, _dev(blk), n_q, n_kv)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2), "block forward not deterministic"
    y = bf16_values(bits16(Y))
    ref = bf16_values(O.block_forward(x, B, L, blk, n_q, n_kv))
    err = rel_fro(y, ref)
    assert err <= BLOCK_TOL, err


def test_block_forward_zero_projections_is_identity():
    blk, x = _block_case(256, 384, 2, 1, 2, 40, 5)
    blk["o"] = np.zeros_like(blk["o"])
    blk["down"] = np.zeros_like(blk["down"])
    say("block identity")
    Y = w4.block_forward(to_bf16(x), 2, 40, _dev(blk), 2, 1)
    torch.cuda.synchronize()
    assert np.array_equal(bits16(Y), x)


def _noise(x, B, L, blk, nxt, n_q, n_kv):
    """Noise energies (d = 1, d = 0) of a difference of two block outputs: twice the
    mean square GPU - oracle difference of the reference outputs."""
    Yi = w4.block_forward(to_bf16(x), B, L, _dev(blk), n_q, n_kv)
    Yn = w4.block_forward(Yi, B, L, _dev(nxt), n_q, n_kv) if nxt is not None else Yi
    torch.cuda.synchronize()
    ri = O.block_forward(x, B, L, blk, n_q, n_kv)
    rn = O.block_forward(ri, B, L, nxt, n_q, n_kv) if nxt is not None else ri
    n0 = 2 * float(np.mean((bf16_values(bits16(Yi)) - bf16_values(ri)) ** 2))
    n1 = 2 * float(np.mean((bf16_values(bits16(Yn)) - bf16_values(rn)) ** 2))
    return n1, n0


def _losses_ok(g, o, n):
    bar = LOSS_TOL * o + 2 * np.sqrt(o * n) + n
    assert np.all(np.abs(g - o) <= bar), (g, o, bar)
    i, j = int(np.argmin(g)), int(np.argmin(o))
    assert o[i] <= o[j] + bar[i] + bar[j], (i, j, o)


@pytest.mark.parametrize("linear", list(O.LINEARS))
@pytest.mark.parametrize("sym", [False, True])
def test_lookahead_losses(linear, sym):
    H, I, n_q, n_kv, B, L = 256, 384, 2, 1, 2, 48
    blk, x = _block_case(H, I, n_q, n_kv, B, L, 7)
    nxt = synthetic_block(H, I, n_q, n_kv, 8)
    K = blk[linear].shape[1]
    rng = np.random.default_rng(11)
    S = np.stack([np.exp(rng.standard_normal(K) * a).astype(np.float32) for a in (0.0, 0.1, 0.3, 0.3)])
    r = np.array([1.0, 1.0, 0.9, 0.7], np.float32)
    say("lookahead", linear, sym)
    l1, l0 = w4.awq_lookahead_loss(to_bf16(x), B, L, _dev(blk), _dev(nxt), n_q, n_kv, linear, to_f32(S),
                                   to_f32(r), sym)
    torch.cuda.synchronize()
    o1, o0 = O.lookahead_losses(x, B, L, blk, nxt, n_q, n_kv, linear, S, r, sym)
    n1, n0 = _noise(x, B, L, blk, nxt, n_q, n_kv)
    _losses_ok(l1.cpu().numpy().astype(np.float64), o1, n1)
    _losses_ok(l0.cpu().numpy().astype(np.float64), o0, n0)


def test_lookahead_last_block_and_exact_grid():
    """Without a next block the d = 1 loss is the d = 0 loss; a candidate whose weights
    already lie on the int4 grid (s = 1, r = 1) scores near zero against a real one."""
    H, I, n_q, n_kv, B, L = 256, 384, 2, 1, 2, 40
    blk, x = _block_case(H, I, n_q, n_kv, B, L, 13)
    rng = np.random.default_rng(13)
    codes = rng.integers(0, 16, size=blk["up"].shape).astype(np.float32)
    codes[:, ::128], codes[:, 1::128] = 0.0, 15.0
    blk["up"] = round_to_bf16_bits((codes - 8.0) * np.float32(1 / 64))
    S = np.ones((2, H), np.float32)
    r = np.array([1.0, 0.6], np.float32)
    say("lookahead last block")
    l1, l0 = w4.awq_lookahead_loss(to_bf16(x), B, L, _dev(blk), None, n_q, n_kv, "up", to_f32(S), to_f32(r))
    torch.cuda.synchronize()
    g1, g0 = l1.cpu().numpy(), l0.cpu().numpy()
    assert np.array_equal(g1, g0)
    assert g1[0] <= 1e-3 * g1[1], g1
    o1, _ = O.lookahead_losses(x, B, L, blk, None, n_q, n_kv, "up", S, r)
    n1, _ = _noise(x, B, L, blk, None, n_q, n_kv)
    assert o1[0] == 0.0       # the GPU's int4 and bf16 products sum in different orders: near zero (above)
    _losses_ok(g1[1:].astype(np.float64), o1[1:], n1)


def test_lookahead_qwen_shape():
    """Hidden 2048, 16 query heads over 8 key/value heads, feed-forward 6144, two
    sequences of 40 tokens: three candidates for the o-projection and for down."""
    H, I, n_q, n_kv, B, L = 2048, 6144, 16, 8, 2, 40
    blk, x = _block_case(H, I, n_q, n_kv, B, L, 17)
    nxt = synthetic_block(H, I, n_q, n_kv, 18)
    for linear in ("o", "down"):
        K = blk[linear].shape[1]
        m = O.act_mean_abs(round_to_bf16_bits(np.random.default_rng(19).standard_normal((64, K)).astype(np.float32)))
        S = np.stack([O.awq_scales(m, a) for a in (0.0, 0.5, 0.5)])
        r = np.array([1.0, 1.0, 0.8], np.float32)
        say("lookahead qwen shape", linear)
        l1, l0 = w4.awq_lookahead_loss(to_bf16(x), B, L, _dev(blk), _dev(nxt), n_q, n_kv, linear, to_f32(S),
                                       to_f32(r))
        torch.cuda.synchronize()
        o1, o0 = O.lookahead_losses(x, B, L, blk, nxt, n_q, n_kv, linear, S, r)
        n1, n0 = _noise(x, B, L, blk, nxt, n_q, n_kv)
        _losses_ok(l1.cpu().numpy().astype(np.float64), o1, n1)
        _losses_ok(l0.cpu().numpy().astype(np.float64), o0, n0)


def test_search_lookahead_small():
    """Two-phase search of the gate projection scored after the next block: every alpha
    and ratio loss within its bar of the oracle's, the chosen alpha valid, and, when
    it is the oracle's, s(alpha*) within 1e-3 and the chosen ratio valid.  (The
    statistic is taken over the linear's input as each side computes it in its own
    reference pass, whose rare bf16 rounding flips move m by about 2^-8 / T.)"""
    H, I, n_q, n_kv, B, L = 256, 384, 2, 1, 2, 40
    blk, x = _block_case(H, I, n_q, n_kv, B, L, 21)
    nxt = synthetic_block(H, I, n_q, n_kv, 22)
    alphas, ratios = [0.0, 0.25, 0.5, 0.75], [1.0, 0.9, 0.8]
    say("search lookahead")
    res = w4.awq_search_lookahead(to_bf16(x), B, L, _dev(blk), _dev(nxt), n_q, n_kv, "gate", alphas, ratios)
    ref = O.search_lookahead(x, B, L, blk, nxt, n_q, n_kv, "gate", alphas, ratios)
    n1, _ = _noise(x, B, L, blk, nxt, n_q, n_kv)
    la, oa = np.array(res["alpha_losses"], np.float64), ref["alpha_losses"]
    _losses_ok(la, oa, n1)
    if res["alpha_index"] == ref["alpha_index"]:
        assert np.allclose(res["s"].cpu().numpy(), ref["s"], rtol=1e-3, atol=0)
        _losses_ok(np.array(res["ratio_losses"], np.float64), ref["ratio_losses"], n1)
