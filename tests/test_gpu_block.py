"""Decoder block forward and look-ahead (d = 1) candidate losses through the C ABI,
against the CPU oracle on the same seeded inputs.

Bars (the pages fix only "in bf16"):
* block output: relative Frobenius error <= 2^-8 against the oracle.  Both sides
  round every op output to bf16 (2^-9 relative at most) but from fp32 (GPU) and
  fp64 (oracle) values, so a small fraction of roundings land on the other
  neighbour (one ulp, 2^-8 relative) and later ops carry those flips along with
  gains of order one: the RMS difference stays within one ulp of the RMS output.
  The same bar holds for a block with one linear in its deployed int4 form
  (w4_block_forward_quantized), which is how a candidate is scored.  Outputs
  after two chained blocks (the look-ahead depth d = 1) carry both blocks'
  flips, the first block's amplified by the second block's gain on input
  perturbations: bar 2^-7 (measured on the hidden-2048 shape: one block
  1.8e-3, two blocks 4.4e-3, i.e. a gain of about 2).
* losses.  A candidate's loss is L = mean((y_c - y_r)^2) over the scored block's
  outputs (candidate path c, reference path r).  The test computes both sides'
  outputs (GPU: w4_block_forward_quantized / w4_block_forward; oracle:
  block_forward) and requires
  - the GPU's loss to be the mean square difference of the GPU's own outputs
    (relative 1e-6: its fp64 sum, stored fp32), and
  - |sqrt(L_gpu) - sqrt(L_oracle)| <= delta = sqrt(mean((e_c - e_r)^2)), with
    e_c, e_r the GPU - oracle differences of the candidate and the reference
    outputs (Minkowski's inequality for the root mean square).  delta is the
    whole of the disagreement the bf16 rounding flips of the two sides can cause,
    including the GPU's own candidate path (int4 GEMM) against its reference path
    (bf16 GEMM), whose fp32 sums run in different orders: a candidate already on
    the int4 grid has oracle loss 0 and a GPU loss of at most delta^2.
  The candidate outputs themselves are held to the block bars above.
* choices: the GPU's first minimum i over the candidates satisfies
  sqrt(L_oracle[i]) <= sqrt(L_oracle[j]) + delta_i + delta_j for the oracle's
  first minimum j.
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

BLOCK_TOL = 2.0 ** -8    # one block
CHAIN_TOL = 2.0 ** -7    # two chained blocks (the d = 1 output)
OWN_TOL = 1e-6          # GPU loss against the mean square of its own outputs (fp64 sum, fp32 store)
STAT_TOL = 1e-2         # search losses at the GPU's statistic against losses at the oracle's


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


def _on_grid(W, rng):
    """Weights of W's shape on the asymmetric int4 grid: codes 0..15 with 0 and 15 in
    every group, scale 1/64, zero 8 -- quantize + dequantize returns them exactly."""
    codes = rng.integers(0, 16, size=W.shape).astype(np.float32)
    codes[:, ::128], codes[:, 1::128] = 0.0, 15.0
    return round_to_bf16_bits((codes - 8.0) * np.float32(1 / 64))


class _Paths:
    """Both sides' reference outputs of a block (and of the next one) and, per
    candidate, both sides' candidate outputs; the loss checks of the module docstring."""

    def __init__(self, x, B, L, blk, nxt, n_q, n_kv, linear, sym):
        self.x, self.B, self.L, self.blk, self.nxt, self.n_q, self.n_kv = x, B, L, blk, nxt, n_q, n_kv
        self.linear, self.sym = linear, sym
        self.blk_d = _dev(blk)
        self.nxt_d = None if nxt is None else _dev(nxt)
        ri = w4.block_forward(to_bf16(x), B, L, self.blk_d, n_q, n_kv)
        rn = ri if nxt is None else w4.block_forward(ri, B, L, self.nxt_d, n_q, n_kv)
        torch.cuda.synchronize()
        self.r_gpu = (bf16_values(bits16(rn)), bf16_values(bits16(ri)))
        oi = O.block_forward(x, B, L, blk, n_q, n_kv)
        on = oi if nxt is None else O.block_forward(oi, B, L, nxt, n_q, n_kv)
        self.r_or = (bf16_values(on), bf16_values(oi))

    def candidate(self, s, r):
        """(d = 1, d = 0) outputs of one candidate, GPU and oracle, as values."""
        s = np.asarray(s, np.float32)
        r32 = float(np.float32(r))
        qw, sc, qz = w4.awq_quantize_pack(self.blk_d[self.linear], to_f32(s), r32, self.sym)
        ci = w4.block_forward_quantized(to_bf16(self.x), self.B, self.L, self.blk_d, self.n_q, self.n_kv,
                                        self.linear, to_f32(s), qw, sc, qz, self.sym)
        cn = ci if self.nxt is None else w4.block_forward(ci, self.B, self.L, self.nxt_d, self.n_q, self.n_kv)
        torch.cuda.synchronize()
        packed = O.quantize_pack(self.blk[self.linear], s, r32, self.sym)
        oi = O.block_forward(self.x, self.B, self.L, self.blk, self.n_q, self.n_kv,
                             candidate=(self.linear, s, packed, self.sym))
        on = oi if self.nxt is None else O.block_forward(oi, self.B, self.L, self.nxt, self.n_q, self.n_kv)
        return (bf16_values(bits16(cn)), bf16_values(bits16(ci))), (bf16_values(on), bf16_values(oi))

    def check(self, S, ratios, l_gpu, depth=0, l_oracle=None):
        """Checks the GPU losses l_gpu [C] at depth 0 (d = 1) or 1 (d = 0) of
        candidates (S[c], ratios[c]); l_oracle (optional) is the oracle's
        lookahead_losses at that depth, which must equal the mean square of the
        oracle outputs computed here.  Returns (oracle losses, deltas)."""
        l_gpu = np.asarray(l_gpu, np.float64)
        lo, dl = [], []
        for c in range(len(ratios)):
            cg, co = self.candidate(S[c], ratios[c])
            yg, yo, rg, ro = cg[depth], co[depth], self.r_gpu[depth], self.r_or[depth]
            own = float(np.mean((yg - rg) ** 2))
            L_o = float(np.mean((yo - ro) ** 2))
            delta = float(np.sqrt(np.mean(((yg - yo) - (rg - ro)) ** 2)))
            say("  candidate", c, "depth", depth, "gpu", l_gpu[c], "oracle", L_o, "delta^2", delta ** 2,
                "rel_fro cand", rel_fro(yg, yo), "ref", rel_fro(rg, ro))
            assert abs(l_gpu[c] - own) <= OWN_TOL * own + 1e-30, (c, l_gpu[c], own)
            assert abs(np.sqrt(l_gpu[c]) - np.sqrt(L_o)) <= delta * (1 + OWN_TOL) + 1e-30, (c, l_gpu[c], L_o, delta)
            bar = BLOCK_TOL if depth == 1 or self.nxt is None else CHAIN_TOL
            assert rel_fro(yg, yo) <= bar, (c, depth, rel_fro(yg, yo))
            if l_oracle is not None:
                assert abs(l_oracle[c] - L_o) <= 1e-12 * L_o + 1e-300, (c, l_oracle[c], L_o)
            lo.append(L_o)
            dl.append(delta)
        lo, dl = np.array(lo), np.array(dl)
        i, j = int(np.argmin(l_gpu)), int(np.argmin(lo))
        assert np.sqrt(lo[i]) <= np.sqrt(lo[j]) + dl[i] + dl[j] + 1e-30, (i, j, lo, dl)
        return lo, dl


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
    p = _Paths(x, B, L, blk, nxt, n_q, n_kv, linear, sym)
    p.check(S, r, l1.cpu().numpy(), 0, o1)
    p.check(S, r, l0.cpu().numpy(), 1, o0)


def test_lookahead_last_block_and_exact_grid():
    """Without a next block the d = 1 loss is the d = 0 loss; a candidate whose weights
    already lie on the int4 grid (s = 1, r = 1) has oracle loss 0 and meets the same
    bar as every other candidate (its GPU loss at most delta^2)."""
    H, I, n_q, n_kv, B, L = 256, 384, 2, 1, 2, 40
    blk, x = _block_case(H, I, n_q, n_kv, B, L, 13)
    blk["up"] = _on_grid(blk["up"], np.random.default_rng(13))
    S = np.ones((2, H), np.float32)
    r = np.array([1.0, 0.6], np.float32)
    say("lookahead last block")
    l1, l0 = w4.awq_lookahead_loss(to_bf16(x), B, L, _dev(blk), None, n_q, n_kv, "up", to_f32(S), to_f32(r))
    torch.cuda.synchronize()
    g1, g0 = l1.cpu().numpy(), l0.cpu().numpy()
    assert np.array_equal(g1, g0)
    o1, _ = O.lookahead_losses(x, B, L, blk, None, n_q, n_kv, "up", S, r)
    assert o1[0] == 0.0
    p = _Paths(x, B, L, blk, None, n_q, n_kv, "up", False)
    p.check(S, r, g1, 0, o1)


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
        p = _Paths(x, B, L, blk, nxt, n_q, n_kv, linear, False)
        p.check(S, r, l1.cpu().numpy(), 0, o1)
        p.check(S, r, l0.cpu().numpy(), 1, o0)


def test_search_lookahead_small():
    """Two-phase search of the gate projection scored after the next block.  Each side
    takes the statistic over the linear's input in its own reference pass (rare bf16
    rounding flips move m by about 2^-8 / T), so the GPU search scores s(alpha) from
    its statistic.  Checks: s(alpha*) within 1e-3 of the oracle's s at that alpha;
    the GPU's losses at the oracle's s (awq_lookahead_loss) against the oracle by
    the bar above; the search's losses within 1e-2 of those (the statistic
    difference); the chosen alpha valid by the choice rule.  Phase 2 runs at the
    GPU's own s(alpha*), which the test passes to both sides: its losses meet the
    bar above exactly, whether or not alpha* is the oracle's."""
    H, I, n_q, n_kv, B, L = 256, 384, 2, 1, 2, 40
    blk, x = _block_case(H, I, n_q, n_kv, B, L, 21)
    nxt = synthetic_block(H, I, n_q, n_kv, 22)
    alphas, ratios = [0.0, 0.25, 0.5, 0.75], [1.0, 0.9, 0.8]
    say("search lookahead")
    res = w4.awq_search_lookahead(to_bf16(x), B, L, _dev(blk), _dev(nxt), n_q, n_kv, "gate", alphas, ratios)
    ref = O.search_lookahead(x, B, L, blk, nxt, n_q, n_kv, "gate", alphas, ratios)
    ins = {}
    O.block_forward(x, B, L, blk, n_q, n_kv, inputs=ins)
    m = np.abs(ins["gate"]).mean(axis=0)
    S_or = np.stack([O.awq_scales(m, a) for a in alphas])
    ia = res["alpha_index"]
    s_gpu = res["s"].cpu().numpy()
    assert np.allclose(s_gpu, S_or[ia], rtol=1e-3, atol=0)
    p = _Paths(x, B, L, blk, nxt, n_q, n_kv, "gate", False)
    ones = np.ones(len(alphas), np.float32)
    la_at_or, _ = w4.awq_lookahead_loss(to_bf16(x), B, L, _dev(blk), _dev(nxt), n_q, n_kv, "gate", to_f32(S_or),
                                        to_f32(ones), want_d0=False)
    la_at_or = la_at_or.cpu().numpy().astype(np.float64)
    lo, dl = p.check(S_or, ones, la_at_or, 0, ref["alpha_losses"])
    la = np.array(res["alpha_losses"], np.float64)
    assert np.all(np.abs(la - la_at_or) <= STAT_TOL * la_at_or), (la, la_at_or)
    j = int(np.argmin(lo))
    assert np.sqrt(lo[ia]) <= np.sqrt(lo[j]) * np.sqrt(1 + STAT_TOL) ** 2 + dl[ia] + dl[j], (ia, j, lo, dl)
    S2 = np.broadcast_to(s_gpu, (len(ratios), s_gpu.size))
    p.check(S2, np.array(ratios, np.float32), np.array(res["ratio_losses"], np.float64), 0)
