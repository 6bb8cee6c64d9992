"""Plant plausible mistakes in a copy of the CPU oracle and require that at
least one pin in ``tests/oracle_pins.py`` catches each of them.

Each mutant is a source substitution applied to the oracle's text, executed as
a fresh module on the CPU; the real oracle module's functions are then swapped
for the mutant's while the pins run.  Nothing here touches a GPU.
"""
import importlib.util
import inspect
import types

import pytest

from oracle import w4a16_oracle as O
from tests import oracle_pins as P

MUTANTS = {
    "rint_half_up": ("q = np.clip(np.rint(v / sc) + z, 0, ASYM_LEVELS)",
                     "q = np.clip(np.floor(v / sc + np.float32(0.5)) + z, 0, ASYM_LEVELS)"),
    "reciprocal_multiply": ("q = np.clip(np.rint(v / sc) + z, 0, ASYM_LEVELS)",
                            "q = np.clip(np.rint(v * (np.float32(1.0) / sc)) + z, 0, ASYM_LEVELS)"),
    "zero_sign": ("z = np.clip(np.rint(-lo / sc), 0, ASYM_LEVELS)",
                  "z = np.clip(np.rint(lo / sc), 0, ASYM_LEVELS)"),
    "zero_unclamped": ("z = np.clip(np.rint(-lo / sc), 0, ASYM_LEVELS)", "z = np.rint(-lo / sc)"),
    "asym_levels_16": ("np.maximum(hi - lo, RANGE_FLOOR) / np.float32(ASYM_LEVELS)",
                       "np.maximum(hi - lo, RANGE_FLOOR) / np.float32(16.0)"),
    "sym_divisor_8": ("np.maximum(absmax, RANGE_FLOOR) / np.float32(SYM_MAX)",
                      "np.maximum(absmax, RANGE_FLOOR) / np.float32(8.0)"),
    "sym_no_offset": ("q = np.clip(np.rint(v / sc), -SYM_OFFSET, SYM_MAX) + SYM_OFFSET",
                      "q = np.clip(np.rint(v / sc), -SYM_OFFSET, SYM_MAX) % 16"),
    "scale_not_rounded": ("        sc = bf16_to_f32(sc_bits)\n        z = np.clip",
                          "        sc = np.maximum(hi - lo, RANGE_FLOOR) / np.float32(ASYM_LEVELS)\n        z = np.clip"),
    "clip_scales_instead_of_clamps": ("v = np.minimum(np.maximum(v, -t), t)", "v = v * r"),
    "s_on_rows": ("v = v * np.asarray(s, dtype=np.float32)[None, :]",
                  "v = v * np.asarray(s, dtype=np.float32)[:v.shape[0], None]"),
    "nibbles_reversed": ("out |= padded[..., j] << np.uint32(4 * j)",
                         "out |= padded[..., j] << np.uint32(4 * (7 - j))"),
    "dequant_plus_zero": ("return ((codes.reshape(N, G, GROUP) - z) * sc).reshape(N, K)",
                          "return ((codes.reshape(N, G, GROUP) + z - 2 * np.float32(SYM_OFFSET)) * sc).reshape(N, K)"),
    "linear_transposed_weight": ("@ np.asarray(W_hat, dtype=np.float64).T",
                                 "@ np.asarray(W_hat, dtype=np.float64).T[::-1]"),
    "loss_multiplies_s": ("W_eff = W_hat / np.asarray(s", "W_eff = W_hat * np.asarray(s"),
    "reference_unrounded": ("return bf16_to_f32(f32_to_bf16(y.astype(np.float32))).astype(np.float64)",
                            "return y"),
    "stat_without_abs": ("return np.abs(bf16_to_f32(X_bf16).astype(np.float64)).mean(axis=0)",
                         "return bf16_to_f32(X_bf16).astype(np.float64).mean(axis=0)"),
    "scales_unnormalised": ("return (p / np.sqrt(p.max() * p.min())).astype(np.float32)",
                            "return p.astype(np.float32)"),
    "alpha_linspace": ("return np.arange(n, dtype=np.float64) / n", "return np.linspace(0.0, 1.0, n)"),
    "bf16_truncates": ("return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)",
                       "return (u >> np.uint64(16)).astype(np.uint16)"),
    "bf16_ties_away": ("return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)",
                       "return ((u + np.uint64(0x8000)) >> np.uint64(16)).astype(np.uint16)"),
    "w4a8_scale_128": ("amax / np.float32(INT8_MAX)", "amax / np.float32(128.0)"),
    "w4a8_floor": ("q = np.rint(x / sx[:, None])", "q = np.floor(x / sx[:, None])"),
    "w4a8_half_up": ("q = np.rint(x / sx[:, None])", "q = np.floor(x / sx[:, None] + np.float32(0.5))"),
    "w4a8_zero_ignored": ("d = codes.reshape(N, G, GROUP) - z[:, :, None]", "d = codes.reshape(N, G, GROUP) - 8"),
    "w4a8_no_act_scale": ("return y * np.asarray(sx, dtype=np.float64)[:, None]", "return y"),
    "w4a8_group_sum_shifted": ("xsum = xq.astype(np.int64).reshape(M, K // GROUP, GROUP).sum(axis=2)",
                               "xsum = np.roll(xq.astype(np.int64), 1, axis=1).reshape(M, K // GROUP, GROUP).sum(axis=2)"),
    "clip_loss_x_times_s": ("bf16_to_f32(f32_to_bf16(bf16_to_f32(X_bf16) / s32[None, :]))",
                            "bf16_to_f32(f32_to_bf16(bf16_to_f32(X_bf16) * s32[None, :]))"),
    "clip_loss_v_unscaled": ("v = (bf16_to_f32(W_bf16) * s32[None, :])", "v = (bf16_to_f32(W_bf16) * 1)"),
    "clip_loss_abs": ("L[g, :, ir] = (P * P).sum(axis=0)", "L[g, :, ir] = np.abs(P).sum(axis=0)"),
    "clip_loss_half_group": ("sl = slice(GROUP * g, GROUP * (g + 1))", "sl = slice(GROUP * g, GROUP * g + 64)"),
    "clip_loss_x_transposed_tokens": ("P = xs[:, sl] @ e[:, sl].T", "P = xs[::-1, sl][:, ::-1] @ e[:, sl].T"),
    "clip_best_last": ("best = np.argmin(L, axis=2).T", "best = (L.shape[2] - 1 - np.argmin(L[:, :, ::-1], axis=2)).T"),
    "clip_best_max": ("best = np.argmin(L, axis=2).T", "best = np.argmax(L, axis=2).T"),
    "rope_sign": ("out = np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)",
                  "out = np.concatenate([x1 * c + x2 * s, x2 * c + x1 * s], axis=-1)"),
    "rope_adjacent_pairs": ("x1, x2 = xr[..., :64], xr[..., 64:]", "x1, x2 = xr[..., 0::2], xr[..., 1::2]"),
    "rope_frequency": ("inv = base ** (-(2.0 * np.arange(HEAD_DIM // 2)) / HEAD_DIM)",
                       "inv = base ** (-(1.0 * np.arange(HEAD_DIM // 2)) / HEAD_DIM)"),
    "attention_sees_next_token": ("mask = np.triu(np.ones((L, L), dtype=bool), 1)",
                                  "mask = np.triu(np.ones((L, L), dtype=bool), 2)"),
    "attention_gqa_interleaved": ("            kv = h // rep\n            sc = qh", "            kv = h % n_kv\n            sc = qh"),
    "attention_scale": ("sc = qh[b, :, h, :] @ kh[b, :, kv, :].T / np.sqrt(HEAD_DIM)",
                        "sc = qh[b, :, h, :] @ kh[b, :, kv, :].T / HEAD_DIM"),
    "rmsnorm_mean_abs": ("r = 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps)", "r = 1.0 / np.sqrt(np.mean(np.abs(x), axis=1) + eps)"),
    "silu_is_sigmoid": ("return _bf16_round(g / (1.0 + np.exp(-g)) * u)", "return _bf16_round(1.0 / (1.0 + np.exp(-g)) * u)"),
    "block_no_attention_residual": ('h = _bf16_round(x + lin("o", o))', 'h = _bf16_round(lin("o", o))'),
    "candidate_input_times_s": ("xs = bf16_to_f32(f32_to_bf16(a.astype(np.float32) / s32[None, :])).astype(np.float64)",
                                "xs = bf16_to_f32(f32_to_bf16(a.astype(np.float32) * s32[None, :])).astype(np.float64)"),
    "lookahead_next_on_input": ("yn = block_forward(yi, B, L, nxt, n_q, n_kv) if nxt is not None else yi",
                                "yn = block_forward(x_bf16, B, L, nxt, n_q, n_kv) if nxt is not None else yi"),
    "clip_after_scale_choice": ("        absmax = np.abs(v).max(axis=2, keepdims=True)\n    if symmetric:",
                                "    if symmetric:"),
    "gate_up_swapped": ('m = silu_mul(lin("gate", b2), lin("up", b2))', 'm = silu_mul(lin("up", b2), lin("gate", b2))'),
    "norm2_on_input": ('b2 = rmsnorm(h, val(blk["norm2"]))', 'b2 = rmsnorm(x, val(blk["norm2"]))'),
    "norm2_weight_is_norm1": ('b2 = rmsnorm(h, val(blk["norm2"]))', 'b2 = rmsnorm(h, val(blk["norm1"]))'),
    "rms_eps_1e-5": ("RMS_EPS = 1e-6", "RMS_EPS = 1e-5"),
    "rms_eps_zero": ("RMS_EPS = 1e-6", "RMS_EPS = 0.0"),
    "rope_on_values": ('v = lin("v", a)', 'v = rope(lin("v", a), B, L, n_kv)'),
    "rope_missing_on_keys": ('k = rope(lin("k", a), B, L, n_kv)', 'k = lin("k", a)'),
    "final_residual_from_input": ('y = _bf16_round(h + lin("down", m))', 'y = _bf16_round(x + lin("down", m))'),
    "queries_from_block_input": ('q = rope(lin("q", a), B, L, n_q)', 'q = rope(lin("q", x), B, L, n_q)'),
    "candidate_unrounded_input": ("xs = bf16_to_f32(f32_to_bf16(a.astype(np.float32) / s32[None, :])).astype(np.float64)",
                                  "xs = a / s32[None, :].astype(np.float64)"),
}


def _mutant_module(old, new):
    src = inspect.getsource(O)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["__name__"] = "oracle_mutant"
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    old, new = MUTANTS[name]
    mod = _mutant_module(old, new)
    for attr, val in vars(mod).items():
        if callable(val) and getattr(val, "__module__", None) == "oracle_mutant":
            monkeypatch.setattr(O, attr, val)
    caught = []
    for check in P.ALL_CHECKS:
        try:
            check()
        except Exception as e:          # AssertionError or a shape error: the mistake is visible
            caught.append((check.__name__, type(e).__name__))
            break
    assert caught, f"mutant {name} passed every pin"
