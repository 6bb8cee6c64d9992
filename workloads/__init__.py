"""Seeded synthetic inputs for the W4A16 group-128 workloads.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark. It draws random tensors and nothing else: it holds none of the
method's arithmetic (no quantization, no packing, no contraction, no loss).
The only numeric step besides the draws is rounding the fp32 draws to the bf16
storage type the workloads are defined in (round-to-nearest-even on the top 16
bits), which is input preparation, not part of the method.

Shapes and distributions follow the five workloads the method is measured on:

* ``gemv_2048``   -- one linear, M=1, K=N=2048, W ~ N(0, 0.02), X ~ N(0, 1), seed 0.
* ``decode_sweep`` -- the seven linears of a hidden-2048 decoder block
  (q 2048->2048, k/v 2048->1024, o 2048->2048, gate/up 2048->6144,
  down 6144->2048), repeated for 28 blocks; the layer shapes are those of the
  hidden-2048, 16-query-head / 8-kv-head (head_dim 128), FFN-6144 model card
  ("Model Architecture" section of the Qwen3-1.7B bundle page).
* ``prefill``     -- M=2048 tokens at (K,N) = (2048,6144) and (6144,2048);
  X ~ N(0,1) with round(0.01*K) seeded channels scaled x20 before rounding.
* ``large_sym``   -- (K,N) = (5120,17408) and (17408,5120), M in {1,8,64,512},
  W ~ N(0, 0.015); symmetric form.
* ``awq_search``  -- T=4096 calibration rows, K=2048, N=6144; per-channel
  magnitudes m_k = exp(N(0,1)) (LogNormal(0,1)), X[t,k] = m_k * N(0,1),
  W ~ N(0, 0.02).  These stand in for the calibration text of the pages
  (OpenR1-CMA rows, the Pile), which are not available.
* ``checkpoint``  -- a sharded bf16 checkpoint of a decoder-only model with
  hidden-2048 blocks (the seven linears above, two norm vectors per block),
  token embedding and output head, for the streaming data-free conversion:
  linears ~ N(0, 0.015), embedding / head ~ N(0, 0.02), norms ~ 1 + N(0, 0.05).

Every tensor has its own ``numpy.random.SeedSequence`` entropy
``[0, workload_id, block, tensor_id]`` so any one can be regenerated alone.
bf16 tensors are returned as ``uint16`` bit patterns.
"""
from __future__ import annotations

import numpy as np

# workload ids used in the seed entropy
GEMV_2048, DECODE_SWEEP, PREFILL, LARGE_SYM, AWQ_SEARCH, CHECKPOINT, LOOKAHEAD = 1, 2, 3, 4, 5, 6, 7

# (name, K, N) of one hidden-2048 decoder block, in execution order
BLOCK_LINEARS = (
    ("q", 2048, 2048),
    ("k", 2048, 1024),
    ("v", 2048, 1024),
    ("o", 2048, 2048),
    ("gate", 2048, 6144),
    ("up", 2048, 6144),
    ("down", 6144, 2048),
)
N_BLOCKS = 28
PREFILL_SHAPES = ((2048, 6144), (6144, 2048))       # (K, N)
PREFILL_M = 2048
LARGE_SHAPES = ((5120, 17408), (17408, 5120))       # (K, N)
LARGE_MS = (1, 8, 64, 512)
DECODE_MS = (1, 4, 16)
AWQ_T, AWQ_K, AWQ_N = 4096, 2048, 6144


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _rng(workload: int, block: int = 0, tensor: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([0, workload, block, tensor]))


def normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return round_to_bf16_bits(x)


def gemv_2048():
    """Single GEMV: returns (X[1][2048], W[2048][2048]) as bf16 bits, seed 0."""
    rng = np.random.default_rng(0)
    W = normal_bf16(rng, (2048, 2048), 0.02)
    X = normal_bf16(rng, (1, 2048), 1.0)
    return X, W


def decode_weight(block: int, layer: int) -> np.ndarray:
    """W[N][K] bf16 of linear ``layer`` (index into BLOCK_LINEARS) of ``block``."""
    _, K, N = BLOCK_LINEARS[layer]
    return normal_bf16(_rng(DECODE_SWEEP, block, layer), (N, K), 0.02)


def decode_act(block: int, layer: int, M: int) -> np.ndarray:
    """X[M][K] bf16 activations for linear ``layer`` of ``block`` at row count M."""
    _, K, _ = BLOCK_LINEARS[layer]
    return normal_bf16(_rng(DECODE_SWEEP, block, 100 + 16 * layer + M), (M, K), 1.0)


def prefill(shape_idx: int, M: int = PREFILL_M):
    """(X[M][K], W[N][K]) bf16 bits; round(0.01K) channels of X scaled by 20."""
    K, N = PREFILL_SHAPES[shape_idx]
    W = normal_bf16(_rng(PREFILL, shape_idx, 0), (N, K), 0.02)
    rng = _rng(PREFILL, shape_idx, 1)
    x = rng.standard_normal(size=(M, K), dtype=np.float32)
    n_out = int(round(0.01 * K))
    cols = rng.permutation(K)[:n_out]
    x[:, cols] *= np.float32(20.0)
    return round_to_bf16_bits(x), W


def prefill_outlier_channels(shape_idx: int) -> np.ndarray:
    """Indices of the x20 channels used by ``prefill(shape_idx)``."""
    K, _ = PREFILL_SHAPES[shape_idx]
    rng = _rng(PREFILL, shape_idx, 1)
    rng.standard_normal(size=(PREFILL_M, K), dtype=np.float32)
    return np.sort(rng.permutation(K)[: int(round(0.01 * K))])


def large_weight(shape_idx: int) -> np.ndarray:
    K, N = LARGE_SHAPES[shape_idx]
    return normal_bf16(_rng(LARGE_SYM, shape_idx, 0), (N, K), 0.015)


def large_act(shape_idx: int, M: int) -> np.ndarray:
    K, _ = LARGE_SHAPES[shape_idx]
    return normal_bf16(_rng(LARGE_SYM, shape_idx, 10 + M), (M, K), 1.0)


def awq_calibration(T: int = AWQ_T, K: int = AWQ_K, N: int = AWQ_N, seed_block: int = 0):
    """(X[T][K], W[N][K]) bf16 bits; per-channel magnitudes LogNormal(0, 1)."""
    rng = _rng(AWQ_SEARCH, seed_block, 0)
    mag = np.exp(rng.standard_normal(size=K)).astype(np.float32)
    x = rng.standard_normal(size=(T, K), dtype=np.float32) * mag[None, :]
    W = normal_bf16(_rng(AWQ_SEARCH, seed_block, 1), (N, K), 0.02)
    return round_to_bf16_bits(x), W


def small_case(M: int, K: int, N: int, seed: int, w_std: float = 0.02, x_std: float = 1.0):
    """Generic small (X[M][K], W[N][K]) bf16 pair for parity tests at odd sizes."""
    rng = np.random.default_rng(np.random.SeedSequence([0, 99, seed, M * 1000003 + K * 1009 + N]))
    W = normal_bf16(rng, (N, K), w_std)
    X = normal_bf16(rng, (M, K), x_std)
    return X, W


# ----------------------------------------------------------------------------- look-ahead block

# block shape of the base model: hidden 2048, 16 query / 8 key-value heads of 128, FFN 6144
QWEN_BLOCK = dict(H=2048, I=6144, n_q=16, n_kv=8)
LOOKAHEAD_B, LOOKAHEAD_L = 8, 512            # 4096 calibration tokens as 8 sequences of 512


def synthetic_block(H: int = 2048, I: int = 6144, n_q: int = 16, n_kv: int = 8, seed: int = 0,
                    w_std: float = 0.02) -> dict:
    """bf16 weights of one decoder block: norm1, norm2 ~ N(1, 0.1) [H]; q [128 n_q][H],
    k, v [128 n_kv][H], o [H][128 n_q], gate, up [I][H], down [H][I] ~ N(0, w_std)."""
    rng = np.random.default_rng(np.random.SeedSequence([0, LOOKAHEAD, seed, H, I, n_q, n_kv]))
    shapes = dict(q=(128 * n_q, H), k=(128 * n_kv, H), v=(128 * n_kv, H), o=(H, 128 * n_q),
                  gate=(I, H), up=(I, H), down=(H, I))
    blk = {"norm1": round_to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32)),
           "norm2": round_to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))}
    for name, shape in shapes.items():
        blk[name] = normal_bf16(rng, shape, w_std)
    return blk


def block_input(T: int, H: int = 2048, seed: int = 0) -> np.ndarray:
    """Hidden states entering a block: [T][H] bf16 ~ N(0, 1)."""
    return normal_bf16(np.random.default_rng(np.random.SeedSequence([0, LOOKAHEAD, 1000 + seed, T, H])), (T, H), 1.0)


# ----------------------------------------------------------------------------- sharded checkpoint

_CKPT_LINEARS = (("self_attn.q_proj", 0), ("self_attn.k_proj", 1), ("self_attn.v_proj", 2),
                 ("self_attn.o_proj", 3), ("mlp.gate_proj", 4), ("mlp.up_proj", 5), ("mlp.down_proj", 6))


def checkpoint_tensor_list(blocks: int, vocab: int = 8192, hidden: int = 2048):
    """(name, shape) of every tensor of the synthetic checkpoint, in storage order.
    Linear shapes are [N][K] (out x in); at hidden = 2048 they are BLOCK_LINEARS."""
    scale = hidden / 2048
    out = [("model.embed_tokens.weight", (vocab, hidden))]
    for b in range(blocks):
        out.append((f"model.layers.{b}.input_layernorm.weight", (hidden,)))
        for name, li in _CKPT_LINEARS:
            _, K, N = BLOCK_LINEARS[li]
            out.append((f"model.layers.{b}.{name}.weight", (int(N * scale), int(K * scale))))
        out.append((f"model.layers.{b}.post_attention_layernorm.weight", (hidden,)))
    out.append(("model.norm.weight", (hidden,)))
    out.append(("lm_head.weight", (vocab, hidden)))
    return out


def checkpoint_tensor(index: int, name: str, shape) -> np.ndarray:
    """bf16 bits of tensor ``index`` of checkpoint_tensor_list (seeded by its index)."""
    rng = _rng(CHECKPOINT, 0, index)
    if len(shape) == 1:
        return round_to_bf16_bits(1.0 + 0.05 * rng.standard_normal(size=shape, dtype=np.float32))
    std = 0.02 if ("embed" in name or "lm_head" in name) else 0.015
    return normal_bf16(rng, shape, std)


def write_checkpoint(directory: str, blocks: int, shards: int, vocab: int = 8192, hidden: int = 2048):
    """Write the synthetic checkpoint as ``shards`` safetensors files of about equal
    size (tensors in storage order, never split), named model-0000i-of-0000n.
    Returns the list of file paths."""
    import os
    import torch
    from safetensors.torch import save_file
    tensors = checkpoint_tensor_list(blocks, vocab, hidden)
    total = sum(int(np.prod(s)) * 2 for _, s in tensors)
    target = total / shards
    os.makedirs(directory, exist_ok=True)
    paths, cur, cur_bytes = [], {}, 0

    def flush():
        nonlocal cur, cur_bytes
        path = os.path.join(directory, f"model-{len(paths) + 1:05d}-of-{shards:05d}.safetensors")
        save_file(cur, path, metadata={"format": "pt"})
        paths.append(path)
        cur, cur_bytes = {}, 0

    for i, (name, shape) in enumerate(tensors):
        u16 = checkpoint_tensor(i, name, shape)
        cur[name] = torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16)
        cur_bytes += u16.nbytes
        if cur_bytes >= target and len(paths) < shards - 1:
            flush()
    if cur:
        flush()
    return paths
