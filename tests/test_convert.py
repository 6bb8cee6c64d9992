"""Streaming data-free symmetric conversion of a sharded checkpoint.

Host tests (CPU): which tensors are converted, the output names, the synthetic
checkpoint writer.  GPU test: a small two-shard checkpoint converted through the
library; every converted tensor bit-exact against the oracle's symmetric
quantize + pack (s = 1, no clip), every other tensor copied unchanged, one
tensor resident on the device at a time.
"""
import json
import os

import numpy as np
import pytest
import torch

import workloads as wl
from weight_only_int4_amd import convert as C


def test_selection_rule():
    assert C.is_converted("model.layers.3.self_attn.q_proj.weight", (2048, 2048))
    assert C.is_converted("model.layers.0.mlp.down_proj.weight", (2048, 6144))
    assert not C.is_converted("model.layers.0.input_layernorm.weight", (2048,))
    assert not C.is_converted("model.embed_tokens.weight", (8192, 2048))
    assert not C.is_converted("lm_head.weight", (8192, 2048))
    assert not C.is_converted("model.layers.0.mlp.down_proj.bias", (2048,))
    assert not C.is_converted("model.layers.0.odd.weight", (64, 100))          # K not a multiple of 128
    assert not C.is_converted("model.layers.1.self_attn.q_proj.weight", (2048, 2048),
                              ignore=[r"model\.layers\.1\..*"])
    assert C.converted_names("model.layers.0.mlp.up_proj.weight") == (
        "model.layers.0.mlp.up_proj.qweight", "model.layers.0.mlp.up_proj.scales")


def test_checkpoint_writer(tmp_path):
    from safetensors import safe_open
    paths = wl.write_checkpoint(str(tmp_path), blocks=2, shards=2, vocab=512, hidden=256)
    assert len(paths) == 2
    names = {}
    for p in paths:
        with safe_open(p, framework="pt") as f:
            for k in f.keys():
                names[k] = tuple(f.get_tensor(k).shape)
    want = dict(wl.checkpoint_tensor_list(2, 512, 256))
    assert names == want
    lin = [n for n, s in want.items() if C.is_converted(n, s)]
    assert len(lin) == 14


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")
def test_convert_small_checkpoint_bit_exact(tmp_path):
    from safetensors import safe_open
    from oracle import w4a16_oracle as O
    src, dst = tmp_path / "src", tmp_path / "dst"
    blocks, vocab, hidden = 2, 512, 256
    wl.write_checkpoint(str(src), blocks=blocks, shards=2, vocab=vocab, hidden=hidden)
    torch.cuda.reset_peak_memory_stats()
    stats = C.convert_checkpoint(str(src), str(dst))
    peak = torch.cuda.max_memory_allocated()
    tensors = wl.checkpoint_tensor_list(blocks, vocab, hidden)
    largest = max(int(np.prod(s)) * 2 for n, s in tensors if C.is_converted(n, s))
    assert peak <= 4 * largest, (peak, largest)
    assert stats["converted"] == 14 and stats["shards"] == 2
    out = {}
    for p in sorted(dst.glob("*.safetensors")):
        with safe_open(str(p), framework="pt") as f:
            assert json.loads(f.metadata()["w4a16"])["symmetric"] is True
            for k in f.keys():
                out[k] = f.get_tensor(k)
    cfg = json.loads((dst / "w4a16_config.json").read_text())
    for i, (name, shape) in enumerate(tensors):
        W = wl.checkpoint_tensor(i, name, shape)
        if C.is_converted(name, shape):
            assert name in cfg["converted"] and name not in out
            qn, sn = C.converted_names(name)
            oq, osc, _ = O.quantize_pack(W, None, 1.0, True)
            assert np.array_equal(out[qn].numpy().view(np.uint32), oq), name
            assert np.array_equal(out[sn].view(torch.int16).numpy().view(np.uint16), osc), name
        else:
            assert np.array_equal(out[name].view(torch.int16).numpy().view(np.uint16), W), name
