"""Streaming data-free symmetric W4A16 conversion of a sharded safetensors checkpoint.

Model card "Qwen3.6-27B-W4A16", opening paragraphs and the build notes: the
linears are converted from bf16 to int4 with group size 128, symmetric
(scale = absmax / 7), weight-only, with no calibration data and without building
the model -- the converter reads tensors straight from the safetensors files and
keeps one source shard at a time, so peak GPU memory stays at the size of the
largest tensor being converted.

Every quantization runs in the library's ``awq_quantize_pack`` kernel (s = 1,
no clipping, symmetric); this module only moves tensors between files, host and
device.  A tensor is converted when it is a 2-D ``*.weight`` inside a decoder
block (its name contains ``.layers.``), its input dimension is a multiple of 128
and no ``ignore`` pattern matches its name; everything else (norms, embeddings,
the output head) is copied unchanged.  Converted ``<prefix>.weight`` [N][K] bf16
becomes ``<prefix>.qweight`` int32 [N][K/8] (nibble j of word i holds the code of
input channel 8 i + j, stored as q + 8) and ``<prefix>.scales`` bf16 [N][K/128].
Output shards keep the source shard names; each carries the conversion settings
in its metadata, and ``w4a16_config.json`` lists the converted tensors.

    python -m weight_only_int4_amd.convert SRC_DIR DST_DIR [--ignore REGEX ...]
"""
from __future__ import annotations

import argparse
import glob
import json
import os
import re
import sys
import time

import torch

from . import GROUP_SIZE, awq_quantize_pack

FORMAT = {
    "bits": 4,
    "group_size": GROUP_SIZE,
    "symmetric": True,
    "scale": "bf16(max(absmax, 1e-5) / 7) per 128-group",
    "qweight": "int32 [N][K/8]; nibble j of word i = code of input channel 8 i + j, stored as q + 8",
    "scales": "bf16 [N][K/128]",
}


def is_converted(name: str, shape, ignore=()) -> bool:
    """Whether the tensor ``name`` of ``shape`` is a decoder-block linear weight to convert."""
    if len(shape) != 2 or not name.endswith(".weight") or ".layers." not in name:
        return False
    if shape[1] % GROUP_SIZE != 0 or shape[0] == 0:
        return False
    return not any(re.fullmatch(p, name) for p in ignore)


def converted_names(name: str):
    prefix = name[: -len(".weight")]
    return prefix + ".qweight", prefix + ".scales"


class _Staging:
    """Reusable pinned host buffer for host -> device copies."""

    def __init__(self):
        self.buf = None

    def to_device(self, t: torch.Tensor, device) -> torch.Tensor:
        n = t.numel()
        if self.buf is None or self.buf.numel() < n:
            self.buf = torch.empty(max(n, 1 << 20), dtype=t.dtype, pin_memory=True)
        view = self.buf[:n].view(t.shape)
        view.copy_(t)
        return view.to(device, non_blocking=True)


def convert_checkpoint(src_dir: str, dst_dir: str, ignore=(), device="cuda", log=None) -> dict:
    """Convert every shard of ``src_dir`` into ``dst_dir``, one shard at a time.

    Returns statistics: shards, converted tensor count, bf16 bytes converted,
    bytes written, wall seconds, and the seconds spent in the quantization kernel
    (event-timed on the device)."""
    from safetensors import safe_open
    from safetensors.torch import save_file

    shards = sorted(glob.glob(os.path.join(src_dir, "*.safetensors")))
    if not shards:
        raise FileNotFoundError(f"no .safetensors files in {src_dir}")
    os.makedirs(dst_dir, exist_ok=True)
    dev = torch.device(device)
    staging = _Staging()
    stats = {"shards": len(shards), "converted": 0, "bytes_converted": 0, "bytes_copied": 0, "bytes_written": 0,
             "kernel_s": 0.0}
    converted = {}
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    for shard in shards:
        out = {}
        with safe_open(shard, framework="pt", device="cpu") as f:
            for name in f.keys():
                t = f.get_tensor(name)
                if t.dtype == torch.bfloat16 and is_converted(name, t.shape, ignore):
                    W = staging.to_device(t, dev)
                    start.record()
                    qw, sc, _ = awq_quantize_pack(W, symmetric=True)
                    stop.record()
                    qn, sn = converted_names(name)
                    out[qn] = qw.to("cpu")
                    out[sn] = sc.to("cpu")
                    stop.synchronize()
                    stats["kernel_s"] += start.elapsed_time(stop) * 1e-3
                    stats["converted"] += 1
                    stats["bytes_converted"] += t.numel() * 2
                    converted[name] = os.path.basename(shard)
                    del W, qw, sc
                else:
                    out[name] = t
                    stats["bytes_copied"] += t.numel() * t.element_size()
        dst = os.path.join(dst_dir, os.path.basename(shard))
        save_file(out, dst, metadata={"format": "pt", "w4a16": json.dumps(FORMAT)})
        stats["bytes_written"] += os.path.getsize(dst)
        del out
        if log:
            log(f"converted {os.path.basename(shard)}")
    with open(os.path.join(dst_dir, "w4a16_config.json"), "w") as fh:
        json.dump({"format": FORMAT, "converted": converted}, fh, indent=1, sort_keys=True)
    stats["wall_s"] = time.perf_counter() - t0
    return stats


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("src")
    ap.add_argument("dst")
    ap.add_argument("--ignore", action="append", default=[], help="regex (full match) of tensor names to keep")
    ap.add_argument("--device", default="cuda")
    args = ap.parse_args(argv)
    stats = convert_checkpoint(args.src, args.dst, args.ignore, args.device,
                               log=lambda m: print(m, file=sys.stderr, flush=True))
    print(json.dumps(stats))
    return 0


if __name__ == "__main__":
    sys.exit(main())
