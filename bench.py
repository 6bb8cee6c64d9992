"""Benchmark of the W4A16 group-128 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--step-only]

One step is one decode sweep: the seven linears of a hidden-2048 decoder block
(q 2048->2048, k/v 2048->1024, o 2048->2048, gate/up 2048->6144, down
6144->2048) for 28 blocks, M = 1 bf16 activation row, asymmetric int4 group-128
weights resident in HBM (734 MB of packed weights per sweep, more than the
256 MB Infinity Cache, so every step streams them from HBM).  The linears that
read the same activation row run as one GEMV (q|k|v, o, gate|up, down), as a
decoder runs them: the step is replayed as one HIP graph of 112 GEMV launches.

``value`` is the sweep's algorithmic bytes (packed weights + bf16 scales +
packed zeros + X + Y) divided by the wall time per step (TB/s).  The same JSON
line carries:
  * ``roofline`` of the dominant kernel (the GEMV): algorithmic bytes per launch
    over its average launch duration -- the event-timed graph replay (only GEMV
    launches, back to back on one stream) divided by the launches -- against
    the 8 TB/s HBM peak, with the latency floor: t0, the per-launch time of an
    empty kernel replayed as a graph of as many launches, and the step's
    latency-adjusted ceiling
    sum(bytes / BW) / sum(t0 + bytes / BW), which no kernel of the sweep can beat,
    and the plain-read yardstick: the best of 40 settings of a streaming-read probe
    replayed as a graph with the step's launch sizes and order, over the same bytes;
  * ``rows``: every other step of the path measured in the same run (cold-cache
    GEMV on the 27B-shaped linears, decode sweeps at M = 4 and 16, prefill GEMM
    at M = 2048 and the 27B shapes, quantize + pack, the full 30-candidate AWQ
    search), each with its own roofline fraction;
  * ``cpu_baseline``: the CPU oracle on a bounded sample of the same sweep.
All inputs are seeded synthetic tensors (``workloads``).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
GROUP = 128


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- helpers

def packed_bytes(N, K, symmetric):
    G = K // GROUP
    b = N * K // 2 + N * G * 2
    if not symmetric:
        b += N * ((G + 7) // 8) * 4
    return b


def gemv_bytes(M, K, N, symmetric):
    return packed_bytes(N, K, symmetric) + M * K * 2 + M * N * 2


def to_dev_bf16(torch, u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


class Launch:
    """One prepared GEMV/GEMM launch (operands preallocated, arguments validated once)."""

    def __init__(self, launcher, nbytes, flops):
        self.launcher, self.nbytes, self.flops = launcher, nbytes, flops

    def __call__(self):
        self.launcher()


def latency_floor_us(torch, w4, launches):
    """Per-launch time (us) of a graph of `launches` launches of an empty kernel
    (one 64-thread workgroup; a kernel of its own, so that profiles of the GEMV
    keep only real GEMV dispatches)."""
    ls = [Launch(lambda: w4.probe_empty(), 0, 0) for _ in range(launches)]
    g = capture_graph(torch, ls)
    ms = time_events(torch, g.replay, 20)
    del g, ls
    return ms * 1e3 / launches


def latency_ceiling(t0_us, nbytes):
    """Fraction of the HBM peak that a launch moving nbytes reaches at best when
    every launch also costs t0."""
    ideal_us = nbytes / (HBM_PEAK_GBS * 1e3)
    return ideal_us / (t0_us + ideal_us)


_SPACER = {}


def spacer(torch, ms=20.0):
    """Queue ~ms of GPU busy time so that every launch and event recorded after it
    is already enqueued when the GPU reaches it (the host never sits inside a
    timed interval).  torch.cuda._sleep spins a fixed number of cycles."""
    if "cycles_per_ms" not in _SPACER:
        torch.cuda._sleep(1000)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(2_000_000)
        b.record()
        b.synchronize()
        _SPACER["cycles_per_ms"] = 2_000_000 / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(_SPACER["cycles_per_ms"] * ms))


def time_events(torch, fn, iters):
    """Average ms per call of fn over iters calls bracketed by one pair of events."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    spacer(torch)
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / iters


def profiled_traffic():
    """HBM bytes per GEMV launch of the decode sweep as measured by rocprofv3 (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain-copy calibration) in profiles/gemv_decode_sweep_M1.md, or
    None when the GEMV sources have changed since that profile was taken."""
    try:
        text = open(os.path.join(ROOT, "profiles", "gemv_decode_sweep_M1.md")).read()
        vals = dict(re.findall(r"^(\w+): (\S+)$", text, flags=re.M))
        h = hashlib.sha256()
        for f in ("gemv.hip", "gemv_mfma.hip", "common.hpp"):
            with open(os.path.join(ROOT, "weight_only_int4_amd", "csrc", f), "rb") as fh:
                h.update(fh.read())
        if vals.get("gemv_source_sha256_16") != h.hexdigest()[:16]:
            return None
        return int(vals["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------- workloads

def pack_sweep(torch, w4, wl, blocks):
    """Packed asymmetric weights of every linear of the sweep, in block order."""
    packed = []
    for b in range(blocks):
        for layer, (_, K, N) in enumerate(wl.BLOCK_LINEARS):
            W = to_dev_bf16(torch, wl.decode_weight(b, layer))
            qw, sc, qz = w4.awq_quantize_pack(W)
            del W
            packed.append((b, layer, K, N, qw, sc, qz))
    torch.cuda.synchronize()
    return packed


def sweep_launches(torch, w4, wl, packed, M):
    launches = []
    for b, layer, K, N, qw, sc, qz in packed:
        X = to_dev_bf16(torch, wl.decode_act(b, layer, M))
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        launches.append(Launch(w4.gemv_launcher(X, qw, sc, qz, False, Y), gemv_bytes(M, K, N, False),
                               2 * M * K * N))
    torch.cuda.synchronize()
    return launches


def w4a8_sweep_launches(torch, w4, wl, packed, M):
    """The decode sweep on the W4A8 path: activations quantized once up front (in a
    real decoder the previous op emits them), one w4a8_gemv per linear."""
    launches = []
    for b, layer, K, N, qw, sc, qz in packed:
        X = to_dev_bf16(torch, wl.decode_act(b, layer, M))
        Xq, sx, xs = w4.w4a8_quantize_activations(X)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        launches.append(Launch(w4.w4a8_gemv_launcher(Xq, sx, xs, qw, sc, qz, False, Y),
                               packed_bytes(N, K, False) + M * K + M * 4 + M * (K // GROUP) * 4 + M * N * 2,
                               2 * M * K * N))
    torch.cuda.synchronize()
    return launches


def capture_graph(torch, launches):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for l in launches:          # warm the launch path outside capture
            l()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for l in launches:
            l()
    torch.cuda.synchronize()
    return g


def rotation_launches(torch, w4, X, qw, sc, qz, sym, min_bytes, make, M, K, N, flops_fn):
    """Copies of one packed weight whose total exceeds min_bytes: launch i uses copy i."""
    per = packed_bytes(N, K, sym)
    copies = max(1, -(-min_bytes // per))
    launches = []
    for _ in range(copies):
        q2, s2 = qw.clone(), sc.clone()
        z2 = None if qz is None else qz.clone()
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        launches.append(Launch(make(X, q2, s2, z2, sym, Y), gemv_bytes(M, K, N, sym), flops_fn(M, K, N)))
    return launches


def measure_rotation(torch, launches, reps):
    """Cold-cache average ms per launch: the launches over every copy, in order, are
    captured in one HIP graph; each rep replays it once (no host launch cost)."""
    g = capture_graph(torch, launches)
    g.replay()
    torch.cuda.synchronize()
    ms = time_events(torch, g.replay, reps) / len(launches)
    del g
    return ms


def fused_sweep_launches(torch, w4, wl, packed, M, w4a8=False):
    """The decode step as a decoder runs it: the linears of a block that read the same
    activations (q, k, v; gate, up) are one GEMV each over their packed rows stored
    concatenated along N (contiguous in the N-major layout): q|k|v (N = 4096) and
    gate|up (N = 12288), with the activation row of the block's first linear of the
    group.  Four launches per block: q|k|v, o, gate|up, down; the same weight bytes
    as one launch per linear.  w4a8: the same launches on the W4A8 path (activations
    quantized up front, as for w4a8_sweep_launches)."""
    by_block = {}
    for b, layer, K, N, qw, sc, qz in packed:
        by_block.setdefault(b, {})[layer] = (K, N, qw, sc, qz)
    launches = []
    for b in sorted(by_block):
        L = by_block[b]
        for group in ((0, 1, 2), (3,), (4, 5), (6,)):
            K = L[group[0]][0]
            N = sum(L[i][1] for i in group)
            qw = torch.cat([L[i][2] for i in group], 0)
            sc = torch.cat([L[i][3] for i in group], 0)
            qz = torch.cat([L[i][4] for i in group], 0)
            X = to_dev_bf16(torch, wl.decode_act(b, group[0], M))
            Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            if w4a8:
                Xq, sx, xs = w4.w4a8_quantize_activations(X)
                launches.append(Launch(w4.w4a8_gemv_launcher(Xq, sx, xs, qw, sc, qz, False, Y),
                                       packed_bytes(N, K, False) + M * K + M * 4 + M * (K // GROUP) * 4 + M * N * 2,
                                       2 * M * K * N))
            else:
                launches.append(Launch(w4.gemv_launcher(X, qw, sc, qz, False, Y), gemv_bytes(M, K, N, False),
                                       2 * M * K * N))
    torch.cuda.synchronize()
    return launches


# ----------------------------------------------------------------------------- rows

def row_gemv(name, nbytes, ms, extra=None):
    gbs = nbytes / (ms * 1e-3) / 1e9
    d = {"name": name, "bytes": int(nbytes), "us": round(ms * 1e3, 3), "GB/s": round(gbs, 1),
         "bound": "hbm", "frac": round(gbs / HBM_PEAK_GBS, 4)}
    if extra:
        d.update(extra)
    return d


def row_gemm(name, flops, ms, extra=None):
    tf = flops / (ms * 1e-3) / 1e12
    d = {"name": name, "flops": int(flops), "us": round(ms * 1e3, 3), "TFLOP/s": round(tf, 1),
         "bound": "mfma", "frac": round(tf / BF16_PEAK_TFLOPS, 4)}
    if extra:
        d.update(extra)
    return d


def stream_read_sweep(torch, w4, nbytes, reps, min_bytes=640 << 20):
    """Cold plain read of nbytes: a graph of launches of the streaming-read probe, launch i
    reading slice i of a buffer larger than the Infinity Cache, for every unroll depth,
    load kind and grid size; returns (best ms per launch, its settings, all settings' us)."""
    nbytes = (nbytes + 255) // 256 * 256
    copies = max(2, -(-min_bytes // nbytes))
    buf = torch.empty(copies * nbytes // 4, dtype=torch.int32, device="cuda")
    buf.fill_(1)
    sink = torch.empty(8192 * 256, dtype=torch.int32, device="cuda")
    table, best = {}, None
    for unroll in (1, 2, 4, 8):
        for nt in (False, True):
            for blocks in (256, 512, 1024, 2048, 4096, 8192):
                ls = [Launch(lambda sl=buf[i * nbytes // 4:(i + 1) * nbytes // 4], u=unroll, n=nt, b=blocks:
                             w4.probe_stream_read(sl, unroll=u, nontemporal=n, blocks=b, sink=sink), nbytes, 0)
                      for i in range(copies)]
                ms = measure_rotation(torch, ls, reps)
                key = f"u{unroll}{'nt' if nt else ''}b{blocks}"
                table[key] = round(ms * 1e3, 2)
                if best is None or ms < best[0]:
                    best = (ms, {"unroll": unroll, "nontemporal": nt, "blocks": blocks})
    del buf, sink
    torch.cuda.empty_cache()
    return best[0], best[1], table


def plain_read_step(torch, w4, sizes, reps=10, settings=None):
    """Yardstick for the decode step: one graph of plain streaming reads with the step's
    launch sizes in its order, each over a buffer of its own (nothing cached from the previous
    replay once the step exceeds the Infinity Cache), for every probe unroll depth, load kind and
    grid size (or only the given settings); returns (best ms per step, its settings)."""
    sizes = [(n + 255) // 256 * 256 for n in sizes]
    offs = [0]
    for n in sizes:
        offs.append(offs[-1] + n)
    buf = torch.empty(offs[-1] // 4, dtype=torch.int32, device="cuda")
    buf.fill_(1)
    sink = torch.empty(4096 * 256, dtype=torch.int32, device="cuda")
    best = None
    if settings is None:
        settings = [{"unroll": u, "nontemporal": nt, "blocks": b}
                    for u in (1, 2, 4, 8) for nt in (False, True) for b in (256, 512, 1024, 2048, 4096)]
    for cfg in settings:
        ls = [Launch(lambda sl=buf[offs[i] // 4:offs[i + 1] // 4], u=cfg["unroll"], n=cfg["nontemporal"],
                     b=cfg["blocks"]: w4.probe_stream_read(sl, unroll=u, nontemporal=n, blocks=b, sink=sink),
                     sizes[i], 0)
              for i in range(len(sizes))]
        g = capture_graph(torch, ls)
        g.replay()
        ms = min(time_events(torch, g.replay, reps) for _ in range(2))
        del g, ls
        if best is None or ms < best[0]:
            best = (ms, dict(cfg))
    del buf, sink
    torch.cuda.empty_cache()
    return best


def rows_large(torch, w4, wl, reps):
    rows = []
    # 27B-shaped symmetric linears: cold-cache GEMV at M = 1, 8 and GEMM at M = 16, 32, 48, 64, 512
    for si, (K, N) in enumerate(wl.LARGE_SHAPES):
        # yardstick: the best cold plain read of the M = 1 GEMV's bytes
        read_bytes = gemv_bytes(1, K, N, True)
        read_ms, read_cfg, read_table = stream_read_sweep(torch, w4, read_bytes, max(2, reps // 4))
        rows.append(row_gemv(f"plain read cold {read_bytes} B (best of {len(read_table)} settings)", read_bytes,
                             read_ms, {"settings": read_cfg, "us_by_setting": read_table}))
        W = to_dev_bf16(torch, wl.large_weight(si))
        # quantize + pack (HBM-bound read of bf16 W and write of the packed form)
        qw, sc, _ = w4.awq_quantize_pack(W, symmetric=True)
        ms = time_events(torch, lambda: w4.awq_quantize_pack(W, symmetric=True, qweight=qw, scales=sc), reps)
        qbytes = N * K * 2 + packed_bytes(N, K, True)
        rows.append(row_gemv(f"quantize_pack sym K={K} N={N}", qbytes, ms))
        del W
        for M in (1, 8):
            X = to_dev_bf16(torch, wl.large_act(si, M))
            ls = rotation_launches(torch, w4, X, qw, sc, None, True, 600 << 20, w4.gemv_launcher, M, K, N,
                                   lambda m, k, n: 2 * m * k * n)
            ms = measure_rotation(torch, ls, max(2, reps // 4))
            rows.append(row_gemv(f"gemv cold M={M} K={K} N={N} sym", ls[0].nbytes, ms,
                                 {"cache": f"cold ({len(ls)} rotating copies)",
                                  "of_best_plain_read": round(read_ms / ms, 4) if M == 1 else None}))
            del ls
        for M in (1, 16):
            X = to_dev_bf16(torch, wl.large_act(si, M))
            Xq, sx, xs = w4.w4a8_quantize_activations(X)
            nbytes = packed_bytes(N, K, True) + M * K + M * 4 + M * (K // GROUP) * 4 + M * N * 2
            ls = rotation_launches(torch, w4, None, qw, sc, None, True, 600 << 20,
                                   lambda _x, q2, s2, z2, sym, Y: w4.w4a8_gemv_launcher(Xq, sx, xs, q2, s2, z2, sym, Y),
                                   M, K, N, lambda m, k, n: 2 * m * k * n)
            for l in ls:
                l.nbytes = nbytes
            ms = measure_rotation(torch, ls, max(2, reps // 4))
            rows.append(row_gemv(f"W4A8 gemv cold M={M} K={K} N={N} sym", nbytes, ms,
                                 {"cache": f"cold ({len(ls)} rotating copies)"}))
            del ls
        # M = 16: the decode GEMV's kernels; M = 32, 48: the one-pass form; M = 64, 512: the tiled core
        for M in (16, 32, 48, 64, 512):
            X = to_dev_bf16(torch, wl.large_act(si, M))
            Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            ms = time_events(torch, w4.gemm_launcher(X, qw, sc, None, True, Y), reps)
            rows.append(row_gemm(f"gemm M={M} K={K} N={N} sym", 2 * M * K * N, ms,
                                 {"GB/s": round(gemv_bytes(M, K, N, True) / (ms * 1e-3) / 1e9, 1)}))
        torch.cuda.synchronize()
        del qw, sc
    return rows


def rows_prefill(torch, w4, wl, reps):
    rows = []
    # prefill GEMM, M = 2048, outlier channels
    for si, (K, N) in enumerate(wl.PREFILL_SHAPES):
        Xn, Wn = wl.prefill(si)
        X, W = to_dev_bf16(torch, Xn), to_dev_bf16(torch, Wn)
        qw, sc, qz = w4.awq_quantize_pack(W)
        Y = torch.empty((wl.PREFILL_M, N), dtype=torch.bfloat16, device="cuda")
        ms = time_events(torch, w4.gemm_launcher(X, qw, sc, qz, False, Y), reps)
        rows.append(row_gemm(f"gemm prefill M=2048 K={K} N={N}", 2 * wl.PREFILL_M * K * N, ms))
    return rows


def rows_gemv2048(torch, w4, wl, reps):
    rows = []
    # single GEMV, M = 1, K = N = 2048: warm (cache-resident) and cold (rotation)
    Xn, Wn = wl.gemv_2048()
    X, W = to_dev_bf16(torch, Xn), to_dev_bf16(torch, Wn)
    qw, sc, qz = w4.awq_quantize_pack(W)
    Y = torch.empty((1, 2048), dtype=torch.bfloat16, device="cuda")
    same = [w4.gemv_launcher(X, qw, sc, qz, False, Y)] * 100
    g = capture_graph(torch, same)
    ms = time_events(torch, g.replay, max(3, reps // 4)) / len(same)
    del g
    rows.append(row_gemv("gemv M=1 K=2048 N=2048 (cache-resident, graph of 100)", gemv_bytes(1, 2048, 2048, False),
                         ms))
    ls = rotation_launches(torch, w4, X, qw, sc, qz, False, 600 << 20, w4.gemv_launcher, 1, 2048, 2048,
                           lambda m, k, n: 2 * m * k * n)
    ms = measure_rotation(torch, ls, 3)
    rows.append(row_gemv("gemv M=1 K=2048 N=2048 (cold)", gemv_bytes(1, 2048, 2048, False), ms,
                         {"cache": f"cold ({len(ls)} rotating copies)"}))
    del ls
    return rows


def rows_search(torch, w4, wl, reps):
    rows = []
    # full AWQ search: 20 alphas then 10 ratios, T=4096, K=2048, N=6144
    Xn, Wn = wl.awq_calibration()
    X, W = to_dev_bf16(torch, Xn), to_dev_bf16(torch, Wn)
    alphas = [i / 20 for i in range(20)]
    ratios = [1 - j / 20 for j in range(10)]
    res = w4.awq_search(X, W, alphas, ratios)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 2
    for _ in range(n):
        res = w4.awq_search(X, W, alphas, ratios)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / n
    flops = 31 * 2 * wl.AWQ_T * wl.AWQ_K * wl.AWQ_N
    rows.append(row_gemm("awq_search T=4096 K=2048 N=6144 (20 alpha + 10 ratio + ref)", flops, ms,
                         {"alpha_index": res["alpha_index"], "ratio_index": res["ratio_index"]}))
    return rows


def rows_clip(torch, w4, wl, reps):
    """Per-output-channel clipping search at the search workload's full size: T=4096
    calibration tokens, K=2048, N=6144, the 10-ratio grid, s = s(alpha*) from the
    two-phase search (untimed).  Algorithmic work: the Gram matrices (2 T K 128
    flops) and e^T H_g e for every (channel, group, ratio) (2 N K R 128 flops)."""
    rows = []
    Xn, Wn = wl.awq_calibration()
    X, W = to_dev_bf16(torch, Xn), to_dev_bf16(torch, Wn)
    res = w4.awq_search(X, W, [i / 20 for i in range(20)], [1 - j / 20 for j in range(10)])
    s = res["s"]
    ratios = torch.tensor([1 - j / 20 for j in range(10)], dtype=torch.float32, device="cuda")
    T, K = X.shape
    N = W.shape[0]
    R = ratios.numel()
    flops = 2 * T * K * 128 + 2 * N * K * R * 128
    for sym in (False, True):
        L, best = w4.awq_clip_search(X, W, ratios, s=s, symmetric=sym)
        ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
        ms = time_events(torch, lambda: w4.awq_clip_search(X, W, ratios, s=s, symmetric=sym, losses=L, best=best,
                                                          workspace=ws), reps)
        hist = torch.bincount(best.flatten().long(), minlength=R).tolist()
        rows.append(row_gemm(f"per-channel clip search T={T} K={K} N={N} R={R} {'sym' if sym else 'asym'}",
                             flops, ms, {"choice_histogram": hist}))
    return rows


def block_flops(T, B, L, H, I, n_q, n_kv):
    """Algorithmic flops of one decoder-block forward: the seven linears (2 T per weight)
    and causal attention (q k^T and p v over the L (L + 1) / 2 visible pairs per head)."""
    params = H * 128 * n_q * 2 + 2 * H * 128 * n_kv + 3 * H * I
    return 2 * T * params + 2 * 2 * B * n_q * (L * (L + 1) // 2) * 128


def rows_lookahead(torch, w4, wl, reps):
    """Look-ahead (d = 1) scoring at the base model's block shape: 8 sequences x 512
    tokens, hidden 2048, 16 / 8 heads, FFN 6144.  Each candidate runs the scored block
    with the candidate linear and the next block (two block forwards)."""
    rows = []
    shp = wl.QWEN_BLOCK
    H, I, n_q, n_kv = shp["H"], shp["I"], shp["n_q"], shp["n_kv"]
    B, L = wl.LOOKAHEAD_B, wl.LOOKAHEAD_L
    T = B * L
    dev = lambda b: {k: to_dev_bf16(torch, v) for k, v in b.items()}
    blk, nxt = dev(wl.synthetic_block(H, I, n_q, n_kv, 0)), dev(wl.synthetic_block(H, I, n_q, n_kv, 1))
    X = to_dev_bf16(torch, wl.block_input(T, H, 0))
    f_blk = block_flops(T, B, L, H, I, n_q, n_kv)
    ws = torch.empty(1, dtype=torch.uint8, device="cuda")
    Y = w4.block_forward(X, B, L, blk, n_q, n_kv)
    ms = time_events(torch, lambda: w4.block_forward(X, B, L, blk, n_q, n_kv, Y=Y), reps)
    rows.append(row_gemm(f"decoder block forward T={T} (B={B} L={L}) H={H} I={I} heads {n_q}/{n_kv}", f_blk, ms))
    C = 10
    S = torch.ones((C, 2048), dtype=torch.float32, device="cuda")
    ratios = torch.tensor([1 - j / 20 for j in range(C)], dtype=torch.float32, device="cuda")
    w4.awq_lookahead_loss(X, B, L, blk, nxt, n_q, n_kv, "gate", S, ratios)
    t0 = time.perf_counter()
    n = 2
    for _ in range(n):
        l1, _ = w4.awq_lookahead_loss(X, B, L, blk, nxt, n_q, n_kv, "gate", S, ratios)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / n
    # a gate candidate reruns the feed-forward half of the scored block (the attention
    # half is the reference's) and the whole next block; of the feed-forward half only
    # gate and down change with the candidate (the up projection runs once per call)
    f_cand = 2 * T * 2 * H * I + f_blk
    f_up = 2 * T * H * I
    rows.append(row_gemm(f"look-ahead losses, gate, {C} candidates (feed-forward half + next block each) + reference",
                         C * f_cand + 2 * f_blk + f_up, ms, {"ms_per_candidate_with_reference_share": round(ms / C, 3)}))
    res = w4.awq_search_lookahead(X, B, L, blk, nxt, n_q, n_kv, "gate", [i / 20 for i in range(20)],
                                  [1 - j / 20 for j in range(10)])
    t0 = time.perf_counter()
    res = w4.awq_search_lookahead(X, B, L, blk, nxt, n_q, n_kv, "gate", [i / 20 for i in range(20)],
                                  [1 - j / 20 for j in range(10)])
    ms = (time.perf_counter() - t0) * 1e3
    rows.append(row_gemm("look-ahead two-phase search, gate (20 alpha + 10 ratio + reference)",
                         30 * f_cand + 2 * f_blk + 2 * f_up, ms,
                         {"alpha_index": res["alpha_index"], "ratio_index": res["ratio_index"]}))
    return rows


def rows_convert(torch, w4, wl, reps):
    """Streaming data-free symmetric conversion of a synthetic 3-shard checkpoint
    (8 hidden-2048 blocks, 0.87 GB of bf16) written to a temporary directory."""
    import shutil
    import tempfile
    from weight_only_int4_amd import convert as C
    rows = []
    tmp = tempfile.mkdtemp(prefix="w4ckpt_")
    try:
        src, dst = os.path.join(tmp, "src"), os.path.join(tmp, "dst")
        wl.write_checkpoint(src, blocks=8, shards=3)
        C.convert_checkpoint(src, dst)                  # warm: library, staging buffer, page cache
        st = C.convert_checkpoint(src, dst)
        n_w = st["bytes_converted"] // 2
        alg = n_w * 2 + packed_bytes(1, GROUP, True) * n_w // GROUP     # bf16 read + packed written
        rows.append({"name": "streaming symmetric conversion, 3 shards, 8 blocks (end to end, files on host)",
                     "bytes": int(st["bytes_converted"]), "us": round(st["wall_s"] * 1e6, 1),
                     "GB/s": round(st["bytes_converted"] / st["wall_s"] / 1e9, 2), "bound": "host IO",
                     "tensors": st["converted"], "written_bytes": int(st["bytes_written"])})
        rows.append(row_gemv("streaming symmetric conversion: quantize kernel only (sum over tensors)", alg,
                             st["kernel_s"] * 1e3, {"weights": int(n_w)}))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return rows


# ----------------------------------------------------------------------------- CPU baseline

def _cpu_threads():
    """(threads BLAS uses, os.cpu_count(), CPUs this process may run on)."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas = 1
    try:
        aff = len(os.sched_getaffinity(0))
    except Exception:
        aff = os.cpu_count() or 1
    return int(blas), int(os.cpu_count() or 1), int(aff)


def _cpu_timed(fn, budget_s):
    """Calls fn() until budget_s of wall time is spent (at least once); (calls, seconds)."""
    n, spent = 0, 0.0
    while n == 0 or spent < budget_s:
        t0 = time.perf_counter()
        fn()
        spent += time.perf_counter() - t0
        n += 1
    return n, spent


def cpu_baseline(wl, gpu_rows=None, budget_s=8.0):
    """The CPU oracle on bounded samples of the workloads, on this host's cores.

    value: the decode sweep's metric -- oracle dequantize + fp64 linear over the 14
    linears of the sweep's first two blocks (M = 1), repeated for budget_s; TB/s of
    algorithmic bytes.  rows: the other steps of the path, each on a sample of its
    own workload, with the GPU row of the same workload when this run measured it:
    quantize + pack (NumPy elementwise, one thread), dequantize, the prefill fp64
    contraction (BLAS, multithreaded) and the AWQ search (reference output plus three
    candidates of the 30, each a quantize + dequantize + fp64 contraction)."""
    from oracle import w4a16_oracle as O
    blas, ncpu, aff = _cpu_threads()
    gpu = {r["name"]: r for r in (gpu_rows or [])}
    # decode sweep GEMV (the metric)
    cache = {}
    for b in range(2):
        for layer, (_, K, N) in enumerate(wl.BLOCK_LINEARS):
            cache[(b, layer)] = (K, N, wl.decode_act(b, layer, 1), O.quantize_pack(wl.decode_weight(b, layer)))
    done = {"bytes": 0, "n": 0}

    def sweep_pass():
        for K, N, X, (qw, sc, qz) in cache.values():
            O.linear(X, O.dequantize(qw, sc, qz, K, False))
            done["bytes"] += gemv_bytes(1, K, N, False)
            done["n"] += 1
    _, spent = _cpu_timed(sweep_pass, budget_s)
    out = {"value": round(done["bytes"] / spent / 1e12, 6), "unit": "TB/s", "cores": blas, "kind": "oracle",
           "sample": f"{done['n']} GEMVs over the 14 linears of the first 2 blocks of the decode sweep (M=1), "
                     f"repeated: oracle dequantize + fp64 linear, {spent:.1f} s",
           "cpu_count": ncpu, "affinity_cpus": aff, "blas_threads": blas}
    rows = []
    # quantize + pack and dequantize: one 27B-shaped symmetric linear, a slice of 2048 rows
    K, N = wl.LARGE_SHAPES[0]
    W = wl.large_weight(0)[:2048]
    n, t = _cpu_timed(lambda: O.quantize_pack(W, None, 1.0, True), 1.0)
    nb = W.size * 2 + packed_bytes(W.shape[0], K, True)
    row = {"name": f"oracle quantize_pack sym K={K}, {W.shape[0]} of N={N} rows", "GB/s": round(nb * n / t / 1e9, 3),
           "threads": 1, "seconds": round(t, 2)}
    g = [r for r in gpu.values() if r["name"].startswith(f"quantize_pack sym K={K}")]
    if g:
        row["gpu_GB/s"] = g[0]["GB/s"]
        row["gpu_speedup"] = round(g[0]["GB/s"] / row["GB/s"], 1)
    rows.append(row)
    qw, sc, _ = O.quantize_pack(W, None, 1.0, True)
    n, t = _cpu_timed(lambda: O.dequantize(qw, sc, None, K, True), 1.0)
    rows.append({"name": f"oracle dequantize sym K={K}, {W.shape[0]} rows",
                 "GB/s": round(packed_bytes(W.shape[0], K, True) * n / t / 1e9, 3), "threads": 1,
                 "seconds": round(t, 2)})
    # prefill contraction: the first prefill shape, all 2048 rows, fp64 (BLAS)
    X, Wp = wl.prefill(0)
    Kp, Np = wl.PREFILL_SHAPES[0]
    qp = O.quantize_pack(Wp)
    What = O.dequantize(*qp, Kp, False)
    n, t = _cpu_timed(lambda: O.linear(X, What), 1.0)
    fl = 2 * X.shape[0] * Kp * Np
    row = {"name": f"oracle fp64 linear M={X.shape[0]} K={Kp} N={Np}", "GFLOP/s": round(fl * n / t / 1e9, 2),
           "threads": blas, "seconds": round(t, 2)}
    g = [r for r in gpu.values() if r["name"].startswith(f"gemm prefill M={X.shape[0]} K={Kp} N={Np}")]
    if g:
        row["gpu_TFLOP/s"] = g[0]["TFLOP/s"]
        row["gpu_speedup"] = round(g[0]["TFLOP/s"] * 1e3 / row["GFLOP/s"], 1)
    rows.append(row)
    del X, Wp, What
    # AWQ search: reference output and 3 of the 30 candidates; scaled to the full search
    Xs, Ws = wl.awq_calibration()
    t0 = time.perf_counter()
    m = O.act_mean_abs(Xs)
    Yref = O.reference_output(Xs, Ws)
    for a in (0.0, 0.25, 0.5):
        O.candidate_loss(Xs, Ws, O.awq_scales(m, a), 1.0, False, Yref)
    t = time.perf_counter() - t0
    full_s = t / 4 * 31
    row = {"name": "oracle AWQ search T=4096 K=2048 N=6144: reference + 3 of 30 candidates",
           "seconds": round(t, 2), "threads": blas, "full_search_estimate_s": round(full_s, 1)}
    g = [r for r in gpu.values() if r["name"].startswith("awq_search T=4096")]
    if g:
        row["gpu_ms"] = g[0]["us"] / 1e3
        row["gpu_speedup"] = round(full_s * 1e3 / row["gpu_ms"], 1)
    rows.append(row)
    out["rows"] = rows
    return out


def trace_summary(trace_dir):
    """Kernel durations inside the timed region of a rocprofv3 kernel trace of this
    script (--kernel-trace --output-format csv): the dispatches that start after the
    first launch of the empty probe kernel ends and end before the second starts.
    Prints one JSON line per kernel name: dispatches, mean / median / min duration
    (us) and the region's wall time."""
    import csv
    import glob
    path = sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True))
    if not path:
        print(f"no kernel_trace.csv under {trace_dir}", file=sys.stderr)
        return 2
    rows = list(csv.DictReader(open(path[0])))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    marks = [r for r in rows if "empty_kernel" in r["Kernel_Name"]][:2]
    if len(marks) < 2:
        print("the trace holds no timed-region markers", file=sys.stderr)
        return 2
    lo, hi = int(marks[0]["End_Timestamp"]), int(marks[1]["Start_Timestamp"])
    inside = [r for r in rows if int(r["Start_Timestamp"]) >= lo and int(r["End_Timestamp"]) <= hi]
    by = {}
    for r in inside:
        by.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    first = min(int(r["Start_Timestamp"]) for r in inside)
    last = max(int(r["End_Timestamp"]) for r in inside)
    for name, d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        d = sorted(d)
        print(json.dumps({"kernel": name, "dispatches": len(d), "mean_us": round(sum(d) / len(d), 3),
                          "median_us": round(d[len(d) // 2], 3), "min_us": round(d[0], 3),
                          "sum_us": round(sum(d), 1), "region_us": round((last - first) / 1e3, 1)}))
    return 0


# ----------------------------------------------------------------------------- main

def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--step-only", action="store_true", help="measure only the decode-sweep step")
    ap.add_argument("--only", default="", help="comma list of extra rows to measure "
                    "(sweeps,w4a8,large,prefill,gemv2048,search,clip,lookahead,convert); default all")
    ap.add_argument("--blocks", type=int, default=28)
    ap.add_argument("--skip-step", action="store_true",
                    help="profiling aid: skip the decode-sweep step (value is null) and run only --only rows")
    ap.add_argument("--trace-summary", default="", metavar="DIR",
                    help="print the kernel durations inside the timed step of a rocprofv3 kernel trace "
                         "of this script written under DIR, and exit (no GPU)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="counter calibration: run only a plain device copy of MIB MiB ten times and exit")
    args = ap.parse_args(argv)
    if args.trace_summary:
        return trace_summary(args.trace_summary)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the kernels would shard by "
              "output rows with no exchange). Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    import weight_only_int4_amd as w4
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if args.copy_probe:
        # a plain copy of known size: reads and writes copy_probe MiB per dispatch, so
        # the HBM counters of a profiler run over it calibrate FETCH_SIZE / WRITE_SIZE
        src = torch.ones(args.copy_probe << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": src.numel() * 4, "dispatches": 10}), flush=True)
        return 0
    w4.load_library()

    out = {
        "metric": "W4A16 g128 GEMV achieved TB/s (M=1) + GEMM TFLOP/s (M=2048), % roofline",
        "value": None,
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 x int4 (fp32 accumulate)",
        "data": "synthetic (seeded; W ~ N(0,0.02) bf16, X ~ N(0,1) bf16)",
        "config": {"workload": f"decode sweep: {args.blocks} blocks x 7 linears of a hidden-2048 decoder block "
                               f"(q,k,v,o,gate,up,down), M=1, asymmetric int4 g128, the shared-input linears "
                               f"launched together as a decoder runs them (q|k|v, o, gate|up, down: 4 GEMV "
                               f"launches per block), HIP-graph replay"},
    }
    packed = []
    t0 = None                       # latency floor per launch (us), measured with the step
    read_cfg = None                 # best plain-read setting for the step's launches
    if not args.skip_step:
        log("packing decode-sweep weights")
        packed = pack_sweep(torch, w4, wl, args.blocks)
        sweep = fused_sweep_launches(torch, w4, wl, packed, 1)
        step_bytes = sum(l.nbytes for l in sweep)
        graph = capture_graph(torch, sweep)

        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # the first two launches of the empty probe kernel in the run bracket the timed
        # region, so that a kernel trace of this run can be cut to it (--trace-summary)
        w4.probe_empty()
        s.record()
        for _ in range(args.steps):
            graph.replay()
        e.record()
        w4.probe_empty()
        torch.cuda.synchronize()
        ms_step = s.elapsed_time(e) / args.steps
        value = step_bytes / (ms_step * 1e-3) / 1e12
        log(f"sweep: {ms_step * 1e3:.1f} us/step, {value:.3f} TB/s")

        # dominant kernel: the step is a graph of GEMV launches only, so its event-timed
        # duration over the timed region divided by the launches is the average launch
        # duration on the launch stream (back-to-back, inter-kernel gaps included)
        avg_launch_ms = ms_step / len(sweep)
        avg_bytes = step_bytes / len(sweep)
        achieved = avg_bytes / (avg_launch_ms * 1e-3) / 1e9
        eager_ms = time_events(torch, lambda: [l() for l in sweep], max(2, args.steps // 4))
        out["value"] = round(value, 4)
        out["ms_per_step"] = round(ms_step, 5)
        out["config"].update({"bytes_per_step": int(step_bytes), "launches_per_step": len(sweep),
                              "eager_ms_per_step": round(eager_ms, 5)})
        out["roofline"] = {"kernel": "gemv_kernel<M=1>", "bound": "hbm", "achieved": round(achieved, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": profiled_traffic(), "avg_launch_us": round(avg_launch_ms * 1e3, 3),
                           "bytes_per_launch": int(avg_bytes)}
        t0 = latency_floor_us(torch, w4, len(sweep))
        ideal_us = step_bytes / (HBM_PEAK_GBS * 1e3)
        ceil_frac = ideal_us / (len(sweep) * t0 + ideal_us)
        out["roofline"]["latency_floor"] = {"t0_us": round(t0, 3), "ceiling_frac": round(ceil_frac, 4),
                                            "frac_of_ceiling": round(achieved / HBM_PEAK_GBS / ceil_frac, 4)}
        log(f"latency floor: t0 {t0:.2f} us per launch, step ceiling {ceil_frac:.3f} of HBM peak")
        read_ms, read_cfg = plain_read_step(torch, w4, [l.nbytes for l in sweep])
        out["roofline"]["plain_read_step"] = {
            "us_per_launch": round(read_ms * 1e3 / len(sweep), 3), "settings": read_cfg,
            "frac": round(step_bytes / (read_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "gemv_of_read": round(read_ms / ms_step, 4)}
        log(f"plain read of the step's bytes in the same launches: {read_ms * 1e3:.1f} us per step")
        del graph, sweep
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    want = set(x for x in args.only.split(",") if x) or {"sweeps", "w4a8", "large", "prefill", "gemv2048",
                                                         "search", "clip", "lookahead", "convert"}
    if not args.step_only:
        rows = []
        if "sweeps" in want and packed:
            log("decode sweep M=1, one launch per linear")
            fs = sweep_launches(torch, w4, wl, packed, 1)
            g = capture_graph(torch, fs)
            ms = time_events(torch, g.replay, max(3, args.steps // 2))
            rows.append(row_gemv("decode sweep M=1, one GEMV launch per linear (graph)",
                                 sum(l.nbytes for l in fs), ms, {"launches": len(fs)}))
            del g, fs
            torch.cuda.empty_cache()
        for M in ((1, 4, 8, 16) if "w4a8" in want and packed else ()):
            log(f"W4A8 decode sweep M={M}")
            sw = w4a8_sweep_launches(torch, w4, wl, packed, M)
            g = capture_graph(torch, sw)
            ms = time_events(torch, g.replay, max(3, args.steps // 2))
            rows.append(row_gemv(f"W4A8 decode sweep M={M} (graph)", sum(l.nbytes for l in sw), ms))
            del g, sw
            sw = fused_sweep_launches(torch, w4, wl, packed, M, w4a8=True)
            g = capture_graph(torch, sw)
            ms = time_events(torch, g.replay, max(3, args.steps // 2))
            rows.append(row_gemv(f"W4A8 decode sweep M={M}, shared-input linears fused (graph)",
                                 sum(l.nbytes for l in sw), ms, {"launches": len(sw)}))
            del g, sw
            torch.cuda.empty_cache()
        for M in ((4, 8, 16) if "sweeps" in want and packed else ()):
            log(f"decode sweep M={M}")
            sw = sweep_launches(torch, w4, wl, packed, M)
            g = capture_graph(torch, sw)
            ms = time_events(torch, g.replay, max(3, args.steps // 2))
            rows.append(row_gemv(f"decode sweep M={M} (graph)", sum(l.nbytes for l in sw), ms))
            del g, sw
            sw = fused_sweep_launches(torch, w4, wl, packed, M)
            g = capture_graph(torch, sw)
            ms = time_events(torch, g.replay, max(3, args.steps // 2))
            extra = {"launches": len(sw)}
            if read_cfg is not None:
                # the same bytes read plainly in the same launches (the step's best setting)
                rms, _ = plain_read_step(torch, w4, [l.nbytes for l in sw], settings=[read_cfg])
                extra.update({"plain_read_us": round(rms * 1e3, 1), "of_plain_read": round(rms / ms, 4)})
            rows.append(row_gemv(f"decode sweep M={M}, shared-input linears fused (graph)",
                                 sum(l.nbytes for l in sw), ms, extra))
            del g, sw
            torch.cuda.empty_cache()
        del packed
        torch.cuda.empty_cache()
        reps = max(5, args.steps)
        for name, fn in (("large", rows_large), ("prefill", rows_prefill), ("gemv2048", rows_gemv2048),
                         ("search", rows_search), ("clip", rows_clip), ("lookahead", rows_lookahead),
                         ("convert", rows_convert)):
            if name in want:
                log(f"rows: {name}")
                rows += fn(torch, w4, wl, reps)
        # single-GEMV rows: the best fraction of the HBM peak a launch of that size can
        # reach when every launch also costs t0
        gemv_rows = [r for r in rows if r["name"].startswith("gemv") and "bytes" in r]
        if gemv_rows:
            t0 = t0 if t0 is not None else latency_floor_us(torch, w4, 112)
            for r in gemv_rows:
                r["latency_ceiling_frac"] = round(latency_ceiling(t0, r["bytes"]), 4)
        out["rows"] = rows
        pre = [r for r in rows if r["name"].startswith("gemm prefill")]
        if pre:
            out["prefill_gemm_tflops"] = [r["TFLOP/s"] for r in pre]
            out["prefill_gemm_frac"] = [r["frac"] for r in pre]
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(wl, out.get("rows"))
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
