"""Weight-only int4, group-128 linear layers (W4A16) on AMD MI355X (gfx950).

Thin Python binding over the C-ABI library ``libw4a16.so`` (see
``include/w4a16.h``).  The functions keep the C names; they check dtype,
device and contiguity, allocate outputs with torch (device memory only),
pass raw pointers and the current HIP stream, and raise ``W4Error`` on a
non-zero status.  Every computation runs in the library's HIP kernels: there
is no Python or CPU fallback, and a missing library is an error.

Tensor conventions: bf16 data as ``torch.bfloat16``; packed uint32 words
(qweight, qzeros) as ``torch.int32`` tensors holding the same bits.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "W4Error", "library_path", "load_library", "awq_quantize_pack", "w4a16_gemv", "w4a16_gemv_noalloc", "w4a16_gemm", "bf16_linear",
    "awq_grid_loss", "awq_search", "GROUP_SIZE", "GEMV_MAX_M", "gemv_launcher", "gemm_launcher",
    "w4a8_quantize_activations", "w4a8_gemv", "w4a8_gemv_launcher", "awq_clip_search", "block_forward",
    "block_forward_quantized", "awq_lookahead_loss", "awq_search_lookahead", "BLOCK_LINEARS", "probe_stream_read", "probe_empty",
]

GROUP_SIZE = 128
GEMV_MAX_M = 16
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.POINTER(ctypes.c_size_t)

BLOCK_LINEARS = ("q", "k", "v", "o", "gate", "up", "down")
_BLOCK_FIELDS = ("norm1", "wq", "wk", "wv", "wo", "norm2", "wgate", "wup", "wdown")


class _Block(ctypes.Structure):
    """struct w4_block: device pointers of one decoder block's bf16 weights."""
    _fields_ = [(f, ctypes.c_void_p) for f in _BLOCK_FIELDS]


_bp = ctypes.POINTER(_Block)
_SIGNATURES = {
    "w4_status_string": ([_i], ctypes.c_char_p),
    "awq_quantize_pack": ([_vp, _i, _i, _vp, _f, _i, _i, _vp, _vp, _vp, _vp], _i),
    "w4a16_gemv": ([_vp, _i, _i, _i, _vp, _vp, _vp, _i, _i, _vp, _vp, _sz, _vp], _i),
    "w4a16_gemm": ([_vp, _i, _i, _i, _vp, _vp, _vp, _i, _i, _vp, _vp, _sz, _vp], _i),
    "w4a16_gemv_noalloc": ([_vp, _i, _i, _i, _vp, _vp, _vp, _i, _i, _vp, _vp], _i),
    "w4_bf16_linear": ([_vp, _i, _i, _i, _vp, _vp, _vp], _i),
    "awq_grid_loss": ([_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _i, _i, _vp, _vp, _sz, _vp], _i),
    "w4_probe_stream_read": ([_vp, ctypes.c_size_t, _i, _i, _i, _vp, _vp], _i),
    "w4_probe_empty": ([_vp], _i),
    "w4a8_quantize_activations": ([_vp, _i, _i, _vp, _vp, _vp, _vp], _i),
    "w4a8_gemv": ([_vp, _vp, _vp, _i, _i, _i, _vp, _vp, _vp, _i, _i, _vp, _vp, _sz, _vp], _i),
    "awq_clip_search": ([_vp, _i, _i, _i, _vp, _vp, _vp, _i, _i, _i, _vp, _vp, _vp, _sz, _vp], _i),
    "w4_block_forward": ([_vp, _i, _i, _i, _i, _i, _i, _bp, _vp, _vp, _sz, _vp], _i),
    "w4_block_forward_quantized": ([_vp, _i, _i, _i, _i, _i, _i, _bp, _i, _vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _sz,
                                    _vp], _i),
    "awq_lookahead_loss": ([_vp, _i, _i, _i, _i, _i, _i, _bp, _bp, _i, _vp, _vp, _i, _i, _i, _vp, _vp, _vp, _sz, _vp],
                           _i),
    "awq_search_lookahead": ([_vp, _i, _i, _i, _i, _i, _i, _bp, _bp, _i, ctypes.POINTER(ctypes.c_double), _i,
                              ctypes.POINTER(ctypes.c_double), _i, _i, _i, ctypes.POINTER(ctypes.c_float),
                              ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int), _vp, _vp, _sz, _vp], _i),
    "awq_search": ([_vp, _i, _i, _i, _vp, ctypes.POINTER(ctypes.c_double), _i,
                    ctypes.POINTER(ctypes.c_double), _i, _i, _i, ctypes.POINTER(ctypes.c_float),
                    ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int), _vp, _vp, _sz, _vp], _i),
}


class W4Error(RuntimeError):
    """A W4A16 library call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, "libw4a16.so")


def load_library() -> ctypes.CDLL:
    """Load libw4a16.so (built in-tree by ``python -m weight_only_int4_amd.build``)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m weight_only_int4_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _LIB = lib
    return _LIB


def _check(rc: int) -> None:
    if rc != 0:
        msg = load_library().w4_status_string(rc).decode()
        raise W4Error(rc, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, name, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")


def _workspace(query, device, workspace):
    size = ctypes.c_size_t(0)
    _check(query(ctypes.byref(size)))
    if size.value == 0:
        return None, None
    if workspace is None or workspace.numel() < size.value:
        workspace = torch.empty(size.value, dtype=torch.uint8, device=device)
    return workspace, ctypes.c_size_t(workspace.numel())


def awq_quantize_pack(W, s=None, clip_ratio: float = 1.0, symmetric: bool = False,
                      qweight=None, scales=None, qzeros=None):
    """Quantize W [N][K] bf16 (times diag(s), clipped at clip_ratio) to packed int4.

    Returns (qweight int32 [N][K/8], scales bf16 [N][K/128], qzeros int32
    [N][ceil(K/1024)] or None when symmetric).
    """
    lib = load_library()
    _need(W, torch.bfloat16, "W", 2)
    N, K = W.shape
    dev = W.device
    if s is not None:
        _need(s, torch.float32, "s", 1)
    G = K // GROUP_SIZE
    if qweight is None:
        qweight = torch.empty((N, K // 8), dtype=torch.int32, device=dev)
    if scales is None:
        scales = torch.empty((N, G), dtype=torch.bfloat16, device=dev)
    if not symmetric and qzeros is None:
        qzeros = torch.empty((N, (G + 7) // 8), dtype=torch.int32, device=dev)
    if symmetric:
        qzeros = None
    _check(lib.awq_quantize_pack(_ptr(W), N, K, _ptr(s), float(clip_ratio), int(symmetric), GROUP_SIZE,
                                 _ptr(qweight), _ptr(scales), _ptr(qzeros), _stream(dev)))
    return qweight, scales, qzeros


def _packed_shapes(X, qweight, scales, qzeros, symmetric):
    _need(X, torch.bfloat16, "X", 2)
    _need(qweight, torch.int32, "qweight", 2)
    _need(scales, torch.bfloat16, "scales", 2)
    if not symmetric:
        _need(qzeros, torch.int32, "qzeros", 2)
    M, K = X.shape
    N = qweight.shape[0]
    if qweight.shape[1] * 8 != K:
        raise ValueError("qweight must be [N][K/8] for X [M][K]")
    return M, K, N


def w4a16_gemv(X, qweight, scales, qzeros=None, symmetric: bool = False, Y=None, workspace=None):
    """Decode GEMV: Y [M][N] bf16 = X [M][K] (M <= 16) times the dequantized weight, transposed."""
    lib = load_library()
    M, K, N = _packed_shapes(X, qweight, scales, qzeros, symmetric)
    dev = X.device
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    qz = None if symmetric else qzeros

    def q(sz):
        return lib.w4a16_gemv(None, M, K, N, None, None, None, int(symmetric), GROUP_SIZE, None, None, sz, None)

    ws, wsb = _workspace(q, dev, workspace)
    _check(lib.w4a16_gemv(_ptr(X), M, K, N, _ptr(qweight), _ptr(scales), _ptr(qz), int(symmetric), GROUP_SIZE,
                          _ptr(Y), _ptr(ws), None if wsb is None else ctypes.byref(wsb), _stream(dev)))
    return Y


def w4a16_gemv_noalloc(X, qweight, scales, qzeros, symmetric: bool, Y):
    """Decode GEMV into the caller's Y [M][N] bf16 without any device allocation: the
    K-split partial sums use the library's static scratch array (see include/w4a16.h,
    w4a16_gemv_noalloc; calls overlapping on one device race)."""
    lib = load_library()
    M, K, N = _packed_shapes(X, qweight, scales, qzeros, symmetric)
    _need(Y, torch.bfloat16, "Y", 2)
    if tuple(Y.shape) != (M, N):
        raise ValueError(f"Y must have shape {(M, N)}")
    qz = None if symmetric else qzeros
    _check(lib.w4a16_gemv_noalloc(_ptr(X), M, K, N, _ptr(qweight), _ptr(scales), _ptr(qz), int(symmetric), GROUP_SIZE,
                                  _ptr(Y), _stream(X.device)))
    return Y


def bf16_linear(X, W, Y=None):
    """Unquantized linear Y [M][N] = bf16(X [M][K] W [N][K]^T) on the library's bf16 kernel."""
    lib = load_library()
    _need(X, torch.bfloat16, "X", 2)
    _need(W, torch.bfloat16, "W", 2)
    M, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("W must be [N][K] for X [M][K]")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    _check(lib.w4_bf16_linear(_ptr(X), M, K, N, _ptr(W), _ptr(Y), _stream(X.device)))
    return Y


def w4a8_quantize_activations(X, Xq=None, sx=None, xsum=None):
    """Per-row int8 activations for the W4A8 decode path: returns (Xq int8 [M][K],
    sx fp32 [M], xsum int32 [M][K/128])."""
    lib = load_library()
    _need(X, torch.bfloat16, "X", 2)
    M, K = X.shape
    dev = X.device
    Xq = torch.empty((M, K), dtype=torch.int8, device=dev) if Xq is None else Xq
    sx = torch.empty(M, dtype=torch.float32, device=dev) if sx is None else sx
    xsum = torch.empty((M, K // GROUP_SIZE), dtype=torch.int32, device=dev) if xsum is None else xsum
    _check(lib.w4a8_quantize_activations(_ptr(X), M, K, _ptr(Xq), _ptr(sx), _ptr(xsum), _stream(dev)))
    return Xq, sx, xsum


def _w4a8_args(Xq, sx, xsum, qweight, scales, qzeros, symmetric):
    _need(Xq, torch.int8, "Xq", 2)
    _need(sx, torch.float32, "sx", 1)
    _need(xsum, torch.int32, "xsum", 2)
    _need(qweight, torch.int32, "qweight", 2)
    _need(scales, torch.bfloat16, "scales", 2)
    if not symmetric:
        _need(qzeros, torch.int32, "qzeros", 2)
    M, K = Xq.shape
    N = qweight.shape[0]
    if qweight.shape[1] * 8 != K or sx.shape[0] != M or tuple(xsum.shape) != (M, K // GROUP_SIZE):
        raise ValueError("shapes of Xq [M][K], sx [M], xsum [M][K/128], qweight [N][K/8] disagree")
    return M, K, N


def _w4a8_workspace(lib, M, K, N, symmetric, device, workspace):
    def q(sz):
        return lib.w4a8_gemv(None, None, None, M, K, N, None, None, None, int(symmetric), GROUP_SIZE, None, None,
                             sz, None)

    return _workspace(q, device, workspace)


def w4a8_gemv(Xq, sx, xsum, qweight, scales, qzeros=None, symmetric: bool = False, Y=None, workspace=None):
    """W4A8 decode GEMV: Y [M][N] bf16 from int8 activations (w4a8_quantize_activations)."""
    lib = load_library()
    M, K, N = _w4a8_args(Xq, sx, xsum, qweight, scales, qzeros, symmetric)
    dev = Xq.device
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws, wsb = _w4a8_workspace(lib, M, K, N, symmetric, dev, workspace)
    _check(lib.w4a8_gemv(_ptr(Xq), _ptr(sx), _ptr(xsum), M, K, N, _ptr(qweight), _ptr(scales),
                         _ptr(None if symmetric else qzeros), int(symmetric), GROUP_SIZE, _ptr(Y), _ptr(ws),
                         None if wsb is None else ctypes.byref(wsb), _stream(dev)))
    return Y


def w4a8_gemv_launcher(Xq, sx, xsum, qweight, scales, qzeros, symmetric: bool, Y, workspace=None):
    """As gemv_launcher, for w4a8_gemv."""
    lib = load_library()
    M, K, N = _w4a8_args(Xq, sx, xsum, qweight, scales, qzeros, symmetric)
    _need(Y, torch.bfloat16, "Y", 2)
    if tuple(Y.shape) != (M, N):
        raise ValueError("Y must be [M][N]")
    qz = None if symmetric else qzeros
    dev = Xq.device
    ws, wsb = _w4a8_workspace(lib, M, K, N, symmetric, dev, workspace)
    args = (_ptr(Xq), _ptr(sx), _ptr(xsum), M, K, N, _ptr(qweight), _ptr(scales), _ptr(qz), int(symmetric),
            GROUP_SIZE, _ptr(Y), _ptr(ws), None if wsb is None else ctypes.byref(wsb))

    def launch():
        _check(lib.w4a8_gemv(*args, _stream(dev)))

    launch.tensors = (Xq, sx, xsum, qweight, scales, qz, Y, ws)
    launch.workspace_size = wsb
    return launch


def w4a16_gemm(X, qweight, scales, qzeros=None, symmetric: bool = False, Y=None, workspace=None):
    """Prefill GEMM (MFMA): Y [M][N] bf16 = X [M][K] times the dequantized weight, transposed."""
    lib = load_library()
    M, K, N = _packed_shapes(X, qweight, scales, qzeros, symmetric)
    dev = X.device
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    qz = None if symmetric else qzeros

    def q(sz):
        return lib.w4a16_gemm(None, M, K, N, None, None, None, int(symmetric), GROUP_SIZE, None, None, sz, None)

    ws, wsb = _workspace(q, dev, workspace)
    _check(lib.w4a16_gemm(_ptr(X), M, K, N, _ptr(qweight), _ptr(scales), _ptr(qz), int(symmetric), GROUP_SIZE,
                          _ptr(Y), _ptr(ws), None if wsb is None else ctypes.byref(wsb), _stream(dev)))
    return Y


def awq_grid_loss(X, W, S, ratios, symmetric: bool = False, Yref=None, losses=None, workspace=None):
    """Losses [C] fp32 of the candidates (S[c], ratios[c]) against bf16(X W^T) (or Yref)."""
    lib = load_library()
    _need(X, torch.bfloat16, "X", 2)
    _need(W, torch.bfloat16, "W", 2)
    _need(S, torch.float32, "S", 2)
    _need(ratios, torch.float32, "ratios", 1)
    if Yref is not None:
        _need(Yref, torch.bfloat16, "Yref", 2)
    T, K = X.shape
    N = W.shape[0]
    C = S.shape[0]
    dev = X.device
    if losses is None:
        losses = torch.empty(C, dtype=torch.float32, device=dev)

    def q(sz):
        return lib.awq_grid_loss(None, T, K, N, None, _ptr(Yref) if Yref is not None else None, None, None, C,
                                 int(symmetric), GROUP_SIZE, None, None, sz, None)

    ws, wsb = _workspace(q, dev, workspace)
    _check(lib.awq_grid_loss(_ptr(X), T, K, N, _ptr(W), _ptr(Yref), _ptr(S), _ptr(ratios), C, int(symmetric),
                             GROUP_SIZE, _ptr(losses), _ptr(ws), None if wsb is None else ctypes.byref(wsb),
                             _stream(dev)))
    return losses


def awq_clip_search(X, W, ratios, s=None, symmetric: bool = False, want_losses: bool = True, losses=None,
                    best=None, workspace=None):
    """Per-output-channel clipping search.  Returns (losses [G][N][R] fp32 or None,
    best [N][G] uint8): for channel n and group g, losses over the ratio grid of the
    group's squared partial-output error over the tokens, and the first ratio index
    of least loss."""
    lib = load_library()
    _need(X, torch.bfloat16, "X", 2)
    _need(W, torch.bfloat16, "W", 2)
    _need(ratios, torch.float32, "ratios", 1)
    if s is not None:
        _need(s, torch.float32, "s", 1)
    T, K = X.shape
    N = W.shape[0]
    R = ratios.shape[0]
    G = K // GROUP_SIZE
    dev = X.device
    if want_losses and losses is None:
        losses = torch.empty((G, N, R), dtype=torch.float32, device=dev)
    if best is None:
        best = torch.empty((N, G), dtype=torch.uint8, device=dev)

    def q(sz):
        return lib.awq_clip_search(None, T, K, N, None, None, None, R, int(symmetric), GROUP_SIZE, None, None,
                                   None, sz, None)

    ws, wsb = _workspace(q, dev, workspace)
    _check(lib.awq_clip_search(_ptr(X), T, K, N, _ptr(W), _ptr(s), _ptr(ratios), R, int(symmetric), GROUP_SIZE,
                               _ptr(losses) if want_losses else None, _ptr(best), _ptr(ws),
                               None if wsb is None else ctypes.byref(wsb), _stream(dev)))
    return (losses if want_losses else None), best


def _block_struct(blk, H, n_q, n_kv, I):
    """blk: dict with "norm1", "norm2" (bf16 [H]) and q, k, v, o, gate, up, down (bf16 [out][in])."""
    shapes = {"norm1": (H,), "norm2": (H,), "q": (128 * n_q, H), "k": (128 * n_kv, H), "v": (128 * n_kv, H),
              "o": (H, 128 * n_q), "gate": (I, H), "up": (I, H), "down": (H, I)}
    for name, shape in shapes.items():
        _need(blk[name], torch.bfloat16, name)
        if tuple(blk[name].shape) != shape:
            raise ValueError(f"{name} must have shape {shape}, got {tuple(blk[name].shape)}")
    keys = ("norm1", "q", "k", "v", "o", "norm2", "gate", "up", "down")
    return _Block(*[blk[k].data_ptr() for k in keys])


def block_forward(X, B: int, L: int, blk, n_q: int, n_kv: int, Y=None, workspace=None):
    """Y [B L][H] bf16 = decoder block(X) (see include/w4a16.h, w4_block_forward)."""
    lib = load_library()
    _need(X, torch.bfloat16, "X", 2)
    T, H = X.shape
    if T != B * L:
        raise ValueError("X must have B * L rows")
    I = blk["gate"].shape[0]
    b = _block_struct(blk, H, n_q, n_kv, I)
    if Y is None:
        Y = torch.empty_like(X)

    def q(sz):
        return lib.w4_block_forward(None, B, L, H, n_q, n_kv, I, None, None, None, sz, None)

    ws, wsb = _workspace(q, X.device, workspace)
    _check(lib.w4_block_forward(_ptr(X), B, L, H, n_q, n_kv, I, ctypes.byref(b), _ptr(Y), _ptr(ws),
                                None if wsb is None else ctypes.byref(wsb), _stream(X.device)))
    return Y


def block_forward_quantized(X, B: int, L: int, blk, n_q: int, n_kv: int, linear, s, qweight, scales, qzeros=None,
                            symmetric: bool = False, Y=None, workspace=None):
    """Y [B L][H] bf16 = decoder block(X) with linear `linear` in its deployed int4 form:
    input bf16(a / s) against the packed weights of Q(W diag(s)) (see include/w4a16.h,
    w4_block_forward_quantized)."""
    lib = load_library()
    _need(X, torch.bfloat16, "X", 2)
    _need(s, torch.float32, "s", 1)
    T, H = X.shape
    if T != B * L:
        raise ValueError("X must have B * L rows")
    I = blk["gate"].shape[0]
    li = BLOCK_LINEARS.index(linear) if isinstance(linear, str) else int(linear)
    b = _block_struct(blk, H, n_q, n_kv, I)
    K = blk[BLOCK_LINEARS[li]].shape[1]
    if s.shape[0] != K or qweight.shape[1] * 8 != K:
        raise ValueError("s must have the linear's input size K and qweight K/8 columns")
    qz = None if symmetric else qzeros
    if Y is None:
        Y = torch.empty_like(X)

    def q(sz):
        return lib.w4_block_forward_quantized(None, B, L, H, n_q, n_kv, I, None, li, None, None, None, None,
                                              int(symmetric), GROUP_SIZE, None, None, sz, None)

    ws, wsb = _workspace(q, X.device, workspace)
    _check(lib.w4_block_forward_quantized(_ptr(X), B, L, H, n_q, n_kv, I, ctypes.byref(b), li, _ptr(s),
                                          _ptr(qweight), _ptr(scales), _ptr(qz), int(symmetric), GROUP_SIZE, _ptr(Y),
                                          _ptr(ws), None if wsb is None else ctypes.byref(wsb), _stream(X.device)))
    return Y


def awq_lookahead_loss(X, B: int, L: int, blk, nxt, n_q: int, n_kv: int, linear, S, ratios,
                       symmetric: bool = False, want_d0: bool = True, workspace=None):
    """Look-ahead (d = 1) losses [C] of candidates (S[c], ratios[c]) for one linear of
    block blk scored after block nxt (None: the last block, scored at its own output),
    and the block-output (d = 0) losses [C] (or None)."""
    lib = load_library()
    _need(X, torch.bfloat16, "X", 2)
    _need(S, torch.float32, "S", 2)
    _need(ratios, torch.float32, "ratios", 1)
    T, H = X.shape
    if T != B * L:
        raise ValueError("X must have B * L rows")
    I = blk["gate"].shape[0]
    li = BLOCK_LINEARS.index(linear) if isinstance(linear, str) else int(linear)
    b = _block_struct(blk, H, n_q, n_kv, I)
    nb = None if nxt is None else _block_struct(nxt, H, n_q, n_kv, I)
    C = S.shape[0]
    losses = torch.empty(C, dtype=torch.float32, device=X.device)
    d0 = torch.empty(C, dtype=torch.float32, device=X.device) if want_d0 else None

    def q(sz):
        return lib.awq_lookahead_loss(None, B, L, H, n_q, n_kv, I, None, None, li, None, None, C, int(symmetric),
                                      GROUP_SIZE, None, None, None, sz, None)

    ws, wsb = _workspace(q, X.device, workspace)
    _check(lib.awq_lookahead_loss(_ptr(X), B, L, H, n_q, n_kv, I, ctypes.byref(b),
                                  None if nb is None else ctypes.byref(nb), li, _ptr(S), _ptr(ratios), C,
                                  int(symmetric), GROUP_SIZE, _ptr(losses), _ptr(d0), _ptr(ws),
                                  None if wsb is None else ctypes.byref(wsb), _stream(X.device)))
    return losses, d0


def awq_search_lookahead(X, B: int, L: int, blk, nxt, n_q: int, n_kv: int, linear, alphas, ratios,
                         symmetric: bool = False, workspace=None):
    """Two-phase AWQ search of one linear of block blk scored after block nxt (None:
    the last block).  Returns dict(alpha_losses, ratio_losses, alpha_index,
    ratio_index, s).  Synchronizes."""
    lib = load_library()
    _need(X, torch.bfloat16, "X", 2)
    T, H = X.shape
    if T != B * L:
        raise ValueError("X must have B * L rows")
    I = blk["gate"].shape[0]
    li = BLOCK_LINEARS.index(linear) if isinstance(linear, str) else int(linear)
    b = _block_struct(blk, H, n_q, n_kv, I)
    nb = None if nxt is None else _block_struct(nxt, H, n_q, n_kv, I)
    K = blk[BLOCK_LINEARS[li]].shape[1]
    a = (ctypes.c_double * len(alphas))(*[float(x) for x in alphas])
    r = (ctypes.c_double * len(ratios))(*[float(x) for x in ratios])
    out = (ctypes.c_float * (len(alphas) + len(ratios)))()
    ia, ir = ctypes.c_int(-1), ctypes.c_int(-1)
    s_out = torch.empty(K, dtype=torch.float32, device=X.device)

    def q(sz):
        return lib.awq_search_lookahead(None, B, L, H, n_q, n_kv, I, None, None, li, a, len(alphas), r, len(ratios),
                                        int(symmetric), GROUP_SIZE, None, None, None, None, None, sz, None)

    ws, wsb = _workspace(q, X.device, workspace)
    _check(lib.awq_search_lookahead(_ptr(X), B, L, H, n_q, n_kv, I, ctypes.byref(b),
                                    None if nb is None else ctypes.byref(nb), li, a, len(alphas), r, len(ratios),
                                    int(symmetric), GROUP_SIZE, out, ctypes.byref(ia), ctypes.byref(ir), _ptr(s_out),
                                    _ptr(ws), None if wsb is None else ctypes.byref(wsb), _stream(X.device)))
    vals = list(out)
    return dict(alpha_losses=vals[: len(alphas)], ratio_losses=vals[len(alphas):], alpha_index=ia.value,
                ratio_index=ir.value, s=s_out)


def awq_search(X, W, alphas, ratios, symmetric: bool = False, workspace=None):
    """Two-phase AWQ search.  Returns dict(alpha_losses, ratio_losses, alpha_index,
    ratio_index, s) with s = s(alpha*) as a fp32 GPU tensor.  Synchronizes."""
    lib = load_library()
    _need(X, torch.bfloat16, "X", 2)
    _need(W, torch.bfloat16, "W", 2)
    T, K = X.shape
    N = W.shape[0]
    dev = X.device
    a = (ctypes.c_double * len(alphas))(*[float(x) for x in alphas])
    r = (ctypes.c_double * len(ratios))(*[float(x) for x in ratios])
    out = (ctypes.c_float * (len(alphas) + len(ratios)))()
    ia, ir = ctypes.c_int(-1), ctypes.c_int(-1)
    s_out = torch.empty(K, dtype=torch.float32, device=dev)

    def q(sz):
        return lib.awq_search(None, T, K, N, None, a, len(alphas), r, len(ratios), int(symmetric), GROUP_SIZE,
                              None, None, None, None, None, sz, None)

    ws, wsb = _workspace(q, dev, workspace)
    _check(lib.awq_search(_ptr(X), T, K, N, _ptr(W), a, len(alphas), r, len(ratios), int(symmetric), GROUP_SIZE,
                          out, ctypes.byref(ia), ctypes.byref(ir), _ptr(s_out), _ptr(ws),
                          None if wsb is None else ctypes.byref(wsb), _stream(dev)))
    vals = list(out)
    return dict(alpha_losses=vals[: len(alphas)], ratio_losses=vals[len(alphas):], alpha_index=ia.value,
                ratio_index=ir.value, s=s_out)


def _launcher(cname, X, qweight, scales, qzeros, symmetric, Y, workspace):
    lib = load_library()
    M, K, N = _packed_shapes(X, qweight, scales, qzeros, symmetric)
    _need(Y, torch.bfloat16, "Y", 2)
    if tuple(Y.shape) != (M, N):
        raise ValueError("Y must be [M][N]")
    fn = getattr(lib, cname)
    qz = None if symmetric else qzeros

    def q(sz):
        return fn(None, M, K, N, None, None, None, int(symmetric), GROUP_SIZE, None, None, sz, None)

    ws, wsb = _workspace(q, X.device, workspace)
    keep = (X, qweight, scales, qz, Y, ws)          # tensors stay alive while the launcher does
    args = (_ptr(X), M, K, N, _ptr(qweight), _ptr(scales), _ptr(qz), int(symmetric), GROUP_SIZE, _ptr(Y),
            _ptr(ws), None if wsb is None else ctypes.byref(wsb))
    dev = X.device

    def launch():
        _check(fn(*args, _stream(dev)))

    launch.tensors = keep
    launch.workspace_size = wsb
    return launch


def gemv_launcher(X, qweight, scales, qzeros, symmetric: bool, Y, workspace=None):
    """Validate once and return a zero-argument callable that enqueues the GEMV
    Y = X W_hat^T on the current stream (for graph capture and timing loops)."""
    return _launcher("w4a16_gemv", X, qweight, scales, qzeros, symmetric, Y, workspace)


def gemm_launcher(X, qweight, scales, qzeros, symmetric: bool, Y, workspace=None):
    """As gemv_launcher, for the MFMA GEMM."""
    return _launcher("w4a16_gemm", X, qweight, scales, qzeros, symmetric, Y, workspace)


def probe_stream_read(buf, unroll: int = 4, nontemporal: bool = False, blocks: int = 0, sink=None):
    """Measurement helper: enqueue a plain streaming read of the whole tensor `buf`."""
    lib = load_library()
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    nbytes = buf.numel() * buf.element_size()
    if blocks <= 0:
        blocks = 256 * 8
    if sink is None or sink.numel() < blocks * 256:
        sink = torch.empty(blocks * 256, dtype=torch.int32, device=buf.device)
    _check(lib.w4_probe_stream_read(_ptr(buf), nbytes, int(unroll), int(nontemporal), int(blocks), _ptr(sink),
                                    _stream(buf.device)))
    return sink


def probe_empty(device="cuda"):
    """Measurement helper: enqueue an empty kernel."""
    _check(load_library().w4_probe_empty(_stream(torch.device(device))))
