"""The C-ABI library on the host, no GPU: it loads, exports every function that
include/w4a16.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import weight_only_int4_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")
P = ctypes.c_void_p
A = P(0x10000)        # a 16-byte aligned fake device address (never dereferenced)
MIS = P(0x10004)      # misaligned fake address


@pytest.fixture(scope="module")
def lib():
    return w4.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("awq_quantize_pack", "w4a16_gemv", "w4a16_gemm", "awq_grid_loss", "awq_search", "awq_clip_search",
              "w4_block_forward", "awq_lookahead_loss", "awq_search_lookahead", "w4_status_string"):
        assert n in names, names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(0, -9, -1):
        s = lib.w4_status_string(code).decode()
        assert s.startswith("W4_"), s
    assert lib.w4_status_string(-99).decode() == "W4_ERR_UNKNOWN"


def q(lib, W=A, N=4, K=256, s=None, r=1.0, sym=0, gs=128, qw=A, sc=A, qz=A):
    return lib.awq_quantize_pack(W, N, K, s, r, sym, gs, qw, sc, qz, None)


def test_quantize_validation(lib):
    assert q(lib, K=100) == -2
    assert q(lib, K=0) == -2
    assert q(lib, N=-1) == -2
    assert q(lib, gs=64) == -4
    assert q(lib, W=None) == -1
    assert q(lib, qw=None) == -1
    assert q(lib, sym=1) == -1                  # qzeros must be NULL when symmetric
    assert q(lib, qz=None) == -1                # and set when asymmetric
    assert q(lib, W=MIS) == -3
    assert q(lib, s=MIS) == -3
    assert q(lib, r=0.0) == -7
    assert q(lib, r=1.5) == -7
    assert q(lib, r=float("nan")) == -7
    assert q(lib, sym=2, qz=None) == -7
    assert q(lib, N=0) == 0                     # empty: nothing enqueued


def test_gemv_validation_and_size_query(lib):
    sz = ctypes.c_size_t(123)
    f = lib.w4a16_gemv
    assert f(A, 17, 256, 8, A, A, A, 0, 128, A, None, None, None) == -4
    assert f(A, 1, 200, 8, A, A, A, 0, 128, A, None, None, None) == -2
    assert f(A, 1, 256, 8, A, A, A, 0, 32, A, None, None, None) == -4
    assert f(None, 1, 2048, 2048, None, None, None, 0, 128, None, None, ctypes.byref(sz), None) == 0
    assert sz.value == 0
    assert f(None, 16, 17408, 5120, None, None, None, 1, 128, None, None, ctypes.byref(sz), None) == 0
    assert sz.value > 0
    need = sz.value
    small = ctypes.c_size_t(need - 4)
    assert f(A, 16, 17408, 5120, A, A, None, 1, 128, A, A, ctypes.byref(small), None) == -5
    assert f(A, 16, 17408, 5120, A, A, None, 1, 128, A, None, None, None) == -5
    assert f(None, 1, 256, 8, A, A, A, 0, 128, A, None, None, None) == -1
    assert f(A, 1, 256, 8, A, A, None, 0, 128, A, None, None, None) == -1
    assert f(MIS, 1, 256, 8, A, A, A, 0, 128, A, None, None, None) == -3
    assert f(A, 0, 256, 8, A, A, A, 0, 128, A, None, None, None) == 0      # M = 0: empty


def test_gemv_size_limits(lib):
    """32-bit buffer offsets: N K / 2 < 2^31 and 32 K < 2^31, checked by the size
    query and by the call (before any HIP call), for both decode forms."""
    sz = ctypes.c_size_t(123)
    f = lib.w4a16_gemv
    for M in (1, 16):
        # the largest N at K = 2048 (packed weights 2^31 - 1024 bytes), then one more
        assert f(None, M, 2048, (1 << 21) - 1, None, None, None, 1, 128, None, None, ctypes.byref(sz), None) == 0
        assert f(None, M, 2048, 1 << 21, None, None, None, 1, 128, None, None, ctypes.byref(sz), None) == -2
        assert f(A, M, 2048, 1 << 21, A, A, None, 1, 128, A, None, None, None) == -2
        assert lib.w4a16_gemv_noalloc(A, M, 2048, 1 << 21, A, A, None, 1, 128, A, None) == -2
    assert f(None, 1, 1 << 26, 1, None, None, None, 1, 128, None, None, ctypes.byref(sz), None) == -2   # 32 K = 2^31
    assert f(None, 1, (1 << 26) - 128, 1, None, None, None, 1, 128, None, None, ctypes.byref(sz), None) == 0


def test_grid_loss_search_w4a8_size_limits(lib):
    sz = ctypes.c_size_t(123)
    g = lib.awq_grid_loss
    # (T + 64) K < 2^31 at K = 2048; N K < 2^31; C <= 65535 -- size query and call alike
    assert g(None, (1 << 20) - 65, 2048, 64, None, None, None, None, 1, 0, 128, None, None, ctypes.byref(sz), None) == 0
    assert g(None, (1 << 20) - 64, 2048, 64, None, None, None, None, 1, 0, 128, None, None, ctypes.byref(sz), None) == -2
    assert g(None, 64, 2048, 1 << 20, None, None, None, None, 1, 0, 128, None, None, ctypes.byref(sz), None) == -2
    assert g(None, 64, 2048, 64, None, None, None, None, 65536, 0, 128, None, None, ctypes.byref(sz), None) == -2
    big = ctypes.c_size_t(1 << 40)
    assert g(A, (1 << 20) - 64, 2048, 64, A, None, A, A, 1, 0, 128, A, A, ctypes.byref(big), None) == -2
    al = (ctypes.c_double * 2)(0.0, 0.5)
    ra = (ctypes.c_double * 2)(1.0, 0.9)
    s = lib.awq_search
    assert s(None, 64, 2048, 1 << 20, None, al, 2, ra, 2, 0, 128, None, None, None, None, None,
             ctypes.byref(sz), None) == -2
    assert s(None, 64, 2048, 64, None, al, 2, ra, 2, 0, 128, None, None, None, None, None,
             ctypes.byref(sz), None) == 0
    w = lib.w4a8_gemv
    assert w(None, None, None, 1, 2048, 1 << 21, None, None, None, 1, 128, None, None, ctypes.byref(sz), None) == -2
    assert w(None, None, None, 1, 2048, (1 << 21) - 1, None, None, None, 1, 128, None, None, ctypes.byref(sz),
             None) == 0


def test_gemv_noalloc_validation(lib):
    f = lib.w4a16_gemv_noalloc
    assert f(A, 17, 256, 8, A, A, A, 0, 128, A, None) == -4
    assert f(A, 1, 200, 8, A, A, A, 0, 128, A, None) == -2
    assert f(A, 1, 256, 8, A, A, A, 0, 32, A, None) == -4
    assert f(None, 1, 256, 8, A, A, A, 0, 128, A, None) == -1
    assert f(A, 1, 256, 8, A, A, None, 0, 128, A, None) == -1
    assert f(A, 1, 256, 8, A, A, A, 1, 128, A, None) == -1          # qzeros must be NULL when symmetric
    assert f(MIS, 1, 256, 8, A, A, A, 0, 128, A, None) == -3
    assert f(A, 0, 256, 8, A, A, A, 0, 128, A, None) == 0           # M = 0: empty, no HIP call
    # split partials above the 8 MiB static array: rejected before any HIP call
    sz = ctypes.c_size_t(0)
    assert lib.w4a16_gemv(None, 16, 17408, 50000, None, None, None, 1, 128, None, None, ctypes.byref(sz), None) == 0
    assert sz.value > 8 << 20
    assert f(A, 16, 17408, 50000, A, A, None, 1, 128, A, None) == -8
    assert lib.w4_status_string(-8).decode().startswith("W4_ERR_SCRATCH")


def test_w4a8_validation(lib):
    f = lib.w4a8_quantize_activations
    assert f(A, 17, 256, A, A, A, None) == -4
    assert f(A, 1, 200, A, A, A, None) == -2
    assert f(A, -1, 256, A, A, A, None) == -2
    assert f(None, 1, 256, A, A, A, None) == -1
    assert f(A, 1, 256, A, None, A, None) == -1
    assert f(MIS, 1, 256, A, A, A, None) == -3
    assert f(A, 0, 256, A, A, A, None) == 0                         # M = 0: empty
    g = lib.w4a8_gemv
    assert g(A, A, A, 17, 256, 8, A, A, A, 0, 128, A, None, None, None) == -4
    assert g(A, A, A, 1, 200, 8, A, A, A, 0, 128, A, None, None, None) == -2
    assert g(A, A, A, 1, 256, 8, A, A, A, 0, 64, A, None, None, None) == -4
    assert g(A, A, A, 1, 51328, 8, A, A, A, 0, 128, A, None, None, None) == -4   # 401 groups: beyond the unrolled kernels
    assert g(None, A, A, 1, 256, 8, A, A, A, 0, 128, A, None, None, None) == -1
    assert g(A, A, None, 1, 256, 8, A, A, A, 0, 128, A, None, None, None) == -1
    assert g(A, A, A, 1, 256, 8, A, A, None, 0, 128, A, None, None, None) == -1  # asymmetric needs qzeros
    assert g(A, A, A, 1, 256, 8, A, A, A, 1, 128, A, None, None, None) == -1     # symmetric forbids them
    assert g(MIS, A, A, 1, 256, 8, A, A, A, 0, 128, A, None, None, None) == -3
    assert g(A, A, A, 0, 256, 8, A, A, A, 0, 128, A, None, None, None) == 0
    # K split (at least 64 groups, fewer than 512 column tiles): fp32 partials per split
    sz = ctypes.c_size_t(0)
    assert g(None, None, None, 1, 8192, 2048, None, None, None, 0, 128, None, None, ctypes.byref(sz), None) == 0
    assert sz.value == 4 * 1 * 2048 * 4                  # 64 groups in 4 ranges of 16
    assert g(None, None, None, 16, 17408, 5120, None, None, None, 1, 128, None, None, ctypes.byref(sz), None) == 0
    assert sz.value == 2 * 16 * 5120 * 4                 # 136 groups in 2 ranges of 68
    for K, N in ((5120, 17408), (6144, 2048), (8064, 64)):   # enough tiles, or under 64 groups: no split
        assert g(None, None, None, 4, K, N, None, None, None, 0, 128, None, None, ctypes.byref(sz), None) == 0
        assert sz.value == 0
    assert g(A, A, A, 1, 8192, 2048, A, A, A, 0, 128, A, None, None, None) == -5
    small = ctypes.c_size_t(4 * 2048 * 4 - 1)
    assert g(A, A, A, 1, 8192, 2048, A, A, A, 0, 128, A, A, ctypes.byref(small), None) == -5


def test_gemm_size_query(lib):
    sz = ctypes.c_size_t(0)
    f = lib.w4a16_gemm
    assert f(None, 2048, 2048, 6144, None, None, None, 0, 128, None, None, ctypes.byref(sz), None) == 0
    # pair-arranged X [M rounded to 64][K] bf16, per-group row sums bf16 [G][M rounded to
    # 64][4] and per-group column words u32 [G][N rounded to 128], each rounded up to 256 bytes
    assert sz.value == 2048 * 2048 * 2 + 16 * 2048 * 8 + 16 * 6144 * 4
    assert f(None, 200, 384, 8, None, None, None, 0, 128, None, None, ctypes.byref(sz), None) == 0
    need = 256 * 384 * 2 + 3 * 256 * 8 + 3 * 128 * 4
    assert sz.value == need
    assert f(A, 200, 384, 8, A, A, A, 0, 128, A, None, None, None) == -5
    small = ctypes.c_size_t(need - 1)
    assert f(A, 200, 384, 8, A, A, A, 0, 128, A, A, ctypes.byref(small), None) == -5
    ok = ctypes.c_size_t(need)
    assert f(A, 200, 384, 8, A, A, A, 0, 128, MIS, A, ctypes.byref(ok), None) == -3
    # 32-bit offsets: (M + 64) K < 2^31 (arranged activations) and N K < 2^33 (packed weights),
    # from the size query and the call alike
    K = 2048
    assert f(None, (1 << 20) - 65, K, 64, None, None, None, 0, 128, None, None, ctypes.byref(sz), None) == 0
    assert f(None, (1 << 20) - 64, K, 64, None, None, None, 0, 128, None, None, ctypes.byref(sz), None) == -2
    big = ctypes.c_size_t(1 << 40)
    assert f(A, (1 << 20) - 64, K, 64, A, A, A, 0, 128, A, A, ctypes.byref(big), None) == -2
    assert f(None, 64, K, (1 << 22) - 1, None, None, None, 0, 128, None, None, ctypes.byref(sz), None) == 0
    assert f(None, 64, K, 1 << 22, None, None, None, 0, 128, None, None, ctypes.byref(sz), None) == -2


def test_gemm_short_m_workspace(lib):
    """Up to 16 rows the GEMM takes the decode GEMV's kernels and workspace; 17-48
    rows the one-pass form: no workspace while K fits one workgroup's 16 waves (one
    group each), else fp32 partials for the group ranges only; 49 rows and more the
    tiled core and its workspace."""
    sz = ctypes.c_size_t(7)
    f = lib.w4a16_gemm
    g = lib.w4a16_gemv
    gz = ctypes.c_size_t(7)
    for M, K, N in ((1, 2048, 300), (16, 17408, 5120), (8, 33792, 64)):
        assert f(None, M, K, N, None, None, None, 1, 128, None, None, ctypes.byref(sz), None) == 0
        assert g(None, M, K, N, None, None, None, 1, 128, None, None, ctypes.byref(gz), None) == 0
        assert sz.value == gz.value, (M, K, N)
    for M, K in ((48, 2048), (17, 128)):
        assert f(None, M, K, 300, None, None, None, 0, 128, None, None, ctypes.byref(sz), None) == 0
        assert sz.value == 0, (M, K)
    # 40 groups: 3 ranges; 136 groups: 9 ranges; 17 groups: 2 ranges
    for M, K, N, splits in ((48, 5120, 17408, 3), (33, 17408, 5120, 9), (17, 2176, 96, 2)):
        assert f(None, M, K, N, None, None, None, 1, 128, None, None, ctypes.byref(sz), None) == 0
        assert sz.value == splits * M * N * 4, (M, K, N)
    # 49 rows: the core's arranged activations (rows rounded to 64), row sums, column
    # words and, with 3 column tiles, the fp32 partials of a 4-way K split (M N
    # rounded up to 64 elements)
    assert f(None, 49, 2048, 300, None, None, None, 1, 128, None, None, ctypes.byref(sz), None) == 0
    assert sz.value == 64 * 2048 * 2 + 16 * 64 * 8 + 16 * 384 * 4 + 4 * 14720 * 4
    # a zero-byte workspace is not required; a nonzero one is
    assert f(A, 48, 5120, 17408, A, A, None, 1, 128, A, None, None, None) == -5


def test_grid_loss_validation(lib):
    sz = ctypes.c_size_t(0)
    f = lib.awq_grid_loss
    assert f(None, 4096, 2048, 6144, None, None, None, None, 20, 0, 128, None, None, ctypes.byref(sz), None) == 0
    with_ref = sz.value
    assert f(None, 4096, 2048, 6144, None, A, None, None, 20, 0, 128, None, None, ctypes.byref(sz), None) == 0
    assert with_ref - sz.value >= 4096 * 6144 * 2        # Y_ref buffer only when not given
    assert f(A, 0, 2048, 64, A, None, A, A, 1, 0, 128, A, A, ctypes.byref(sz), None) == -2
    assert f(A, 8, 2048, 64, A, None, A, A, -1, 0, 128, A, A, ctypes.byref(sz), None) == -2
    assert f(A, 8, 2048, 64, A, None, A, A, 1, 3, 128, A, A, ctypes.byref(sz), None) == -7


def test_search_validation(lib):
    sz = ctypes.c_size_t(0)
    f = lib.awq_search
    D = ctypes.c_double
    al = (D * 20)(*[i / 20 for i in range(20)])
    ra = (D * 10)(*[1 - j / 20 for j in range(10)])
    assert f(None, 4096, 2048, 6144, None, al, 20, ra, 10, 0, 128, None, None, None, None, None,
             ctypes.byref(sz), None) == 0
    assert sz.value > 20 * 6144 * 2048 // 2
    assert f(A, 64, 256, 8, A, al, 0, ra, 10, 0, 128, None, None, None, None, None, ctypes.byref(sz), None) == -7
    bad = (D * 1)(float("nan"))
    assert f(A, 64, 256, 8, A, bad, 1, ra, 10, 0, 128, None, None, None, None, None, ctypes.byref(sz), None) == -7
    badr = (D * 1)(0.0)
    assert f(A, 64, 256, 8, A, al, 20, badr, 1, 0, 128, None, None, None, None, None, ctypes.byref(sz), None) == -7
    assert f(A, 64, 256, 8, A, None, 20, ra, 10, 0, 128, None, None, None, None, None, ctypes.byref(sz), None) == -1
    # the workspace is required: the library allocates nothing of its own
    lo, ia, ir = (ctypes.c_float * 30)(), ctypes.c_int(0), ctypes.c_int(0)
    outs = (lo, ctypes.byref(ia), ctypes.byref(ir), A)
    assert f(A, 64, 256, 8, A, al, 20, ra, 10, 0, 128, *outs, None, None, None) == -5
    assert f(A, 64, 256, 8, A, al, 20, ra, 10, 0, 128, None, None, None, None, None, ctypes.byref(sz), None) == 0
    small = ctypes.c_size_t(sz.value - 1)
    assert f(A, 64, 256, 8, A, al, 20, ra, 10, 0, 128, *outs, A, ctypes.byref(small), None) == -5


def test_clip_search_validation(lib):
    sz = ctypes.c_size_t(0)
    f = lib.awq_clip_search
    assert f(None, 4096, 2048, 6144, None, None, None, 10, 0, 128, None, None, None, ctypes.byref(sz), None) == 0
    G = 2048 // 128
    assert sz.value >= G * 65536 and sz.value <= 64 * 2**20
    big = sz.value
    assert f(None, 64, 2048, 6144, None, None, None, 10, 0, 128, None, None, None, ctypes.byref(sz), None) == 0
    assert sz.value < big                                    # Gram partials scale with the token slices
    ok = ctypes.c_size_t(big)
    args = lambda **k: [k.get("X", A), k.get("T", 64), k.get("K", 2048), k.get("N", 64), k.get("W", A),
                        k.get("s", None), k.get("ratios", A), k.get("R", 10), k.get("sym", 0), k.get("gs", 128),
                        k.get("losses", A), k.get("best", A), k.get("ws", A), ctypes.byref(ok), None]
    assert f(*args(gs=64)) == -4
    assert f(*args(K=200)) == -2
    assert f(*args(T=-1)) == -2
    assert f(*args(R=0)) == -7
    assert f(*args(R=65)) == -7
    assert f(*args(sym=2)) == -7
    assert f(*args(W=None)) == -1
    assert f(*args(best=None)) == -1
    assert f(*args(ratios=None)) == -1
    assert f(*args(X=None)) == -1
    assert f(*args(W=MIS)) == -3
    assert f(*args(s=MIS)) == -3
    assert f(*args(N=0, W=None, best=None)) == 0              # no-op
    small = ctypes.c_size_t(16)
    a = args()
    a[13] = ctypes.byref(small)
    assert f(*a) == -5
    a[13] = None
    assert f(*a) == -5


_Blk = w4._Block          # struct w4_block as the binding declares it


def test_block_and_lookahead_validation(lib):
    sz = ctypes.c_size_t(0)
    blk = _Blk(*([0x10000] * 9))
    bad = _Blk(*([0x10000] * 8 + [0]))
    mis = _Blk(*([0x10000] * 8 + [0x10004]))
    f = lib.w4_block_forward
    assert f(None, 8, 512, 2048, 16, 8, 6144, None, None, None, ctypes.byref(sz), None) == 0
    assert sz.value > 2 * 4096 * (5 * 2048 + 3 * 6144) * 2 // 2
    ok = ctypes.c_size_t(sz.value)
    assert f(A, 8, 512, 2000, 16, 8, 6144, ctypes.byref(blk), A, A, ctypes.byref(ok), None) == -2   # H % 128
    assert f(A, 8, 512, 2048, 16, 6, 6144, ctypes.byref(blk), A, A, ctypes.byref(ok), None) == -2   # n_kv !| n_q
    assert f(A, 0, 512, 2048, 16, 8, 6144, ctypes.byref(blk), A, A, ctypes.byref(ok), None) == -2
    assert f(A, 8, 512, 2048, 16, 8, 6144, ctypes.byref(bad), A, A, ctypes.byref(ok), None) == -1
    assert f(A, 8, 512, 2048, 16, 8, 6144, ctypes.byref(mis), A, A, ctypes.byref(ok), None) == -3
    assert f(A, 8, 512, 2048, 16, 8, 6144, ctypes.byref(blk), A, A, ctypes.byref(ctypes.c_size_t(16)), None) == -5
    g = lib.awq_lookahead_loss
    assert g(None, 8, 512, 2048, 16, 8, 6144, None, None, 6, None, None, 10, 0, 128, None, None, None,
             ctypes.byref(sz), None) == 0
    ok = ctypes.c_size_t(sz.value)
    args = lambda **k: [k.get("X", A), 8, 512, 2048, 16, 8, 6144, ctypes.byref(k.get("blk", blk)), k.get("nxt", None),
                        k.get("lin", 6), k.get("S", A), A, 10, k.get("sym", 0), k.get("gs", 128), A, None, A,
                        ctypes.byref(ok), None]
    assert g(*args(lin=7)) == -7
    assert g(*args(sym=2)) == -7
    assert g(*args(gs=64)) == -4
    assert g(*args(S=None)) == -1
    assert g(*args(blk=bad)) == -1
    assert g(*args(nxt=ctypes.byref(bad))) == -1
    assert g(*args(X=MIS)) == -3
    h = lib.awq_search_lookahead
    D = ctypes.c_double
    al = (D * 20)(*[i / 20 for i in range(20)])
    ra = (D * 10)(*[1 - j / 20 for j in range(10)])
    assert h(None, 8, 512, 2048, 16, 8, 6144, None, None, 0, al, 20, ra, 10, 0, 128, None, None, None, None, None,
             ctypes.byref(sz), None) == 0
    assert sz.value > ok.value // 2
    badr = (D * 1)(1.5)
    assert h(A, 8, 512, 2048, 16, 8, 6144, ctypes.byref(blk), None, 0, al, 20, badr, 1, 0, 128, None, None, None, None,
             None, ctypes.byref(sz), None) == -7
    lo, ia, ir = (ctypes.c_float * 30)(), ctypes.c_int(0), ctypes.c_int(0)
    assert h(A, 8, 512, 2048, 16, 8, 6144, ctypes.byref(blk), None, 0, al, 20, ra, 10, 0, 128, lo, ctypes.byref(ia),
             ctypes.byref(ir), A, None, None, None) == -5


def test_block_forward_quantized_validation(lib):
    sz = ctypes.c_size_t(0)
    blk = _Blk(*([0x10000] * 9))
    bad = _Blk(*([0x10000] * 8 + [0]))
    f = lib.w4_block_forward_quantized
    assert f(None, 8, 512, 2048, 16, 8, 6144, None, 6, None, None, None, None, 0, 128, None, None, ctypes.byref(sz),
             None) == 0
    base = ctypes.c_size_t(0)
    assert lib.w4_block_forward(None, 8, 512, 2048, 16, 8, 6144, None, None, None, ctypes.byref(base), None) == 0
    assert sz.value > base.value + 2 * 4096 * 6144      # plus bf16(a / s) of the down projection's input
    ok = ctypes.c_size_t(sz.value)
    args = lambda **k: [k.get("X", A), 8, 512, 2048, 16, 8, 6144, ctypes.byref(k.get("blk", blk)), k.get("lin", 6),
                        k.get("s", A), k.get("qw", A), A, k.get("qz", A), k.get("sym", 0), k.get("gs", 128),
                        k.get("Y", A), A, ctypes.byref(k.get("ws", ok)), None]
    assert f(*args(lin=-1)) == -7
    assert f(*args(sym=3)) == -7
    assert f(*args(gs=32)) == -4
    assert f(*args(s=None)) == -1
    assert f(*args(qw=None)) == -1
    assert f(*args(sym=1)) == -1                 # qzeros must be NULL when symmetric
    assert f(*args(qz=None)) == -1
    assert f(*args(blk=bad)) == -1
    assert f(*args(Y=MIS)) == -3
    assert f(*args(ws=ctypes.c_size_t(64))) == -5


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(w4, "_LIB", None)
    monkeypatch.setattr(w4, "_HERE", str(tmp_path))
    with pytest.raises(RuntimeError, match="missing"):
        w4.load_library()
