"""w4a16_gemv_noalloc (the allocation-free decode GEMV) through the C ABI against
w4a16_gemv on the same inputs: bit-identical outputs (same kernels, fixed
summation order), on two calls in a row -- the second with a smaller problem,
so it runs on the static scratch the first call left behind -- covering the K
split (the path that uses the scratch) and a shape without one."""
import numpy as np
import pytest
import torch

import weight_only_int4_amd as w4
import workloads as wl
from oracle import w4a16_oracle as O
from tests.gpu_util import bits16, gpu_available, say, to_bf16, to_i32

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def _case(M, K, N, sym, seed):
    X, W = wl.small_case(M, K, N, seed)
    qw, sc, qz = O.quantize_pack(W, None, 1.0, sym)
    return to_bf16(X), to_i32(qw), to_bf16(sc), None if sym else to_i32(qz)


@pytest.mark.parametrize("sym", [False, True])
def test_gemv_noalloc_matches_gemv(sym):
    # (M, K, N): K split in 3 with 16 rows (partials 16 x 1500 x 3 fp32), then a
    # smaller problem split in 2 (1 row), then one without a split
    for M, K, N in ((16, 17408, 1500), (1, 33792, 96), (4, 2048, 300)):
        say("gemv noalloc", M, K, N, sym)
        X, qw, sc, qz = _case(M, K, N, sym, 7 + M)
        Y0 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        w4.w4a16_gemv_noalloc(X, qw, sc, qz, sym, Y0)
        Y1 = w4.w4a16_gemv(X, qw, sc, qz, sym)
        torch.cuda.synchronize()
        assert not torch.isnan(Y0.float()).any()
        assert np.array_equal(bits16(Y0), bits16(Y1)), (M, K, N)


def test_gemv_noalloc_rejects_oversized():
    X, qw, sc, _ = _case(16, 17408, 8, True, 3)
    qwb = torch.zeros((50000, 17408 // 8), dtype=torch.int32, device="cuda")
    scb = torch.zeros((50000, 17408 // 128), dtype=torch.bfloat16, device="cuda")
    Y = torch.empty((16, 50000), dtype=torch.bfloat16, device="cuda")
    say("gemv noalloc oversized")
    with pytest.raises(w4.W4Error, match="SCRATCH"):
        w4.w4a16_gemv_noalloc(X, qwb, scb, None, True, Y)
