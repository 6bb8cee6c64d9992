"""The quantization and clip-search kernels take their codes from v / scale
computed as fma(fma(-scale, q0, v), 1/scale, q0) with q0 = v * (1/scale); this must
equal the IEEE quotient that the oracle divides with.  Checked exhaustively (every bf16 scale
significand x every fp32 significand) by a small C program compiled here."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_fma_corrected_quotient_equals_ieee_division(tmp_path):
    exe = str(tmp_path / "division_check")
    # -ffp-contract=off: the multiply q0 = a * y must stay a separate rounding, as in the kernel
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-o", exe,
                    os.path.join(HERE, "division_check.c"), "-lm"], check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "mismatches 0" in res.stdout
    assert "checked 1073741824 pairs" in res.stdout
