"""The fused RMSNorm quantizers' division equals IEEE fp32 y / s.

They divide by the scale as fp32(fp64(y * fp64(1/s))); fp64_quotient_check.c
states why that is the IEEE quotient in the fp32 normal range and tests it on
the CPU over random, quantizer-range, near-boundary and subnormal pairs.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_fp64_product_quotient_is_ieee(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "fp64_quotient_check")
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11",
                    os.path.join(HERE, "fp64_quotient_check.c"), "-o", exe, "-lm"], check=True)
    out = subprocess.run([exe, "4000000"], capture_output=True, text=True, timeout=600)
    print(out.stdout)
    assert out.returncode == 0, out.stdout
    assert " 0 differ" in out.stdout
