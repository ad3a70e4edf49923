"""The dynamic quantizers' reciprocal division equals IEEE x / s.

The quantization cast of the pages divides each element by the per-tensor
scale (amax / 448) before the E4M3 rounding. The GPU quantizers form that
quotient from a reciprocal and one fma correction; this test enumerates
every scale a 16-bit input can produce and every input it divides, on the
CPU, and requires the quotient bits to equal the IEEE division's.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("divcheck") / "scale_division_check")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", "-std=c11",
                    os.path.join(HERE, "scale_division_check.c"), "-o", exe, "-lm"], check=True)
    return exe


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_reciprocal_quotient_is_ieee(checker, fmt):
    out = subprocess.run([checker, fmt], capture_output=True, text=True, timeout=600)
    print(out.stdout)
    assert out.returncode == 0, out.stdout
    assert " 0 differ" in out.stdout
