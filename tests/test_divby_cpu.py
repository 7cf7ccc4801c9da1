"""The corrected reciprocal product the quantizers divide the block maximum
by 6 and 7 with (div_by in the kernels' header) equals the IEEE quotient for
every finite fp32 a >= 2^-119: checked here on the CPU with C's fmaf, and on
the device, with the kernels' own function, by tests/test_gpu_converters.py."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.slow
def test_div_by_6_and_7_every_finite(tmp_path):
    exe = str(tmp_path / "divby")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                    os.path.join(HERE, "cpu", "divby_exhaustive.c"), "-o", exe, "-lm"], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=600).stdout.split()
    b6, f6, b7, f7 = (int(v) for v in out)
    assert b6 == 0, f"{b6} quotients a / 6 differ, first a bits {f6:#010x}"
    assert b7 == 0, f"{b7} quotients a / 7 differ, first a bits {f7:#010x}"
