"""The requantiser forms w/s without a divide (one residual step from the
correctly rounded reciprocal).  Only the integer code matters; this host
check shows that the step gives the IEEE quotient's code everywhere it
could differ: every divisor significand, every dividend within 24 ulps of a
code boundary.  The device kernel itself is checked code by code against
the oracle's IEEE division in the GPU parity tests."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(__file__)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_one_step_quotient_gives_ieee_codes(tmp_path):
    exe = tmp_path / "quotient_check"
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-pthread",
                    os.path.join(HERE, "quotient_check.c"), "-o", str(exe), "-lm"], check=True)
    threads = str(max(1, min(8, os.cpu_count() or 1)))
    r = subprocess.run([str(exe), threads], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    fields = dict(zip(r.stdout.split()[0::2], map(int, r.stdout.split()[1::2])))
    assert fields["cases"] == (1 << 23) * 12 * 2 * 49
    assert r.returncode == 0 and fields["code_mismatches"] == 0
