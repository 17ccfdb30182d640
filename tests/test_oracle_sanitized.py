"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) runs the whole pin suite: any out-of-bounds access,
use after free, signed overflow, bad shift or misaligned load in the C
oracle aborts the run."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _gcc_file(name):
    try:
        p = subprocess.check_output(["gcc", f"-print-file-name={name}"], text=True).strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_pins_under_asan_ubsan(tmp_path):
    asan = _gcc_file("libasan.so")
    if asan is None:
        pytest.skip("gcc has no libasan")
    so = str(tmp_path / "libmoe_oracle_san.so")
    subprocess.check_call(
        ["gcc", "-O1", "-g", "-fPIC", "-shared", "-std=c99", "-fno-fast-math",
         "-ffp-contract=off", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", so,
         "-lm"])
    env = dict(os.environ)
    env.update({
        "MOE_ORACLE_SO": so,
        "LD_PRELOAD": asan,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
         os.path.join(HERE, "test_oracle_pins.py"), os.path.join(HERE, "test_oracle_numpy.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "error" not in r.stdout.lower(), tail
