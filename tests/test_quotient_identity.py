"""The quantizers form x / scale from a reciprocal and one fused-multiply-add
correction instead of a division.  This host check (gcc, correctly rounded
fmaf) shows that the int8 and e4m3fn codes equal those of the correctly
rounded quotient: for every 16-bit input against (every 7th of) the scales a
16-bit amax can produce, and on random fp32 scales with inputs on and next to
the rounding boundaries."""
import os
import shutil
import subprocess

import pytest

SRC = os.path.join(os.path.dirname(__file__), "csrc", "quotient_check.c")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("qc") / "quotient_check")
    subprocess.run([cc, "-O2", "-march=native", "-ffp-contract=off", "-o", exe, SRC, "-lm"], check=True)
    return exe


def test_every_16bit_input(checker):
    # every input against every 7th possible scale; "quotient_check exhaustive 1"
    # runs all of them (about 90 s)
    r = subprocess.run([checker, "exhaustive", "7"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count(": 0 code mismatches") == 4, r.stdout


def test_random_fp32_scales(checker):
    r = subprocess.run([checker, "random", "50000000"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
