"""The int8 quantiser replaces the per-element fp32 division by one FMA
correction step and forms the rounded code with one add; the per-group FP8
quantiser uses the same step and rounds the binary32 bits to E4M3 with
integer arithmetic. tests/quant_division_check.c
verifies, for every pair of 16-bit token values (x, amax) a row can hold, that
the code is the one the correctly rounded division gives (the reading of
quantMode 2 in aclnnMoeDistributeDispatchV4 that the oracle implements), that
it never leaves [-127, 127], and that the add's low byte is that code."""
import os
import re
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("qdiv") / "quant_division_check")
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-o", exe,
                           os.path.join(HERE, "quant_division_check.c"), "-lm"])
    return exe


@pytest.mark.parametrize("fmt,pairs_min", [("bf16", 10 ** 9), ("fp16", 10 ** 9)])
def test_fast_quotient_rounds_like_the_division_for_every_16bit_pair(checker, fmt, pairs_min):
    out = subprocess.run([checker, fmt], stdout=subprocess.PIPE, text=True, timeout=600)
    m = re.search(r"pairs=(\d+) integer_mismatches=(\d+) quotient_mismatches=\d+ out_of_range=(\d+) "
                  r"byte_mismatches=(\d+)", out.stdout)
    assert m, out.stdout
    assert int(m.group(1)) >= pairs_min
    assert int(m.group(2)) == 0 and int(m.group(3)) == 0 and int(m.group(4)) == 0, out.stdout
    assert out.returncode == 0


@pytest.mark.parametrize("fmt,pairs_min", [("bf16", 10 ** 9), ("fp16", 10 ** 9)])
def test_fast_quotient_gives_the_e4m3_code_of_the_division_for_every_16bit_pair(checker, fmt, pairs_min):
    """quantMode 3 (per-group, scale = amax / 448): every code equals the E4M3
    value nearest to the correctly rounded, clamped quotient."""
    out = subprocess.run([checker, fmt, "e4m3"], stdout=subprocess.PIPE, text=True, timeout=600)
    m = re.search(r"pairs=(\d+) code_mismatches=(\d+)", out.stdout)
    assert m, out.stdout
    assert int(m.group(1)) >= pairs_min
    assert int(m.group(2)) == 0, out.stdout
    assert out.returncode == 0
