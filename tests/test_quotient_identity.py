"""The device quantizer computes fl32(x / s) as q0 = x*r, e = fma(-q0, s, x),
q = fma(e, r, q0) with r = fl32(1/s) (Markstein's correction step).  These
tests check on the CPU (C, IEEE binary32 with a real fma) that this equals the
correctly rounded quotient for every bf16 and fp16 input significand against
a sample of fp32 divisor significands, including the all-ones and power-of-two
ones.  (The full 2^23 sweep, run once with the same program, found no
mismatch; it takes minutes, so the suite samples.)  Codes on the GPU are
checked bit-exactly against the oracle's IEEE division by the GPU tests."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("quotient") / "quotient_check")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                    os.path.join(HERE, "csrc", "quotient_check.c"), "-o", exe, "-lm"],
                   check=True)
    return exe


def _run(exe, xbits, first, count, step):
    out = subprocess.run([exe, str(xbits), str(first), str(count), str(step)],
                         check=True, capture_output=True, text=True).stdout.split()
    return int(out[0]), int(out[1])


@pytest.mark.parametrize("xbits", [8, 11])
def test_edges_of_the_divisor_range(checker, xbits):
    # the first and last 4096 significands (s = 1 and s just below 2)
    for first in (0, (1 << 23) - 4096):
        total, bad = _run(checker, xbits, first, 4096, 1)
        assert total == 4096 * (1 << xbits) and bad == 0


@pytest.mark.parametrize("xbits", [8, 11])
def test_strided_sample_of_divisors(checker, xbits):
    # 8192 divisor significands spread over the whole range (odd stride)
    total, bad = _run(checker, xbits, 12345, 8192, 1021)
    assert total == 8192 * (1 << xbits) and bad == 0
