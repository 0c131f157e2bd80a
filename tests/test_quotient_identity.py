"""The device quantizer computes fl32(x / s) as q0 = x*r, e = fma(-q0, s, x),
q = fma(e, r, q0) with r = fl32(1/s) (Markstein's correction step).  These
tests check on the CPU (C, IEEE binary32 with a real fma) that this equals the
correctly rounded quotient for every bf16 and fp16 input significand against a
sample of fp32 divisor significands, including the all-ones and power-of-two
ones.  (The full 2^23 sweep, run once with the same program, found no
mismatch; it takes minutes, so the suite samples.)  On the device q0 is first
clamped to [-896, 896], the result takes the sign of x and is clamped to
[-448, 448] before the E4M3 converter.  A second sweep takes every non-NaN
16-bit input pattern (infinities included) against divisors over the whole
range the device uses the routine for (2^-80 .. 2^120), so quotients overflow
binary32 and underflow to subnormals, and compares the E4M3 codes (round to
nearest even, saturating at +-448) of that routine's result and of the IEEE
quotient.
Codes on the GPU are checked bit-exactly against the oracle's IEEE division
by the GPU tests."""
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
    out = subprocess.run([exe, "id", str(xbits), str(first), str(count), str(step)],
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


def _sat(exe, fmt, e_lo, e_hi, first, count, step):
    out = subprocess.run([exe, "sat", fmt, str(e_lo), str(e_hi), str(first), str(count),
                          str(step)], check=True, capture_output=True, text=True).stdout.split()
    return int(out[0]), int(out[1]), int(out[2])


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
def test_saturated_quotient_over_the_whole_divisor_range(checker, fmt):
    # every input pattern against 4 divisor significands (1.0, the all-ones
    # one and two in between) at each power of two in [2^-80, 2^119]; the
    # codes must agree everywhere
    nan_patterns = 2 * 127 if fmt == "bf16" else 2 * 1023
    for first, count, step in ((0, 2, 0x7fffff), (0x2aaaab, 2, 0x2aaaab)):
        total, bad, _ = _sat(checker, fmt, -80, 119, first, count, step)
        assert total == 200 * count * (65536 - nan_patterns) and bad == 0


def test_overflowing_quotients_need_the_guard(checker):
    # bf16 inputs reach 2^128, so with s <= 2^-1 the product x * r overflows
    # for the largest ones: applying the correction step there turns the
    # infinite product into NaN (x - inf * s = -inf, then -inf * r + inf),
    # which the clamp of q0 avoids.  fp16 inputs (at most 65504, or infinite) show
    # the same for infinite inputs.
    for fmt in ("bf16", "fp16"):
        total, bad, bad_unguarded = _sat(checker, fmt, -80, -1, 0, 3, 0x155555)
        assert bad == 0 and bad_unguarded > 0, (fmt, total, bad, bad_unguarded)
