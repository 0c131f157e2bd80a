"""Pins for the oracle's E4M3 upper-byte NestedFP split (CPU only).

The NestedFP page (§2.1) also names E4M3 as the upper byte's format; the reading (an
fp16 word with a clear top exponent bit keeps sign + 4 exponent + 3 mantissa
bits in the upper byte, and the freed bit with the 7 low mantissa bits in the
lower byte) is fixed here against numpy over all 65,536 fp16 words:
- the rebuild returns every word bit for bit;
- for finite |w| < 1.875 the upper byte read as E4M3 (torch's float8_e4m3fn,
  a library routine) times 2^-8 is w with its 7 low mantissa bits cleared
  (truncation toward zero), subnormals included;
- the count of words outside that range is numpy's count;
- the fp16-output FP8 GEMM equals exact integer results on small integers.
"""
import numpy as np
import torch

import oracle

ALL = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def test_rebuild_is_exact_for_every_word():
    hi, lo, _ = oracle.nested_split_e4m3(ALL)
    assert np.array_equal(oracle.nested_rebuild_e4m3(hi, lo), ALL)


def test_upper_byte_is_the_e4m3_truncation():
    hi, lo, bad = oracle.nested_split_e4m3(ALL)
    w = ALL.view(np.float16).astype(np.float64)
    ok = np.isfinite(w) & (np.abs(w) < 1.875)
    assert bad == int((~ok).sum())
    e4m3 = torch.from_numpy(hi[ok].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    trunc = (ALL[ok] & np.uint16(0xFF80)).view(np.float16).astype(np.float64)
    assert np.array_equal(e4m3 * 2.0 ** -8, trunc)
    assert not np.any((hi[ok] & 0x7F) == 0x7F)           # never the NaN code
    # the subnormal fp16 range maps onto E4M3 subnormals
    sub = ok & (np.abs(w) < 2.0 ** -14) & (w != 0)
    assert np.all(((hi[sub] >> 3) & 0xF) == 0)


def test_fp16out_gemm_small_integers_exact():
    rng = np.random.Generator(np.random.PCG64(3))
    M, N, K = 3, 21, 96
    a = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    w = rng.integers(-8, 9, size=(N, K)).astype(np.float32)
    y = oracle.gemm_fp8_f32_fp16out(oracle.e4m3_encode(a), 1.0, oracle.e4m3_encode(w), 0.25)
    exact = (a.astype(np.int64) @ w.astype(np.int64).T).astype(np.float64) * 0.25
    assert np.array_equal(y, oracle.f16_encode(exact.astype(np.float32)))


def test_e4m3_upper_byte_never_worse_than_e5m2():
    """One more mantissa bit: for every fp16 word in range the FP8-mode value of
    the E4M3 split is at least as close to w as the plain split's E5M2 value."""
    hi4, _, _ = oracle.nested_split_e4m3(ALL)
    hi5, _ = oracle.nested_split(ALL)
    w = ALL.view(np.float16).astype(np.float64)
    ok = np.isfinite(w) & (np.abs(w) < 1.875)
    v4 = torch.from_numpy(hi4[ok].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy() * 2.0 ** -8
    v5 = oracle.e5m2_decode(hi5[ok])
    assert np.all(np.abs(w[ok] - v4) <= np.abs(w[ok] - v5))
    assert np.sum(np.abs(w[ok] - v4) < np.abs(w[ok] - v5)) > ok.sum() // 3
