"""Pins for the oracle's per-token / per-channel functions (CPU only).

Per-row scales are the per-token and per-channel options of the TensorRT-LLM
build on the page "C++与FP8量化" (§4.2).  What fixes the oracle here:
- each row of quantize_rows equals a library-routine quantizer (numpy max,
  IEEE binary32 division, torch's float8_e4m3fn cast) applied to that row;
- scaling a row by 2^e leaves its codes unchanged and scales its amax and
  scale by exactly 2^e (closed form: the quotient x/s is unchanged);
- the row-scaled GEMM checker equals brute force in exact rationals;
- with power-of-two scales 2^a[m], 2^b[n], the row-scaled fp32 GEMM equals the
  unit-scale GEMM times 2^(a[m]+b[n]) bit for bit (exact bf16 scaling), so a
  transposed or swapped scale index fails;
- small-integer operands give exact integer sums.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from fp8_quantized_gemm_amd import synth


def _lib_quantize_row(v: np.ndarray):
    """Quantizer of one row written with library routines only."""
    amax = np.float32(np.max(np.abs(v))) if v.size else np.float32(0)
    s = np.float32(amax) / np.float32(448.0) if amax > 0 else np.float32(1.0)
    t = (v / s).astype(np.float32)
    assert np.all(np.abs(t) < 464.0)          # within one ulp of 448: rounds to 448
    codes = torch.from_numpy(t.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, s, amax


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("rows,cols,outliers", [(1, 64, False), (5, 1000, True), (3, 11008, True)])
def test_quantize_rows_matches_library_per_row(dtype, rows, cols, outliers):
    x = synth.activation(rows, cols, seed=synth.seed_for("qr", rows, cols, dtype), dtype=dtype,
                         outliers=outliers)
    code = oracle.BF16 if dtype == "bf16" else oracle.FP16
    q, s, a = oracle.quantize_rows(synth.bits(x), code)
    v = x.to(torch.float32).numpy()
    for r in range(rows):
        q2, s2, a2 = _lib_quantize_row(v[r])
        assert np.array_equal(q[r], q2), f"row {r}"
        assert s[r] == s2 and a[r] == a2


def test_quantize_rows_power_of_two_invariance():
    """Row r = row 0 * 2^e[r]: identical codes, amax and scale times 2^e[r]."""
    base = synth.activation(1, 512, seed=9, outliers=True).to(torch.float32)
    e = np.array([0, 3, -5, 7, -2])
    x = torch.cat([base * float(2.0 ** k) for k in e]).to(torch.bfloat16)
    q, s, a = oracle.quantize_rows(synth.bits(x), oracle.BF16)
    for r, k in enumerate(e):
        assert np.array_equal(q[r], q[0])
        assert a[r] == np.float32(a[0] * 2.0 ** k)
        assert s[r] == np.float32(s[0] * 2.0 ** k)


def test_quantize_rows_zero_row_and_single_row():
    x = torch.zeros((3, 32), dtype=torch.bfloat16)
    x[1] = -0.0
    x[2, 5] = 3.0
    q, s, a = oracle.quantize_rows(synth.bits(x), oracle.BF16)
    assert list(s[:2]) == [1.0, 1.0] and list(a[:2]) == [0.0, 0.0]
    assert np.all(q[0] == 0x00) and np.all(q[1] == 0x80)
    assert q[2, 5] == 0x7E and s[2] == np.float32(3.0) / np.float32(448.0)
    # one row is the per-tensor quantizer
    x1 = synth.activation(1, 4096, seed=4, outliers=True)
    q1, s1, a1 = oracle.quantize_rows(synth.bits(x1), oracle.BF16)
    qt, st, at = oracle.quantize(synth.bits(x1).ravel(), oracle.BF16)
    assert np.array_equal(q1.ravel(), qt) and (s1[0], a1[0]) == (st, at)


def _frac_codes_e4m3(c):
    return [Fraction(float(v)) for v in oracle.e4m3_decode(np.ascontiguousarray(c).ravel())]


def _random_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3F  # no NaN codes
    return c


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 5), (3, 4, 8), (4, 2, 6)])
def test_rowwise_ref_exact_against_fractions(M, N, K):
    rng = np.random.Generator(np.random.PCG64(M * 100 + N * 10 + K + 7))
    qa = _random_codes(rng, (M, K))
    qw = _random_codes(rng, (N, K))
    sa = (rng.integers(1, 64, M) / 64.0).astype(np.float32)
    sw = (rng.integers(1, 64, N) / 128.0).astype(np.float32)
    ref, ab = oracle.gemm_fp8_rowwise_ref(qa, sa, qw, sw)
    A, W = _frac_codes_e4m3(qa), _frac_codes_e4m3(qw)
    for m in range(M):
        for n in range(N):
            sc = Fraction(float(sa[m])) * Fraction(float(sw[n]))
            exact = sum(A[m * K + k] * W[n * K + k] for k in range(K)) * sc
            exact_abs = sum(abs(A[m * K + k] * W[n * K + k]) for k in range(K)) * sc
            assert Fraction(ref[m * N + n]) == exact
            assert Fraction(ab[m * N + n]) == exact_abs


def test_rowwise_ref_pairs_subset_and_constant_scales():
    rng = np.random.Generator(np.random.PCG64(5))
    qa = _random_codes(rng, (6, 48))
    qw = _random_codes(rng, (7, 48))
    sa = np.full(6, 0.5, np.float32)
    sw = np.full(7, 2.0, np.float32)
    full, fab = oracle.gemm_fp8_rowwise_ref(qa, sa, qw, sw)
    per_tensor, pab = oracle.gemm_fp8_ref(qa, 0.5, qw, 2.0)
    assert np.array_equal(full, per_tensor) and np.array_equal(fab, pab)
    ms, ns = np.array([5, 0, 3]), np.array([6, 2, 0])
    sub, _ = oracle.gemm_fp8_rowwise_ref(qa, sa * np.arange(1, 7, dtype=np.float32), qw, sw, ms, ns)
    whole, _ = oracle.gemm_fp8_rowwise_ref(qa, sa * np.arange(1, 7, dtype=np.float32), qw, sw)
    assert np.array_equal(sub, whole.reshape(6, 7)[ms, ns])


def test_rowwise_f32_power_of_two_scales_exact():
    """With sa[m] = 2^a[m] and sw[n] = 2^b[n] the output is the unit-scale
    output times 2^(a[m] + b[n]), bit for bit."""
    rng = np.random.Generator(np.random.PCG64(17))
    M, N, K = 7, 11, 300
    qa = _random_codes(rng, (M, K))
    qw = _random_codes(rng, (N, K))
    a = rng.integers(-6, 7, M)
    b = rng.integers(-9, 4, N)
    sa = (2.0 ** a).astype(np.float32)
    sw = (2.0 ** b).astype(np.float32)
    y = oracle.gemm_fp8_rowwise_f32(qa, sa, qw, sw)
    unit = oracle.bf16_decode(oracle.gemm_fp8_f32(qa, 1.0, qw, 1.0)).astype(np.float64)
    want = oracle.bf16_encode((unit * 2.0 ** (a[:, None] + b[None, :])).astype(np.float32))
    assert np.array_equal(y, want)


def test_rowwise_f32_small_integers_exact():
    rng = np.random.Generator(np.random.PCG64(23))
    M, N, K = 4, 29, 160
    a = rng.integers(-16, 17, size=(M, K)).astype(np.float32)
    w = rng.integers(-16, 17, size=(N, K)).astype(np.float32)
    qa = oracle.e4m3_encode(a)
    qw = oracle.e4m3_encode(w)
    sa = np.array([1.0, 0.5, 2.0, 0.25], np.float32)
    sw = np.ones(N, np.float32)
    y = oracle.gemm_fp8_rowwise_f32(qa, sa, qw, sw)
    exact = (a.astype(np.int64) @ w.astype(np.int64).T).astype(np.float64) * sa[:, None]
    assert np.array_equal(y, oracle.bf16_encode(exact.astype(np.float32)))
