"""Pins for the oracle's quantizer, NestedFP split and GEMM checkers (CPU only).

The quantizer is pinned against numpy (max of |x|, IEEE binary32 division) and
torch's float8_e4m3fn cast; the split against its invariants over all 65,536
fp16 words; the GEMM checkers against brute force in exact rational
arithmetic (fractions.Fraction) on tiny shapes, and the fp32 GEMMs against
exact integer results and the fp64 checker.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from fp8_quantized_gemm_amd import synth


def _np_f32(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float32).numpy()


def _lib_quantize(x: torch.Tensor):
    """Quantizer written with library routines only."""
    v = _np_f32(x).ravel()
    amax = np.float32(np.max(np.abs(v))) if v.size else np.float32(0)
    s = np.float32(amax) / np.float32(448.0) if amax > 0 else np.float32(1.0)
    t = (v / s).astype(np.float32)
    codes = torch.from_numpy(t.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch does not saturate; |t| <= 448 up to one ulp of the division, which
    # rounds to 448 anyway, so no clamp is needed here.
    assert np.all(np.abs(t) < 464.0)
    return codes, float(s), float(amax)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("shape,outliers", [((1, 4096), False), ((4, 1000), False),
                                            ((8, 11008), True), ((3, 17), True)])
def test_quantize_matches_library(dtype, shape, outliers):
    x = synth.activation(*shape, seed=synth.seed_for("q", shape, dtype), dtype=dtype,
                         outliers=outliers)
    code = oracle.BF16 if dtype == "bf16" else oracle.FP16
    q, s, a = oracle.quantize(synth.bits(x).ravel(), code)
    q2, s2, a2 = _lib_quantize(x)
    assert a == a2
    assert np.float32(s).view(np.uint32) == np.float32(s2).view(np.uint32)
    assert np.array_equal(q, q2)


def test_quantize_weights_fp16():
    w = synth.normal((64, 512), 0.02, "fp16", seed=synth.seed_for("w"))
    q, s, a = oracle.quantize(synth.bits(w).ravel(), oracle.FP16)
    q2, s2, a2 = _lib_quantize(w)
    assert (a, s) == (a2, s2)
    assert np.array_equal(q, q2)
    # the largest-magnitude element maps to +-448 exactly
    i = int(np.argmax(np.abs(_np_f32(w).ravel())))
    assert q[i] & 0x7F == 0x7E


def test_quantize_zero_and_degenerate():
    z = np.zeros(37, np.uint16)
    q, s, a = oracle.quantize(z, oracle.BF16)
    assert (s, a) == (1.0, 0.0) and not q.any()
    negz = np.full(5, 0x8000, np.uint16)
    q, s, a = oracle.quantize(negz, oracle.BF16)
    assert (s, a) == (1.0, 0.0) and np.all(q == 0x80)
    one = synth.bits(torch.tensor([-3.5], dtype=torch.bfloat16))
    q, s, a = oracle.quantize(one, oracle.BF16)
    assert a == 3.5 and q[0] == 0xFE             # -amax -> -448


def test_quantize_identity_scale_when_amax_is_448():
    # amax == 448 -> s == 1 exactly, so codes are the plain E4M3 encodings
    vals = np.array([448.0, -1.0625, 17.0, 2.0 ** -10, 3 * 2.0 ** -10, 0.3], np.float32)
    x = synth.bits(torch.from_numpy(vals).to(torch.float16))
    q, s, a = oracle.quantize(x, oracle.FP16)
    assert s == 1.0 and a == 448.0
    back = torch.from_numpy(vals).to(torch.float16).to(torch.float32).numpy()
    assert np.array_equal(q, oracle.e4m3_encode(back))


# ----------------------------------------------------------------- NestedFP split
def test_split_rebuild_exhaustive():
    w = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    hi, lo = oracle.nested_split(w)
    assert np.array_equal(oracle.nested_rebuild(hi, lo), w)
    # every (hi, lo) pair appears exactly once
    assert len(set(zip(hi.tolist(), lo.tolist()))) == 65536


def test_split_fp8_mode_value_is_truncation():
    """FP8-mode weight = E5M2(upper byte): |w| rounded toward zero to 2 mantissa
    bits, same sign, error below one E5M2 ulp of |w|."""
    w = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    hi, _ = oracle.nested_split(w)
    full = w.view(np.float16).astype(np.float64)
    fp8 = oracle.e5m2_decode(hi)
    fin = np.isfinite(full)
    f, g = full[fin], fp8[fin]
    assert np.all(np.abs(g) <= np.abs(f))
    assert np.all((np.signbit(g) == np.signbit(f)))
    # one E5M2 ulp at |w|: 2^(max(e,-14) - 2)
    e = np.floor(np.log2(np.where(f == 0, 1.0, np.abs(f))))
    ulp = np.exp2(np.maximum(e, -14) - 2)
    assert np.all(np.abs(f) - np.abs(g) < ulp)


# ----------------------------------------------------------------- GEMM checkers
def _frac_codes_e4m3(c):
    return [Fraction(float(v)) for v in
            torch.from_numpy(np.ascontiguousarray(c, np.uint8).ravel()).view(torch.float8_e4m3fn)
            .to(torch.float64).numpy()]


def _frac_codes_e5m2(c):
    return [Fraction(float(v)) for v in
            torch.from_numpy(np.ascontiguousarray(c, np.uint8).ravel()).view(torch.float8_e5m2)
            .to(torch.float64).numpy()]


def _frac_half(h):
    return [Fraction(float(v)) for v in np.ascontiguousarray(h, np.uint16).ravel()
            .view(np.float16).astype(np.float64)]


def _random_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3F  # no NaN codes
    return c


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (1, 3, 5), (2, 5, 3), (3, 2, 8), (4, 7, 6)])
def test_fp8_ref_exact_against_fractions(M, N, K):
    rng = np.random.Generator(np.random.PCG64(M * 100 + N * 10 + K))
    qa = _random_codes(rng, (M, K))
    qw = _random_codes(rng, (N, K))
    sa, sw = np.float32(0.375), np.float32(1.25)
    ref, ab = oracle.gemm_fp8_ref(qa, float(sa), qw, float(sw))
    A = _frac_codes_e4m3(qa)
    W = _frac_codes_e4m3(qw)
    sc = Fraction(float(sa)) * Fraction(float(sw))
    for m in range(M):
        for n in range(N):
            exact = sum(A[m * K + k] * W[n * K + k] for k in range(K)) * sc
            exact_abs = sum(abs(A[m * K + k] * W[n * K + k]) for k in range(K)) * sc
            assert Fraction(ref[m * N + n]) == exact        # transposition or index slip fails
            assert Fraction(ab[m * N + n]) == exact_abs


def test_fp8_ref_pairs_subset():
    rng = np.random.Generator(np.random.PCG64(3))
    qa = _random_codes(rng, (5, 32))
    qw = _random_codes(rng, (9, 32))
    full, fab = oracle.gemm_fp8_ref(qa, 0.5, qw, 2.0)
    ms = np.array([4, 0, 2])
    ns = np.array([8, 1, 5])
    sub, sab = oracle.gemm_fp8_ref(qa, 0.5, qw, 2.0, ms, ns)
    assert np.array_equal(sub, full.reshape(5, 9)[ms, ns])
    assert np.array_equal(sab, fab.reshape(5, 9)[ms, ns])


@pytest.mark.parametrize("M,N,K", [(1, 2, 3), (3, 4, 5), (2, 3, 8)])
def test_nested_refs_against_fractions(M, N, K):
    rng = np.random.Generator(np.random.PCG64(K))
    a16 = synth.bits(synth.normal((M, K), 1.0, "fp16", seed=K))
    w16 = synth.bits(synth.normal((N, K), 0.02, "fp16", seed=K + 1))
    hi, lo = oracle.nested_split(w16)
    ref, ab = oracle.nested_fp16_ref(a16, hi, lo)
    A, Wf = _frac_half(a16), _frac_half(w16)
    for m in range(M):
        for n in range(N):
            exact = sum(A[m * K + k] * Wf[n * K + k] for k in range(K))
            assert abs(Fraction(ref[m * N + n]) - exact) <= Fraction(1, 2**50) * (
                sum(abs(A[m * K + k] * Wf[n * K + k]) for k in range(K)))
    qa = _random_codes(rng, (M, K))
    sa = np.float32(0.0078125)
    ref8, _ = oracle.nested_fp8_ref(qa, float(sa), hi)
    A8, H8 = _frac_codes_e4m3(qa), _frac_codes_e5m2(hi)
    for m in range(M):
        for n in range(N):
            exact = sum(A8[m * K + k] * H8[n * K + k] for k in range(K)) * Fraction(float(sa))
            assert Fraction(ref8[m * N + n]) == exact


# ----------------------------------------------------------------- fp32 GEMMs
def _small_int_operands(rng, M, N, K):
    """Integer activations/weights in [-16, 16] plus one 448 each (exact in E4M3)."""
    a = rng.integers(-16, 17, size=(M, K)).astype(np.float32)
    w = rng.integers(-16, 17, size=(N, K)).astype(np.float32)
    a.flat[rng.integers(a.size)] = 448.0
    w.flat[rng.integers(w.size)] = 448.0
    return a, w


def test_fp8_f32_small_integers_exact():
    rng = np.random.Generator(np.random.PCG64(11))
    M, N, K = 5, 37, 160
    a, w = _small_int_operands(rng, M, N, K)
    xa = synth.bits(torch.from_numpy(a).to(torch.bfloat16))
    xw = synth.bits(torch.from_numpy(w).to(torch.float16))
    qa, sa, _ = oracle.quantize(xa, oracle.BF16)
    qw, sw, _ = oracle.quantize(xw, oracle.FP16)
    assert sa == 1.0 and sw == 1.0
    y = oracle.gemm_fp8_f32(qa.reshape(M, K), sa, qw.reshape(N, K), sw)
    exact = a.astype(np.int64) @ w.astype(np.int64).T
    want = synth.bits(torch.from_numpy(exact.astype(np.float64)).to(torch.bfloat16))
    assert np.array_equal(y, want.reshape(M, N))


@pytest.mark.parametrize("threads", [1, 3])
def test_fp8_f32_within_tolerance_of_ref(threads):
    M, N, K = 3, 50, 4096
    x = synth.activation(M, K, seed=5)
    w = synth.normal((N, K), 0.02, "fp16", seed=6)
    qa, sa, _ = oracle.quantize(synth.bits(x), oracle.BF16)
    qw, sw, _ = oracle.quantize(synth.bits(w), oracle.FP16)
    y = oracle.gemm_fp8_f32(qa.reshape(M, K), sa, qw.reshape(N, K), sw, nthreads=threads)
    ref, ab = oracle.gemm_fp8_ref(qa.reshape(M, K), sa, qw.reshape(N, K), sw)
    out = oracle.bf16_decode(y).astype(np.float64).ravel()
    assert np.all(oracle.within_tolerance(out, ref, ab, "bf16"))


def test_nested_f32_within_tolerance_of_ref():
    M, N, K = 2, 40, 1024
    a16 = synth.bits(synth.activation(M, K, seed=9, dtype="fp16"))
    w16 = synth.bits(synth.normal((N, K), 0.02, "fp16", seed=10))
    hi, lo = oracle.nested_split(w16)
    y = oracle.nested_fp16_f32(a16, hi, lo)
    ref, ab = oracle.nested_fp16_ref(a16, hi, lo)
    assert np.all(oracle.within_tolerance(oracle.f16_decode(y).ravel(), ref, ab, "fp16"))
    qa, sa, _ = oracle.quantize(a16, oracle.FP16)
    y8 = oracle.nested_fp8_f32(qa.reshape(M, K), sa, hi)
    ref8, ab8 = oracle.nested_fp8_ref(qa.reshape(M, K), sa, hi)
    assert np.all(oracle.within_tolerance(oracle.f16_decode(y8).ravel(), ref8, ab8, "fp16"))


def test_nested_fp16_identity_returns_weights():
    """A one-hot fp16 activation picks out one weight column, bit-exactly."""
    N, K = 24, 16
    w16 = synth.bits(synth.normal((N, K), 0.02, "fp16", seed=12))
    hi, lo = oracle.nested_split(w16)
    a = np.zeros((K, K), np.uint16)
    a[np.arange(K), np.arange(K)] = 0x3C00            # fp16 1.0
    y = oracle.nested_fp16_f32(a, hi, lo)
    assert np.array_equal(y, w16.T)


def test_tolerance_catches_a_dropped_k_block():
    """A result that omits one 128-wide K block must fail the bound on random
    data most of the time (why the bit-exact cases exist as well)."""
    M, N, K = 2, 64, 1024
    qa, sa, _ = oracle.quantize(synth.bits(synth.activation(M, K, seed=1)), oracle.BF16)
    qw, sw, _ = oracle.quantize(synth.bits(synth.normal((N, K), 0.02, "fp16", seed=2)),
                                oracle.FP16)
    qa, qw = qa.reshape(M, K), qw.reshape(N, K)
    ref, ab = oracle.gemm_fp8_ref(qa, sa, qw, sw)
    qa2 = qa.copy()
    qa2[:, 128:256] = 0
    bad, _ = oracle.gemm_fp8_ref(qa2, sa, qw, sw)
    assert not np.all(oracle.within_tolerance(bad, ref, ab))


def test_half_ulp_against_numpy_spacing():
    """half_ulp(v) is half of numpy's spacing of float16 at v, and half of the
    bf16 spacing (2^(e-7)) computed from torch's own rounding."""
    v = np.array([1.0, 1.5, 4.015, 60000.0, 2.0**-14, 2.0**-20, 3e-5, 0.0, 7.9e4 / 2])
    assert np.array_equal(oracle.half_ulp(v, "fp16"),
                          np.spacing(v.astype(np.float16)).astype(np.float64) / 2)
    b = torch.tensor(v, dtype=torch.float32).to(torch.bfloat16)
    nxt = (b.view(torch.int16) + 1).view(torch.bfloat16).to(torch.float64).numpy()
    spacing = nxt - b.to(torch.float64).numpy()
    assert np.array_equal(oracle.half_ulp(v, "bf16"), spacing / 2)


def test_tolerance_admits_correct_rounding_of_the_exact_result():
    """Outlier channels on a short K make single products dominate; the exact
    result rounded to bf16 must still pass (it is the best answer a bf16
    output can give), while the bound stays tight enough to reject a result
    missing one K block (test above)."""
    M, N, K = 512, 64, 176
    x = synth.activation(M, K, seed=M * 1000 + N + K, outliers=True)
    w = synth.normal((N, K), 0.02, "fp16", seed=M * 1000 + N + K + 1)
    qa, sa, _ = oracle.quantize(synth.bits(x), oracle.BF16)
    qw, sw, _ = oracle.quantize(synth.bits(w), oracle.FP16)
    ref, ab = oracle.gemm_fp8_ref(qa.reshape(M, K), sa, qw.reshape(N, K), sw)
    rounded = oracle.bf16_decode(oracle.bf16_encode(ref.astype(np.float32))).astype(np.float64)
    assert not np.all(oracle.within_tolerance(rounded, ref, ab, "exact"))
    assert np.all(oracle.within_tolerance(rounded, ref, ab, "bf16"))
