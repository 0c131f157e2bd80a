"""GPU parity of NestedFP with an E4M3 upper byte (nested_split_e4m3,
nested_rebuild_e4m3, nested_gemm_fp16_e4m3, nested_gemm_fp8_e4m3,
nested_linear_fp8_e4m3) against the oracle.

- Split and rebuild: bit-exact over all 65,536 fp16 words (and a ragged
  tail), with the count of words outside the FP8 mode's range.
- FP16 mode: bit-identical to nested_gemm_fp16 on the plain-split planes of
  the same weights (both rebuild the same words), on the row, GEMV and tile
  paths, and within tolerance of the oracle.
- FP8 mode: bit-exact on small-integer operands, within
  |y - ref| <= 2e-3 * sum|a*b| + 1e-6 on random ones, on each path.
- nested_linear_fp8_e4m3 equals fp8_quantize_act + nested_gemm_fp8_e4m3.
- Full Llama-7B shapes at M = 1 and 256, both modes, sampled outputs.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_quantized_gemm_amd import fp8q, synth
from gpu_helpers import DEV, assert_within, dense_sample, host, say, scalar_dev, to_dev_u8

pytestmark = pytest.mark.gpu

ALL = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
SHAPES = [(1, 4096, 4096), (2, 300, 1040), (5, 1000, 4096), (16, 64, 11008), (256, 4100, 4096),
          (300, 129, 272)]


def _words_tensor(words: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(words.copy()).view(torch.float16).to(DEV)


@pytest.mark.parametrize("extra", [0, 5])
def test_split_and_rebuild_every_word(extra):
    words = np.concatenate([ALL, ALL[:extra]])
    want_hi, want_lo, want_bad = oracle.nested_split_e4m3(words)
    say("split e4m3 all words", extra)
    hi, lo, bad = fp8q.nested_split_e4m3(_words_tensor(words))
    assert np.array_equal(host(hi), want_hi) and np.array_equal(host(lo), want_lo)
    assert int(host(bad)[0]) == want_bad
    w = fp8q.nested_rebuild_e4m3(hi, lo)
    assert np.array_equal(synth.bits(w.cpu()), words)


def test_model_weights_are_in_range():
    w = synth.normal((4096, 4096), 0.02, "fp16", seed=5, device=DEV)
    say("split e4m3 weights")
    _, _, bad = fp8q.nested_split_e4m3(w)
    assert int(bad.item()) == 0


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_fp16_mode_equals_plain_split(M, N, K):
    w = synth.normal((N, K), 0.02, "fp16", seed=synth.seed_for("e4w", M, N, K), device=DEV)
    a = synth.activation(M, K, seed=synth.seed_for("e4a", M, N, K), dtype="fp16", device=DEV)
    hi4, lo4, _ = fp8q.nested_split_e4m3(w)
    hi, lo = fp8q.nested_split(w)
    say("fp16 mode e4m3 split", M, N, K)
    y4 = fp8q.nested_gemm_fp16_e4m3(a, hi4, lo4)
    y = fp8q.nested_gemm_fp16(a, hi, lo)
    assert torch.equal(y4.view(torch.int16), y.view(torch.int16))
    if M * N <= 300_000:
        ohi, olo = oracle.nested_split(synth.bits(w.cpu()))
        ref, ab = oracle.nested_fp16_ref(synth.bits(a.cpu()), ohi, olo)
        assert_within(oracle.f16_decode(synth.bits(y4.cpu())).ravel(), ref, ab,
                      f"fp16 e4m3 {M}x{N}x{K}", "fp16")


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_fp8_mode_small_integers_bit_exact(M, N, K):
    rng = np.random.Generator(np.random.PCG64(M * 7 + N + K))
    table = np.array([0x00, 0x38, 0x40, 0x48, 0xB8, 0xC0, 0xC8], np.uint8)   # 0, +-1, +-2, +-4
    qa = table[rng.integers(0, 7, size=(M, K))]
    hi = table[rng.integers(0, 7, size=(N, K))]
    sa = np.float32(0.5)
    say("fp8 mode e4m3 small int", M, N, K)
    y = fp8q.nested_gemm_fp8_e4m3(to_dev_u8(qa), scalar_dev(float(sa)), to_dev_u8(hi))
    want = oracle.gemm_fp8_f32_fp16out(qa, float(sa), hi, oracle.NESTED_E4M3_SCALE)
    assert np.array_equal(synth.bits(y.cpu()), want)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_fp8_mode_random_within_tolerance(M, N, K):
    w = synth.normal((N, K), 0.02, "fp16", seed=synth.seed_for("e4r", M, N, K))
    x = synth.activation(M, K, seed=synth.seed_for("e4x", M, N, K), dtype="fp16", outliers=M > 16)
    ohi, _, bad = oracle.nested_split_e4m3(synth.bits(w))
    assert bad == 0
    qa, sa, _ = oracle.quantize(synth.bits(x).ravel(), oracle.FP16)
    qa = qa.reshape(M, K)
    say("fp8 mode e4m3 random", M, N, K)
    y = fp8q.nested_gemm_fp8_e4m3(to_dev_u8(qa), scalar_dev(sa), to_dev_u8(ohi))
    if M * N <= 300_000:
        ref, ab = oracle.gemm_fp8_ref(qa, sa, ohi, oracle.NESTED_E4M3_SCALE)
        out = oracle.f16_decode(synth.bits(y.cpu())).ravel()
    else:
        rng = np.random.Generator(np.random.PCG64(M + N))
        ms, ns = rng.integers(0, M, 8192), rng.integers(0, N, 8192)
        ref, ab = oracle.gemm_fp8_ref(qa, sa, ohi, oracle.NESTED_E4M3_SCALE, ms, ns)
        out = oracle.f16_decode(synth.bits(y.cpu())[ms, ns])
    assert_within(out, ref, ab, f"fp8 e4m3 {M}x{N}x{K}", "fp16")


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (2, 300, 11008), (5, 1000, 4096), (300, 129, 272),
                                   (12, 16401, 5456)])
def test_linear_fp8_e4m3_matches_quantize_then_gemm(M, N, K):
    w = synth.normal((N, K), 0.02, "fp16", seed=synth.seed_for("e4l", M, N, K), device=DEV)
    a = synth.activation(M, K, seed=synth.seed_for("e4la", M, N, K), dtype="fp16", device=DEV)
    hi, _, _ = fp8q.nested_split_e4m3(w)
    say("linear fp8 e4m3", M, N, K)
    y, q, s, _ = fp8q.nested_linear_fp8_e4m3(a, hi)
    q2, s2, _ = fp8q.fp8_quantize_act(a)
    y2 = fp8q.nested_gemm_fp8_e4m3(q2, s2, hi)
    assert torch.equal(q.view(-1), q2.view(-1)) and torch.equal(s, s2)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("M", [1, 256])
@pytest.mark.parametrize("K,N", [(K, N) for _, K, N in synth.LLAMA7B_LINEARS])
def test_full_size_llama_shapes_dense(M, K, N):
    """Both modes on the Llama-7B linear shapes as the benchmark runs them (GPU
    split; FP8 mode through nested_linear_fp8_e4m3, which quantizes the fp16
    activation itself): the split of every weight row and the activation codes
    bit-exact; outputs within tolerance of the oracle on every element at
    M = 1, on 32 seeded rows x all N plus 32 seeded columns x all M at
    M = 256."""
    seed = synth.seed_for("nested-e4m3-full", M, K, N)
    a = synth.activation(M, K, seed=seed, dtype="fp16", device=DEV)
    w = synth.normal((N, K), 0.02, "fp16", seed=seed + 1, device=DEV)
    say("nested e4m3 full", M, K, N)
    hi, lo, bad = fp8q.nested_split_e4m3(w)
    y16 = fp8q.nested_gemm_fp16_e4m3(a, hi, lo)
    y8, qa, sa, _ = fp8q.nested_linear_fp8_e4m3(a, hi)
    torch.cuda.synchronize()
    assert int(bad.item()) == 0
    rng = np.random.Generator(np.random.PCG64(seed))
    wb = synth.bits(w.cpu())
    ohi, olo, _ = oracle.nested_split_e4m3(wb)
    assert np.array_equal(host(hi), ohi) and np.array_equal(host(lo), olo)
    ab16 = synth.bits(a.cpu())
    ms, ns = dense_sample(M, N, rng)
    phi, plo = oracle.nested_split(wb)              # the same words, plain planes
    ref, ab = oracle.nested_fp16_ref(ab16, phi, plo, ms, ns)
    out = oracle.f16_decode(host(y16)[ms, ns]).astype(np.float64)
    assert_within(out, ref, ab, f"fp16 e4m3 M={M} {K}->{N}", "fp16")
    oqa, osa, _ = oracle.quantize(ab16.ravel(), oracle.FP16)
    assert np.array_equal(host(qa).ravel(), oqa) and host(sa)[0] == np.float32(osa)
    ref8, ab8 = oracle.gemm_fp8_ref(oqa.reshape(M, K), osa, ohi, oracle.NESTED_E4M3_SCALE, ms, ns)
    out8 = oracle.f16_decode(host(y8)[ms, ns]).astype(np.float64)
    assert_within(out8, ref8, ab8, f"fp8 e4m3 M={M} {K}->{N}", "fp16")
