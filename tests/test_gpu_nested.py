"""GPU parity of the NestedFP path against the oracle: the byte split and the
fp16 rebuild bit-exact over all 65,536 words, the FP16- and FP8-mode GEMMs
bit-exact on identity activations and within the GEMM tolerance on random
operands (decode and tile paths)."""
import numpy as np
import pytest
import torch

import oracle
from fp8_quantized_gemm_amd import fp8q, synth
from gpu_helpers import DEV, assert_within, dense_sample, host, say, scalar_dev, to_dev_bits, to_dev_u8

pytestmark = pytest.mark.gpu

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


@pytest.mark.parametrize("reps,extra", [(1, 0), (3, 7), (1, 5)])
def test_split_and_rebuild_exhaustive(reps, extra):
    w = np.concatenate([np.tile(ALL16, reps), ALL16[:extra]]) if extra else np.tile(ALL16, reps)
    if extra == 5:
        w = w[:13]                                   # tiny: tail-only path
    say("split/rebuild", w.size)
    wd = to_dev_bits(w, "fp16")
    hi, lo = fp8q.nested_split(wd)
    ohi, olo = oracle.nested_split(w)
    assert np.array_equal(host(hi), ohi)
    assert np.array_equal(host(lo), olo)
    back = fp8q.nested_rebuild_fp16(hi, lo)
    assert np.array_equal(host(back), w)
    assert np.array_equal(host(back), oracle.nested_rebuild(ohi, olo))


def _finite_weights(rng, N, K):
    """fp16 words over the whole finite range (normals, subnormals, zeros)."""
    w = rng.integers(0, 65536, size=(N, K), dtype=np.uint32).astype(np.uint16)
    bad = (w & 0x7C00) == 0x7C00                       # inf / NaN
    w[bad] &= 0x83FF
    return w


def _run(fn, *args, M, N, guard=32):
    ybuf = torch.full((M * N + guard,), 3.0, dtype=torch.float16, device=DEV)
    y = ybuf[:M * N].view(M, N)
    fn(*args, y)
    out = host(ybuf)
    assert np.all(out[M * N:] == 0x4200), "wrote past the end of y"
    return out[:M * N].reshape(M, N)


def _one_hot_f16(M, K, cols):
    a = np.zeros((M, K), np.uint16)
    a[np.arange(M), cols] = 0x3C00                    # fp16 1.0
    return a


@pytest.mark.parametrize("M,N,K", [(1, 24, 32), (2, 40, 48), (16, 40, 64), (256, 130, 256),
                                   (48, 33, 48), (16, 40, 272), (7, 17, 400)])
def test_fp16_mode_identity_bit_exact(M, N, K):
    """a = one-hot rows: y = rebuilt weight bit-exactly (subnormals included);
    16 x 40 x 272 and 7 x 17 x 400 run the decode GEMV over several whole-line
    128-element blocks and a one-unit last block."""
    rng = np.random.Generator(np.random.PCG64(M * N * K))
    w = _finite_weights(rng, N, K)
    hi, lo = oracle.nested_split(w)
    dhi, dlo = to_dev_u8(hi), to_dev_u8(lo)
    want = np.where(w == 0x8000, 0, w).astype(np.uint16)   # -0 * 1 + (+0) = +0
    for c0 in range(0, K, M):
        m = min(M, K - c0)
        say("fp16 identity", m, N, K, c0)
        a = to_dev_bits(_one_hot_f16(m, K, np.arange(c0, c0 + m)), "fp16")
        y = _run(fp8q.nested_gemm_fp16, a, dhi, dlo, M=m, N=N)
        assert np.array_equal(y, want[:, c0:c0 + m].T), f"columns {c0}.."


@pytest.mark.parametrize("M,N,K", [(1, 21, 32), (2, 30, 64), (16, 40, 128), (200, 70, 208)])
def test_fp8_mode_identity_bit_exact(M, N, K):
    """qa = one-hot E4M3 1.0, sa = 1: y = fp16(hi << 8) bit-exactly."""
    rng = np.random.Generator(np.random.PCG64(M + N + K))
    w = _finite_weights(rng, N, K)
    hi, _ = oracle.nested_split(w)
    want = (hi.astype(np.uint16) << 8)
    want[want == 0x8000] = 0                            # -0 * 1 + (+0) = +0
    dhi = to_dev_u8(hi)
    for c0 in range(0, K, M):
        m = min(M, K - c0)
        qa = np.zeros((m, K), np.uint8)
        qa[np.arange(m), np.arange(c0, c0 + m)] = 0x38
        say("fp8 identity", m, N, K, c0)
        y = _run(fp8q.nested_gemm_fp8, to_dev_u8(qa), scalar_dev(1.0), dhi, M=m, N=N)
        assert np.array_equal(y, want[:, c0:c0 + m].T), f"columns {c0}.."


SHAPES = [(1, 1, 16), (1, 40, 4096), (2, 33, 1040), (2, 9, 11008), (3, 17, 48), (8, 100, 11008),
          (16, 64, 4112),
          (17, 33, 272), (64, 129, 1024), (256, 300, 4096), (300, 77, 160)]


def _operands(M, N, K, seed):
    a16 = synth.bits(synth.activation(M, K, seed=seed, dtype="fp16"))
    w16 = synth.bits(synth.normal((N, K), 0.02, "fp16", seed=seed + 1))
    hi, lo = oracle.nested_split(w16)
    return a16, hi, lo


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_fp16_mode_random(M, N, K):
    a16, hi, lo = _operands(M, N, K, seed=M * 100 + N + K)
    say("fp16 mode", M, N, K)
    y = _run(fp8q.nested_gemm_fp16, to_dev_bits(a16, "fp16"), to_dev_u8(hi), to_dev_u8(lo),
             M=M, N=N)
    ref, ab = oracle.nested_fp16_ref(a16, hi, lo)
    assert_within(oracle.f16_decode(y).ravel(), ref, ab, f"fp16 mode {M}x{N}x{K}", "fp16")


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_fp8_mode_random(M, N, K):
    a16, hi, _ = _operands(M, N, K, seed=M * 100 + N + K + 5)
    qa, sa, _ = oracle.quantize(a16.ravel(), oracle.FP16)
    qa = qa.reshape(M, K)
    say("fp8 mode", M, N, K)
    y = _run(fp8q.nested_gemm_fp8, to_dev_u8(qa), scalar_dev(sa), to_dev_u8(hi), M=M, N=N)
    ref, ab = oracle.nested_fp8_ref(qa, sa, hi)
    assert_within(oracle.f16_decode(y).ravel(), ref, ab, f"fp8 mode {M}x{N}x{K}", "fp16")


@pytest.mark.parametrize("M", [1, 4, 16, 256, 512, 2048])
@pytest.mark.parametrize("K,N", [(K, N) for _, K, N in synth.LLAMA7B_LINEARS])
def test_full_size_llama_shapes_dense(M, K, N):
    """NestedFP on the Llama-7B linear shapes (GPU split, GPU fp16-activation
    quantization for FP8 mode): both planes of every weight row and the
    activation codes bit-exact; outputs of both modes within tolerance of the
    oracle on every element at M <= 16, on 32 seeded rows x all N plus 32
    seeded columns x all M otherwise."""
    seed = synth.seed_for("nested", M, K, N)
    a = synth.activation(M, K, seed=seed, dtype="fp16", device=DEV)
    w = synth.normal((N, K), 0.02, "fp16", seed=seed + 1, device=DEV)
    say("nested full", M, K, N)
    hi, lo = fp8q.nested_split(w)
    y16 = fp8q.nested_gemm_fp16(a, hi, lo)
    qa, sa, _ = fp8q.fp8_quantize_act(a)
    y8 = fp8q.nested_gemm_fp8(qa, sa, hi)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(seed))
    ohi, olo = oracle.nested_split(synth.bits(w))
    assert np.array_equal(host(hi), ohi) and np.array_equal(host(lo), olo)
    ab16 = synth.bits(a)
    ms, ns = dense_sample(M, N, rng)
    ref, ab = oracle.nested_fp16_ref(ab16, ohi, olo, ms, ns)
    out = oracle.f16_decode(host(y16)[ms, ns]).astype(np.float64)
    assert_within(out, ref, ab, f"fp16 mode M={M} {K}->{N}", "fp16")
    oqa, osa, _ = oracle.quantize(ab16.ravel(), oracle.FP16)
    assert np.array_equal(host(qa).ravel(), oqa)
    ref8, ab8 = oracle.nested_fp8_ref(oqa.reshape(M, K), osa, ohi, ms, ns)
    out8 = oracle.f16_decode(host(y8)[ms, ns]).astype(np.float64)
    assert_within(out8, ref8, ab8, f"fp8 mode M={M} {K}->{N}", "fp16")


def test_fp8_mode_large_grid_sampled():
    """FP8 mode (E5M2 weights, fp16 output) on a large grid (3072 x 16384,
    K = 1040, 3072 tiles of 128x128): 2 rows, 2 columns and 256 random
    outputs against the fp64 checker."""
    M, N, K = 3072, 16384, 1040
    seed = synth.seed_for("nested-large", M, N, K)
    a16, hi, _ = _operands(M, N, K, seed=seed)
    qa, sa, _ = oracle.quantize(a16.ravel(), oracle.FP16)
    qa = qa.reshape(M, K)
    say("fp8 mode large grid", M, N, K)
    y = fp8q.nested_gemm_fp8(to_dev_u8(qa), scalar_dev(sa), to_dev_u8(hi))
    yb = host(y)
    rng = np.random.Generator(np.random.PCG64(seed))
    ms = np.concatenate([np.repeat([0, M - 1], N), np.tile(np.arange(M), 2), rng.integers(0, M, 256)])
    ns = np.concatenate([np.tile(np.arange(N), 2), np.repeat([0, N - 1], M), rng.integers(0, N, 256)])
    ref, ab = oracle.nested_fp8_ref(qa, sa, hi, ms, ns)
    out = oracle.f16_decode(yb[ms, ns]).astype(np.float64)
    assert_within(out, ref, ab, f"fp8 mode {M}x{N}x{K}", "fp16")


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (2, 300, 11008), (1, 37, 16), (1, 64, 32768),
                                   (1, 64, 16384), (1, 64, 16400), (1, 512, 2048), (3, 16, 81920),
                                   (1, 5120, 8192), (1, 24576, 4096), (1, 25088, 4096), (1, 10240, 5120),
                                   (1, 5120, 3072), (1, 40960, 5120), (64, 256, 4096), (256, 1000, 4112),
                                   (4, 1000, 4096), (16, 300, 2048), (3, 50, 10912),
                                   (16, 16400, 4096)])
def test_fp8_mode_linear_matches_quantize_then_gemm(M, N, K):
    """nested_linear_fp8 (one launch for M <= 2 with M*K <= 32768 and for
    3 <= M <= 16 with M*K <= 32768, or up to 65536 with N > 16384 (16x16400x4096,
    the activation read twice); the two-launch quantizer with partial maxima in
    y otherwise) writes the same
    codes, scale, amax and output bits as fp8_quantize_act followed by
    nested_gemm_fp8; codes equal the oracle's, sampled outputs within the
    GEMM tolerance."""
    seed = synth.seed_for("nested-linear", M, N, K)
    a = synth.activation(M, K, seed=seed, dtype="fp16", device=DEV)
    w = synth.normal((N, K), 0.02, "fp16", seed=seed + 1, device=DEV)
    hi, _ = fp8q.nested_split(w)
    say("nested linear fp8", M, N, K)
    y, q, s, am = fp8q.nested_linear_fp8(a, hi)
    q2, s2, am2 = fp8q.fp8_quantize_act(a)
    y2 = fp8q.nested_gemm_fp8(q2, s2, hi)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2) and torch.equal(am, am2)
    assert torch.equal(y, y2)
    ab16 = synth.bits(a)
    oq, os_, oa = oracle.quantize(ab16.ravel(), oracle.FP16)
    assert np.array_equal(host(q).ravel(), oq)
    assert float(host(s)[0]) == os_ and float(host(am)[0]) == oa
    ohi, _ = oracle.nested_split(synth.bits(w))
    ms = np.repeat(np.arange(min(M, 4)), min(N, 64))
    ns = np.tile(np.arange(min(N, 64)), min(M, 4))
    ref, ab = oracle.nested_fp8_ref(oq.reshape(M, K), os_, ohi, ms, ns)
    out = oracle.f16_decode(host(y)[ms, ns]).astype(np.float64)
    assert_within(out, ref, ab, f"nested linear fp8 {M}x{N}x{K}", "fp16")


@pytest.mark.parametrize("M,N,K", [(250, 12290, 1040), (260, 12300, 1040), (2000, 12000, 1040),
                                   (1000, 9000, 1040), (300, 5000, 1040)])
def test_fp16_mode_tile_shapes_ragged_sampled(M, N, K):
    """FP16 mode on each tile kernel with ragged M, N and K (K % 64 != 0):
    128x128 with 8 waves (250x12290), 256x128 (260x12300, 2000x12000),
    256x256 (1000x9000) and 64x64 (300x5000); the first and last rows and
    columns plus 256 random outputs against the fp64 checker."""
    seed = synth.seed_for("n16-tiles", M, N, K)
    a16, hi, lo = _operands(M, N, K, seed=seed)
    say("fp16 tile shapes", M, N, K)
    y = fp8q.nested_gemm_fp16(to_dev_bits(a16, "fp16"), to_dev_u8(hi), to_dev_u8(lo))
    yb = host(y)
    rng = np.random.Generator(np.random.PCG64(seed))
    ms = np.concatenate([np.repeat([0, M - 1], N), np.tile(np.arange(M), 2), rng.integers(0, M, 256)])
    ns = np.concatenate([np.tile(np.arange(N), 2), np.repeat([0, N - 1], M), rng.integers(0, N, 256)])
    ref, ab = oracle.nested_fp16_ref(a16, hi, lo, ms, ns)
    out = oracle.f16_decode(yb[ms, ns]).astype(np.float64)
    assert_within(out, ref, ab, f"fp16 mode {M}x{N}x{K}", "fp16")


def test_largest_k_fp16_mode_256_row_tiles():
    """NestedFP FP16 mode at K = 2^22 on the 256x256 tile (M = 2048, N = 8192
    pick it): an activation tile of 256 rows spans 256 * 8 MiB = 2^31 bytes,
    the most a buffer resource of the kernel holds, and its last row starts
    at 255 * 2^23 bytes.  Activations and weights take the values 0, +1 and -1
    (fp16 words 0x0000, 0x3C00, 0xBC00: hi plane 0x00 / 0x3C / 0xBC, lo plane
    zero), so every partial sum is an integer far below 2^24, exact in fp32 in
    any order: 16 x 16 sampled outputs, rows and columns on both sides of tile
    borders, equal the oracle's exact sums rounded to fp16 bit for bit.  About
    86 GB of device memory, built on the device in chunks."""
    M, N, K = 2048, 8192, 1 << 22
    gen = torch.Generator(device=DEV)
    gen.manual_seed(synth.seed_for("nested-kmax-256", M, N, K))
    say("fp16 mode largest K, 256-row tiles", M, N, K)
    hi = torch.empty((N, K), dtype=torch.uint8, device=DEV)
    lo = torch.zeros((N, K), dtype=torch.uint8, device=DEV)
    a = torch.empty((M, K), dtype=torch.float16, device=DEV)
    for dst, rows, as_bytes in ((hi, N, True), (a, M, False)):
        for r0 in range(0, rows, 256):
            t = torch.randint(0, 3, (min(256, rows - r0), K), generator=gen, device=DEV,
                              dtype=torch.uint8)
            one, neg = t == 1, t == 2
            if as_bytes:
                dst[r0:r0 + t.shape[0]] = one.to(torch.uint8) * 0x3C + neg.to(torch.uint8) * 0xBC
            else:
                dst[r0:r0 + t.shape[0]] = one.to(torch.float16) - neg.to(torch.float16)
            del t, one, neg
    y = fp8q.nested_gemm_fp16(a, hi, lo)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(K + 7))
    ms = np.unique(np.concatenate([[0, 255, 256, 1023, 1024, M - 1], rng.integers(0, M, 10)]))
    ns = np.unique(np.concatenate([[0, 255, 256, 4096, N - 1], rng.integers(0, N, 11)]))
    mi = torch.from_numpy(ms).to(DEV)
    ni = torch.from_numpy(ns).to(DEV)
    a_rows = synth.bits(a.index_select(0, mi).cpu())
    hi_rows = hi.index_select(0, ni).cpu().numpy()
    lo_rows = lo.index_select(0, ni).cpu().numpy()
    yb = host(y)
    del a, hi, lo, y
    torch.cuda.empty_cache()
    pm = np.repeat(np.arange(ms.size), ns.size)
    pn = np.tile(np.arange(ns.size), ms.size)
    ref, _ = oracle.nested_fp16_ref(a_rows, hi_rows, lo_rows, pm, pn)
    assert np.all(ref == np.round(ref)) and np.all(np.abs(ref) < 2 ** 24)
    want = ref.astype(np.float16).view(np.uint16)
    got = yb[ms[pm], ns[pn]]
    assert np.array_equal(got, want), f"{int(np.sum(got != want))} of {got.size} outputs differ"


def test_largest_k_fp16_mode_sampled():
    """NestedFP FP16 mode at K = 2^22 (activation rows of 8 MiB, tile path):
    sampled outputs within tolerance of the fp64 checker."""
    M, N, K = 20, 16, 1 << 22
    a16, hi, lo = _operands(M, N, K, seed=K + 5)
    say("fp16 mode largest K", M, N, K)
    y = fp8q.nested_gemm_fp16(to_dev_bits(a16, "fp16"), to_dev_u8(hi), to_dev_u8(lo))
    yb = host(y)
    ms = np.repeat(np.arange(M), N)
    ns = np.tile(np.arange(N), M)
    ref, ab = oracle.nested_fp16_ref(a16, hi, lo, ms, ns)
    assert_within(oracle.f16_decode(yb[ms, ns]).astype(np.float64), ref, ab,
                  f"fp16 mode {M}x{N}x{K}", "fp16")
