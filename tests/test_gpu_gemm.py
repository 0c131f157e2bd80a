"""GPU parity of fp8_gemm (decode path M <= 16 and tile path M > 16) against
the oracle: bit-exact on identity and small-integer operands, within
|y - ref| <= 2e-3 * sum|a*b| + 1e-6 per element on random operands.

Operands are quantized by the oracle on the host (so the GEMM is checked on
its own); the end-to-end test quantizes on the GPU and compares the codes too.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_quantized_gemm_amd import fp8q, synth
from gpu_helpers import DEV, assert_within, dense_sample, host, say, scalar_dev, to_dev_u8

pytestmark = pytest.mark.gpu


def _run_gemm(qa, sa, qw, sw, guard=32):
    M, N = qa.shape[0], qw.shape[0]
    ybuf = torch.full((M * N + guard,), 7.0, dtype=torch.bfloat16, device=DEV)
    y = ybuf[:M * N].view(M, N)
    fp8q.fp8_gemm(to_dev_u8(qa), scalar_dev(sa), to_dev_u8(qw), scalar_dev(sw), y)
    out = host(ybuf)
    assert np.all(out[M * N:] == synth.bits(torch.tensor([7.0], dtype=torch.bfloat16))[0]), \
        "wrote past the end of y"
    return out[:M * N].reshape(M, N)


def _random_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E       # no NaN codes; keeps +-448 in play
    return c


def _ident_act(M, K, cols):
    qa = np.zeros((M, K), np.uint8)
    qa[np.arange(M), cols] = 0x38      # E4M3 1.0
    return qa


# ------------------------------------------------------------------ bit-exact
@pytest.mark.parametrize("N,K", [(272, 512), (33, 144), (16, 16)])
def test_decode_identity_returns_every_weight(N, K):
    """One-hot activation rows (M = 16 per launch) read every weight back
    through the decode path: y[m, n] = E4M3(qw[n, c_m]) exactly in bf16."""
    rng = np.random.Generator(np.random.PCG64(N * K))
    qw = _random_codes(rng, (N, K))
    # a -0 weight times 1.0 plus the +0 products of the other columns sums to +0
    want = oracle.bf16_encode((oracle.e4m3_decode(qw) + 0.0).astype(np.float32))
    for c0 in range(0, K, 16):
        M = min(16, K - c0)
        say("decode identity", N, K, c0)
        y = _run_gemm(_ident_act(M, K, np.arange(c0, c0 + M)), 1.0, qw, 1.0)
        assert np.array_equal(y, want[:, c0:c0 + M].T), f"columns {c0}..{c0 + M}"


@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("N,K", [(37, 48), (9, 1040)])
def test_row_path_identity_returns_every_weight(M, N, K):
    """The M <= 2 decode path (row-contiguous, VALU decode) reads every weight
    back bit-exactly through one-hot activation rows."""
    rng = np.random.Generator(np.random.PCG64(N * K + M))
    qw = _random_codes(rng, (N, K))
    want = oracle.bf16_encode((oracle.e4m3_decode(qw) + 0.0).astype(np.float32))
    cols = list(range(K)) if K <= 64 else list(range(0, 40)) + list(range(K - 40, K))
    for c0 in range(0, len(cols), M):
        cc = cols[c0:c0 + M]
        say("row identity", M, N, K, cc[0])
        y = _run_gemm(_ident_act(len(cc), K, np.array(cc)), 1.0, qw, 1.0)
        assert np.array_equal(y, want[:, cc].T), f"columns {cc}"


@pytest.mark.parametrize("M,N,K", [(256, 300, 256), (17, 40, 32), (144, 129, 144)])
def test_tile_identity_returns_every_weight(M, N, K):
    """qa = the first M rows of I (M <= K): the tile path must return the first
    M columns of W, transposed, bit-exactly."""
    rng = np.random.Generator(np.random.PCG64(M + N + K))
    qw = _random_codes(rng, (N, K))
    say("tile identity", M, N, K)
    y = _run_gemm(_ident_act(M, K, np.arange(M)), 1.0, qw, 1.0)
    want = oracle.bf16_encode((oracle.e4m3_decode(qw) + 0.0).astype(np.float32))
    assert np.array_equal(y, want[:, :M].T)


def _small_int(rng, M, N, K):
    a = rng.integers(-16, 17, size=(M, K)).astype(np.float32)
    w = rng.integers(-16, 17, size=(N, K)).astype(np.float32)
    a.flat[rng.integers(a.size)] = 448.0
    w.flat[rng.integers(w.size)] = -448.0
    qa, sa, _ = oracle.quantize(synth.bits(torch.from_numpy(a).to(torch.bfloat16)), oracle.BF16)
    qw, sw, _ = oracle.quantize(synth.bits(torch.from_numpy(w).to(torch.float16)), oracle.FP16)
    assert sa == 1.0 and sw == 1.0
    return qa.reshape(M, K), qw.reshape(N, K)


@pytest.mark.parametrize("M,N,K", [(1, 64, 160), (5, 1000, 4096), (16, 48, 11008),
                                   (17, 64, 160), (100, 300, 4096), (300, 129, 1040),
                                   (16, 16401, 1040), (5, 20007, 272)])
def test_small_integers_bit_exact(M, N, K):
    """Exact small-integer sums on every path; 16 x 16401 and 5 x 20007 take
    the GEMV with two 16-row tiles per workgroup: its last workgroup has a
    one-row second tile (N = 16401) or a 7-row first tile and an empty second
    one (N = 20007)."""
    rng = np.random.Generator(np.random.PCG64(M * 7 + N * 3 + K))
    qa, qw = _small_int(rng, M, N, K)
    say("small int", M, N, K)
    y = _run_gemm(qa, 1.0, qw, 1.0)
    want = oracle.gemm_fp8_f32(qa, 1.0, qw, 1.0)        # exact integer sums, then bf16
    assert np.array_equal(y, want)


@pytest.mark.parametrize("M,N,K", [(16, 48, 4096), (16, 33, 4112), (9, 40, 16384),
                                   (9, 40, 16400), (8, 5000, 11008), (13, 2100, 10000),
                                   (3, 700, 16), (16, 16401, 9232)])
def test_gemv_shapes_small_integers(M, N, K):
    """The decode GEMV on shapes around its launch choices: activations of
    64 Ki and 144 Ki codes and just past them, a K of one 16-byte unit,
    313 tiles (8 x 5000 x 11008) and 16 x 16401 x 9232 (two 16-row tiles
    per workgroup, the last one a one-row tile and an empty one).  Exact
    small-integer sums."""
    rng = np.random.Generator(np.random.PCG64(M * 11 + N * 5 + K))
    qa, qw = _small_int(rng, M, N, K)
    say("gemv shapes", M, N, K)
    y = _run_gemm(qa, 1.0, qw, 1.0)
    want = oracle.gemm_fp8_f32(qa, 1.0, qw, 1.0)
    assert np.array_equal(y, want)


# ------------------------------------------------------------------ tolerance
def _quantized_operands(M, N, K, seed, outliers=False, sigma=0.02):
    x = synth.activation(M, K, seed=seed, outliers=outliers)
    w = synth.normal((N, K), sigma, "fp16", seed=seed + 1)
    qa, sa, _ = oracle.quantize(synth.bits(x), oracle.BF16)
    qw, sw, _ = oracle.quantize(synth.bits(w), oracle.FP16)
    return qa.reshape(M, K), sa, qw.reshape(N, K), sw


SHAPES = [(1, 1, 16), (1, 15, 48), (2, 16, 144), (3, 17, 4096), (8, 100, 11008), (15, 31, 4112),
          (16, 4096, 4096), (17, 33, 272), (31, 129, 1024), (129, 257, 4096), (257, 100, 11008),
          (512, 64, 176)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_random_within_tolerance(M, N, K):
    qa, sa, qw, sw = _quantized_operands(M, N, K, seed=M * 1000 + N + K, outliers=M > 16)
    say("random", M, N, K)
    y = _run_gemm(qa, sa, qw, sw)
    ref, ab = oracle.gemm_fp8_ref(qa, sa, qw, sw)
    assert_within(oracle.bf16_decode(y).astype(np.float64).ravel(), ref, ab, f"{M}x{N}x{K}", "bf16")


def test_cfg_single_linear_all_outputs():
    """M=1, K=N=4096 (weights ~N(0,0.02), activation ~N(0,1)): every output."""
    qa, sa, qw, sw = _quantized_operands(1, 4096, 4096, seed=synth.seed_for("cfg1"))
    say("single 4096x4096")
    y = _run_gemm(qa, sa, qw, sw)
    ref, ab = oracle.gemm_fp8_ref(qa, sa, qw, sw)
    assert_within(oracle.bf16_decode(y).astype(np.float64).ravel(), ref, ab, "4096x4096 M=1", "bf16")


def _gpu_pipeline(M, N, K, seed, outliers, sigma):
    """GPU quantize of x and W, then GPU GEMM; returns device tensors and the
    host bits of x and W (for the oracle)."""
    x = synth.activation(M, K, seed=seed, outliers=outliers, device=DEV)
    w = synth.normal((N, K), sigma, "fp16", seed=seed + 1, device=DEV)
    say("pipeline", M, N, K)
    qw, sw, _ = fp8q.fp8_quantize_act(w)
    qa, sa, _ = fp8q.fp8_quantize_act(x)
    y = fp8q.fp8_gemm(qa, sa, qw, sw)
    torch.cuda.synchronize()
    return x, w, qa, sa, qw, sw, y


LAYER_SHAPES = [(K, N) for _, K, N in synth.LLAMA7B_LINEARS] + \
               [(K, N) for _, K, N in synth.QWEN32B_LINEARS]


@pytest.mark.parametrize("M", [1, 4, 8, 16, 512, 1024, 2048])
@pytest.mark.parametrize("K,N", LAYER_SHAPES)
def test_full_size_layers_dense(M, K, N):
    """Full Llama-7B / Qwen-32B linear shapes, GPU quantization + GEMM: the
    activation codes, scales and every weight code bit-exact; outputs within
    tolerance of the fp64 checker on every element for M <= 16, and on 32
    seeded rows x all N plus 32 seeded columns x all M otherwise."""
    sigma = 0.015 if (K, N) in [(k, n) for _, k, n in synth.QWEN32B_LINEARS] else 0.02
    seed = synth.seed_for("layer", M, K, N)
    x, w, qa, sa, qw, sw, y = _gpu_pipeline(M, N, K, seed, outliers=M > 16, sigma=sigma)
    rng = np.random.Generator(np.random.PCG64(seed))
    wb = synth.bits(w)
    s_w = oracle.scale_from_amax(oracle.amax(wb.ravel(), oracle.FP16))
    xb = synth.bits(x)
    oqa, osa, _ = oracle.quantize(xb.ravel(), oracle.BF16)
    assert np.float32(host(sa)[0]) == np.float32(osa)
    assert np.float32(host(sw)[0]) == np.float32(s_w)
    assert np.array_equal(host(qa).ravel(), oqa)
    oqw = oracle.quantize_with_scale(wb.ravel(), oracle.FP16, s_w).reshape(N, K)
    assert np.array_equal(host(qw), oqw), "weight codes differ"
    del wb
    ms, ns = dense_sample(M, N, rng)
    ref, ab = oracle.gemm_fp8_ref(oqa.reshape(M, K), osa, oqw, s_w, ms, ns)
    out = oracle.bf16_decode(host(y)[ms, ns]).astype(np.float64)
    assert_within(out, ref, ab, f"M={M} {K}->{N}", "bf16")


def test_deterministic_and_stream_order():
    qa, sa, qw, sw = _quantized_operands(300, 1000, 4096, seed=99)
    say("determinism")
    y1 = _run_gemm(qa, sa, qw, sw)
    y2 = _run_gemm(qa, sa, qw, sw)
    assert np.array_equal(y1, y2)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y3 = _run_gemm(qa, sa, qw, sw)
    assert np.array_equal(y1, y3)


# ------------------------------------------------------------------ fp8_linear
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (2, 300, 11008), (1, 37, 16), (1, 64, 32768),
                                   (1, 64, 16384), (1, 64, 16400), (1, 512, 2048),
                                   (1, 5120, 8192), (1, 24576, 4096), (1, 25088, 4096), (1, 10240, 5120),
                                   (1, 5120, 3072), (1, 40960, 5120), (1, 300, 12288),
                                   (2, 64, 16384), (2, 64, 32768),
                                   (1, 100, 65536), (2, 50, 33792), (3, 200, 1024), (16, 64, 4096),
                                   (40, 96, 512), (64, 256, 4096), (3, 16, 81920),
                                   (4, 4096, 4096), (8, 1000, 4096), (16, 300, 2048),
                                   (5, 37, 6544), (3, 12300, 10912), (16, 4096, 4096),
                                   (7, 333, 9360), (3, 64, 16), (12, 100, 5456), (9, 1000, 7296),
                                   (4, 22016, 4096), (6, 20007, 5456), (16, 20007, 4096),
                                   (12, 16401, 5456)])
def test_linear_matches_quantize_then_gemm(M, N, K, dtype):
    """fp8_linear (one launch for M <= 16 with M*K <= 32768 and for
    3 <= M <= 16 with M*K <= 65536 and N > 16384: the row kernel for M <= 2,
    else the quantizing GEMV with 1, 2, 4 or 8 activation vectors per thread,
    ragged K blocks and up to three 16-row tiles per workgroup; 16x4096x4096,
    7x333x9360, 12x100x5456 and 9x1000x7296 are past it) returns the codes, scale and
    amax of fp8_quantize_act bit-exactly and the same y as fp8_gemm on them;
    both agree with the oracle.  Past the one-launch sizes fp8_linear keeps
    its amax partials in y when y holds enough floats (64x256x4096) and falls
    back to the atomic path when it does not (3x16x81920)."""
    seed = synth.seed_for("linear", M, N, K, dtype)
    x = synth.activation(M, K, seed=seed, dtype=dtype, outliers=M > 2)
    w = synth.normal((N, K), 0.02, "fp16", seed=seed + 1)
    oqw, osw, _ = oracle.quantize(synth.bits(w).ravel(), oracle.FP16)
    qw, sw = to_dev_u8(oqw.reshape(N, K)), scalar_dev(osw)
    xd = x.to(DEV)
    say("linear", M, N, K, dtype)
    y, q, s, a = fp8q.fp8_linear(xd, qw, sw)
    q2, s2, a2 = fp8q.fp8_quantize_act(xd)
    y2 = fp8q.fp8_gemm(q2, s2, qw, sw)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2) and torch.equal(a, a2)
    assert torch.equal(y, y2)
    code = oracle.BF16 if dtype == "bf16" else oracle.FP16
    oq, os_, oa = oracle.quantize(synth.bits(x).ravel(), code)
    assert np.array_equal(host(q).ravel(), oq)
    assert float(host(s)[0]) == os_ and float(host(a)[0]) == oa
    ms, ns = dense_sample(M, N, np.random.Generator(np.random.PCG64(seed)))
    ref, ab = oracle.gemm_fp8_ref(oq.reshape(M, K), os_, oqw.reshape(N, K), osw, ms, ns)
    out = oracle.bf16_decode(host(y)[ms, ns]).astype(np.float64)
    assert_within(out, ref, ab, f"linear {M}x{N}x{K}", "bf16")


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (2, 17, 4096), (3, 1, 16), (4, 17, 4096),
                                   (16, 33, 2048), (8, 16400, 8192), (40, 96, 512)])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_linear_zero_activation(M, N, K, dtype):
    """An all-zero (and all negative-zero) activation on every launch pattern
    of fp8_linear (row kernel, one-launch GEMV with one or several tiles per
    workgroup, tile GEMM, single and ragged output columns): amax 0, scale 1,
    every code the encoding of the input's signed zero, every output +0, as
    the oracle gives."""
    seed = synth.seed_for("linear-zero", M, N, K, dtype)
    w = synth.normal((N, K), 0.02, "fp16", seed=seed)
    oqw, osw, _ = oracle.quantize(synth.bits(w).ravel(), oracle.FP16)
    qw, sw = to_dev_u8(oqw.reshape(N, K)), scalar_dev(osw)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    code = oracle.BF16 if dtype == "bf16" else oracle.FP16
    for neg in (False, True):
        x = torch.zeros((M, K), dtype=tdt)
        if neg:
            x = -x
        say("linear zero", M, N, K, dtype, "neg" if neg else "pos")
        y, q, s, a = fp8q.fp8_linear(x.to(DEV), qw, sw)
        oq, os_, oa = oracle.quantize(synth.bits(x).ravel(), code)
        assert float(host(s)[0]) == os_ == 1.0 and float(host(a)[0]) == oa == 0.0
        assert np.array_equal(host(q).ravel(), oq)
        assert np.all(host(y) == 0), "outputs must be +0"


@pytest.mark.parametrize("M,N,K", [(1, 512, 4096), (2, 8192, 1024), (4, 1024, 4096),
                                   (16, 2048, 4096), (3, 64, 8192)])
def test_linear_output_overlapping_input(M, N, K):
    """y laid over x (in place): the one-launch kernels would store y while
    other workgroups still read x, so fp8_linear quantizes first and runs the
    GEMM after; y, q, scale and amax equal those of separate buffers."""
    seed = synth.seed_for("linear-overlap", M, N, K)
    x = synth.activation(M, K, seed=seed, outliers=M > 2)
    w = synth.normal((N, K), 0.02, "fp16", seed=seed + 1)
    oqw, osw, _ = oracle.quantize(synth.bits(w).ravel(), oracle.FP16)
    qw, sw = to_dev_u8(oqw.reshape(N, K)), scalar_dev(osw)
    say("linear overlap", M, N, K)
    y1, q1, s1, a1 = fp8q.fp8_linear(x.to(DEV), qw, sw)
    buf = torch.zeros(max(M * K, M * N), dtype=torch.bfloat16, device=DEV)
    buf[:M * K].copy_(x.reshape(-1).to(DEV))
    y2, q2, s2, a2 = fp8q.fp8_linear(buf[:M * K].view(M, K), qw, sw, buf[:M * N].view(M, N))
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2) and torch.equal(a1, a2)
    assert torch.equal(y1, y2)


def test_linear_output_over_the_codes_is_refused():
    """y sharing bytes with q: the GEMM would read codes that other workgroups
    overwrite, so the call is refused (FP8Q_ERR_OVERLAP) and nothing runs."""
    M, N, K = 4, 64, 256
    x = synth.activation(M, K, seed=5).to(DEV)
    qw = torch.zeros((N, K), dtype=torch.uint8, device=DEV)
    sw = torch.ones(1, dtype=torch.float32, device=DEV)
    buf = torch.zeros(max(M * K, 2 * M * N), dtype=torch.uint8, device=DEV)
    q = buf[:M * K].view(M, K)
    y = buf[:2 * M * N].view(torch.bfloat16).view(M, N)
    with pytest.raises(fp8q.Fp8qError) as err:
        fp8q.fp8_linear(x, qw, sw, y, q)
    assert err.value.status == 7
    torch.cuda.synchronize()
    assert int(buf.count_nonzero()) == 0


# ------------------------------------------------------------------ big-tile path
# The tile shape is picked per call from the cost of its rounds of
# workgroups: 256x256 (4096x4096, 4100x12300), 256x192 (2000x12000,
# 1000x10000), 256x128 (2040x4090, 1024x8192), 128x192 (2065x8292, 4096x4100,
# 200x22000), 128x128 with 8 waves (510x8190, 639x5370), 128x64 (500x4000,
# 1024x2048) and 64x64 (60x5000); ragged M, N (N % 4 != 0 takes the 2-byte
# stores) and K (K % 128 != 0: the last step is partial) on each of them.
def _big_tiles(M, N):
    return -(-M // 256) * -(-N // 256)


@pytest.mark.parametrize("MK,N", [(4096, 4096), (1024, 8192), (1024, 2048)])
def test_big_tile_identity_returns_every_weight(MK, N):
    """qa = I with M = K: y = W^T bit-exactly for every weight, on 256x256
    tiles (4096^3), 256x128 tiles (1024 x 8192) and 128x64 tiles (1024 x 2048)."""
    M = K = MK
    rng = np.random.Generator(np.random.PCG64(4096 + N))
    qw = _random_codes(rng, (N, K))
    say("big identity", M, N, K, "tiles256", _big_tiles(M, N))
    y = _run_gemm(_ident_act(M, K, np.arange(M)), 1.0, qw, 1.0)
    want = oracle.bf16_encode((oracle.e4m3_decode(qw) + 0.0).astype(np.float32))
    assert np.array_equal(y, want.T)


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 80), (4100, 12300, 48), (2000, 12000, 80),
                                   (2040, 4090, 48), (510, 8190, 80), (200, 22000, 48),
                                   (639, 5370, 80), (500, 4000, 48), (60, 5000, 80),
                                   (500, 4000, 272), (512, 4096, 400)])
def test_big_tile_small_integers_bit_exact(M, N, K):
    """Small integers through every tile kernel; K = 80, 48, 272 and 400
    leave a partial K step (out-of-range units read as zero).  500 x 4000 and
    512 x 4096 take the 128x64 tile, here over 1, 3 and 4 K steps."""
    rng = np.random.Generator(np.random.PCG64(K + N))
    qa, qw = _small_int(rng, M, N, K)
    say("big small int", M, N, K, "tiles256", _big_tiles(M, N))
    y = _run_gemm(qa, 1.0, qw, 1.0)
    want = oracle.gemm_fp8_f32(qa, 1.0, qw, 1.0)
    assert np.array_equal(y, want)


@pytest.mark.parametrize("M,N,K", [(2065, 8292, 4112), (4096, 4100, 272), (2040, 4090, 4112),
                                   (4100, 12300, 272), (1000, 10000, 1040), (510, 8190, 1040),
                                   (200, 22000, 1040), (639, 5370, 4112), (500, 4000, 1040),
                                   (60, 5000, 4112)])
def test_big_tile_random_ragged_sampled(M, N, K):
    """Ragged M, N and K on both tile kernels; every output of 3 rows and 3
    columns plus 512 random pairs against the fp64 checker."""
    seed = synth.seed_for("big", M, N, K)
    qa, sa, qw, sw = _quantized_operands(M, N, K, seed=seed, outliers=True)
    say("big random", M, N, K, "tiles256", _big_tiles(M, N))
    y = _run_gemm(qa, sa, qw, sw)
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = np.concatenate([[0, M - 1], rng.integers(0, M, 1)])
    cols = np.concatenate([[0, N - 1], rng.integers(0, N, 1)])
    ms = np.concatenate([np.repeat(rows, N), np.tile(np.arange(M), cols.size),
                         rng.integers(0, M, 512)])
    ns = np.concatenate([np.tile(np.arange(N), rows.size), np.repeat(cols, M),
                         rng.integers(0, N, 512)])
    ref, ab = oracle.gemm_fp8_ref(qa, sa, qw, sw, ms, ns)
    out = oracle.bf16_decode(y[ms, ns]).astype(np.float64)
    assert_within(out, ref, ab, f"big {M}x{N}x{K}", "bf16")


# ------------------------------------------------------------------ largest K
KMAX = 1 << 22


@pytest.mark.parametrize("M", [1, 8, 40])
def test_largest_k_bit_exact(M):
    """K = 2^22 (the largest the boundary accepts) on the row kernel (M = 1,
    codes read from L2), the MFMA GEMV (M = 8) and a tile kernel (M = 40):
    codes of 0, +-1, +-2 keep every partial sum an integer below 2^24, so the
    fp32 accumulation is exact in any order and the bf16 output equals the
    oracle's bit for bit.  32-bit offsets reach 2^30 on the tile kernel."""
    rng = np.random.Generator(np.random.PCG64(M + KMAX))
    table = np.array([0x00, 0x38, 0x40, 0xB8, 0xC0], np.uint8)      # 0, 1, 2, -1, -2
    qa = table[rng.integers(0, 5, size=(M, KMAX))]
    qw = table[rng.integers(0, 5, size=(16, KMAX))]
    say("largest K", M, 16, KMAX)
    y = _run_gemm(qa, 1.0, qw, 1.0)
    want = oracle.gemm_fp8_f32(qa, 1.0, qw, 1.0)
    assert np.array_equal(y, want)


# ------------------------------------------------------------------ split-K rows
# The M <= 2 row kernel cuts each weight row's K range over 2..16 waves when
# its workgroups hold few rows of long K (partial sums added through LDS).
# These shapes take that path with full and ragged last segments, workgroups
# without rows (N = 4000 over 512 workgroups of 8 rows), codes staged in LDS
# (M * K <= 32768) and read from L2 (M = 1, K = 65536).
SPLIT_SHAPES = [(1, 4096, 11008), (1, 4000, 11008), (1, 3, 32752), (2, 16, 16384),
                (2, 300, 16000), (1, 5, 65536), (2, 300, 11008)]


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
def test_split_k_rows_small_integers_bit_exact(M, N, K):
    """Codes of 0, +-1, +-2, +-4 and a few +-448 keep every partial sum an
    integer far below 2^24: exact in any summation order, so the split
    kernel's output equals the oracle's bit for bit."""
    rng = np.random.Generator(np.random.PCG64(M * 31 + N * 7 + K))
    table = np.array([0x00, 0x38, 0x40, 0x48, 0xB8, 0xC0, 0xC8], np.uint8)   # 0, 1, 2, 4, -1, -2, -4
    qa = table[rng.integers(0, 7, size=(M, K))]
    qw = table[rng.integers(0, 7, size=(N, K))]
    qa.flat[rng.integers(qa.size, size=2)] = 0x7E                             # 448
    qw.flat[rng.integers(qw.size, size=4)] = 0xFE                             # -448
    say("split-K rows small int", M, N, K)
    y = _run_gemm(qa, 1.0, qw, 1.0)
    assert np.array_equal(y, oracle.gemm_fp8_f32(qa, 1.0, qw, 1.0))


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
def test_split_k_rows_random_within_tolerance(M, N, K):
    qa, sa, qw, sw = _quantized_operands(M, N, K, seed=M * 17 + N * 5 + K)
    say("split-K rows random", M, N, K)
    y = _run_gemm(qa, sa, qw, sw)
    ref, ab = oracle.gemm_fp8_ref(qa, sa, qw, sw)
    assert_within(oracle.bf16_decode(y).astype(np.float64).ravel(), ref, ab, f"{M}x{N}x{K}", "bf16")


@pytest.mark.parametrize("M,N,K", [(1, 9, 32752), (2, 5, 16384)])
def test_split_k_rows_identity_returns_every_weight(M, N, K):
    """One-hot activations on the columns around every 2048-byte boundary
    (where the split kernel's segments start and end) read the weights back
    bit-exactly."""
    rng = np.random.Generator(np.random.PCG64(N * K + M))
    qw = _random_codes(rng, (N, K))
    want = oracle.bf16_encode((oracle.e4m3_decode(qw) + 0.0).astype(np.float32))
    cols = sorted({c for b in range(0, K + 1, 2048) for c in (b - 1, b) if 0 <= c < K} | {K - 1})
    for c0 in range(0, len(cols), M):
        cc = cols[c0:c0 + M]
        say("split-K identity", M, N, K, cc[0])
        y = _run_gemm(_ident_act(len(cc), K, np.array(cc)), 1.0, qw, 1.0)
        assert np.array_equal(y, want[:, cc].T), f"columns {cc}"
