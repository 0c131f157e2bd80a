"""GPU parity of the per-token / per-channel path (fp8_quantize_rows,
fp8_gemm_rowwise, fp8_linear_rowwise) against the oracle.

- Codes, scales and amax of the row quantizer: bit-exact, on rows short
  enough to stay in registers and long enough to be read twice, bf16 and
  fp16, with outlier channels, zero rows and rows 2^e apart.
- GEMM: bit-exact on small-integer operands with power-of-two row and column
  scales (exact sums, exact scaling), within |y - ref| <= 2e-3 * sum|a*b| +
  1e-6 on random operands, on each dispatch path (M <= 2 row kernel, split
  and unsplit; M <= 16 GEMV; tile shapes) and ragged N.
- Equal scales give exactly what the per-tensor fp8_gemm gives.
- fp8_linear_rowwise equals fp8_quantize_rows + fp8_gemm_rowwise bit for bit.
- Full Llama-7B shapes at M = 1 and 512 through fp8_linear_rowwise: codes and
  scales bit-exact, sampled outputs within tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_quantized_gemm_amd import fp8q, synth
from gpu_helpers import DEV, assert_within, dense_sample, host, say, to_dev_u8

pytestmark = pytest.mark.gpu


def _dev_f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


# ------------------------------------------------------------------ quantizer
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("rows,cols", [(1, 16), (2, 4096), (3, 8192), (5, 8208), (7, 11008),
                                       (16, 25600), (300, 5120), (2048, 272)])
def test_quantize_rows_bit_exact(dtype, rows, cols):
    x = synth.activation(rows, cols, seed=synth.seed_for("gqr", rows, cols, dtype), dtype=dtype,
                         outliers=True)
    code = oracle.BF16 if dtype == "bf16" else oracle.FP16
    want_q, want_s, want_a = oracle.quantize_rows(synth.bits(x), code)
    say("quantize_rows", dtype, rows, cols)
    q, s, a = fp8q.fp8_quantize_rows(x.to(DEV))
    assert np.array_equal(host(q), want_q)
    assert np.array_equal(host(s).view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(host(a).view(np.uint32), want_a.view(np.uint32))


def test_quantize_rows_zero_rows_and_power_of_two_rows():
    base = synth.activation(1, 1024, seed=3, outliers=True).to(torch.float32)
    e = [0, 5, -4, 0, 9, -7]
    x = torch.cat([base * float(2.0 ** k) for k in e]).to(torch.bfloat16)
    x[3] = 0.0
    say("quantize_rows zero / 2^e rows")
    q, s, a = fp8q.fp8_quantize_rows(x.to(DEV))
    want_q, want_s, want_a = oracle.quantize_rows(synth.bits(x), oracle.BF16)
    assert np.array_equal(host(q), want_q)
    assert np.array_equal(host(s), want_s) and np.array_equal(host(a), want_a)
    hq = host(q)
    assert np.all(hq[3] == 0) and host(s)[3] == 1.0
    for r in (1, 2, 4, 5):
        assert np.array_equal(hq[r], hq[0])


# ------------------------------------------------------------------ GEMM
def _run(qa, sa, qw, sw, guard=32):
    M, N = qa.shape[0], qw.shape[0]
    ybuf = torch.full((M * N + guard,), 7.0, dtype=torch.bfloat16, device=DEV)
    y = ybuf[:M * N].view(M, N)
    fp8q.fp8_gemm_rowwise(to_dev_u8(qa), _dev_f32(sa), to_dev_u8(qw), _dev_f32(sw), y)
    out = host(ybuf)
    assert np.all(out[M * N:] == synth.bits(torch.tensor([7.0], dtype=torch.bfloat16))[0]), \
        "wrote past the end of y"
    return out[:M * N].reshape(M, N)


# M = 1, 2: row kernel (N = 4096, K = 11008 splits each row over two waves);
# M = 3..16: GEMV (N >= 16384: two 16-row tiles per workgroup, 16417 leaving
# the last one a one-row tile and an empty one); larger M: tile shapes
# 64x64 .. 256x256
SHAPES = [(1, 37, 160), (1, 4096, 11008), (2, 300, 4096), (2, 16, 16384), (1, 5, 65536),
          (3, 100, 1040), (16, 4100, 4096), (7, 16417, 272), (17, 64, 272), (129, 257, 4096),
          (512, 1000, 4096), (300, 4100, 1040), (2048, 1536, 512), (8, 520, 11008),
          (16, 16417, 9232)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_small_integers_power_of_two_scales_bit_exact(M, N, K):
    rng = np.random.Generator(np.random.PCG64(M * 7 + N * 3 + K))
    table = np.array([0x00, 0x38, 0x40, 0x48, 0xB8, 0xC0, 0xC8], np.uint8)   # 0, +-1, +-2, +-4
    qa = table[rng.integers(0, 7, size=(M, K))]
    qw = table[rng.integers(0, 7, size=(N, K))]
    sa = (2.0 ** rng.integers(-8, 9, M)).astype(np.float32)
    sw = (2.0 ** rng.integers(-12, 5, N)).astype(np.float32)
    say("rowwise small int", M, N, K)
    y = _run(qa, sa, qw, sw)
    assert np.array_equal(y, oracle.gemm_fp8_rowwise_f32(qa, sa, qw, sw))


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_random_within_tolerance(M, N, K):
    x = synth.activation(M, K, seed=synth.seed_for("rwx", M, N, K), outliers=M > 16)
    w = synth.normal((N, K), 0.02, "fp16", seed=synth.seed_for("rww", M, N, K))
    qa, sa, _ = oracle.quantize_rows(synth.bits(x), oracle.BF16)
    qw, sw, _ = oracle.quantize_rows(synth.bits(w), oracle.FP16)
    say("rowwise random", M, N, K)
    y = _run(qa, sa, qw, sw)
    if M * N <= 600_000:
        ref, ab = oracle.gemm_fp8_rowwise_ref(qa, sa, qw, sw)
        out = oracle.bf16_decode(y).astype(np.float64).ravel()
    else:
        rng = np.random.Generator(np.random.PCG64(M + N))
        ms = np.concatenate([np.repeat([0, M - 1], N), rng.integers(0, M, 4096)])
        ns = np.concatenate([np.tile(np.arange(N), 2), rng.integers(0, N, 4096)])
        ref, ab = oracle.gemm_fp8_rowwise_ref(qa, sa, qw, sw, ms, ns)
        out = oracle.bf16_decode(y[ms, ns]).astype(np.float64)
    assert_within(out, ref, ab, f"rowwise {M}x{N}x{K}", "bf16")


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (2, 300, 11008), (8, 100, 4096),
                                   (512, 1000, 4096)])
def test_equal_scales_match_per_tensor_gemm(M, N, K):
    rng = np.random.Generator(np.random.PCG64(M + N + K))
    qa = rng.integers(0, 256, size=(M, K), dtype=np.uint8)
    qw = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x3F
    qw[(qw & 0x7F) == 0x7F] = 0x3F
    s, t = np.float32(0.0123), np.float32(0.000377)
    say("rowwise equal scales vs per-tensor", M, N, K)
    y = _run(qa, np.full(M, s, np.float32), qw, np.full(N, t, np.float32))
    y2 = fp8q.fp8_gemm(to_dev_u8(qa), _dev_f32([s]), to_dev_u8(qw), _dev_f32([t]))
    assert np.array_equal(y, host(y2))


# ------------------------------------------------------------------ linear
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (2, 300, 11008), (2, 4096, 11008), (1, 64, 32768),
                                   (2, 48, 16384), (5, 1000, 4096), (16, 512, 11008), (512, 300, 4096)])
def test_linear_rowwise_matches_quantize_then_gemm(M, N, K, dtype):
    x = synth.activation(M, K, seed=synth.seed_for("rlx", M, N, K, dtype), dtype=dtype,
                         outliers=True).to(DEV)
    w = synth.normal((N, K), 0.02, "fp16", seed=synth.seed_for("rlw", M, N, K), device=DEV)
    qw, sw, _ = fp8q.fp8_quantize_rows(w)
    say("linear_rowwise", dtype, M, N, K)
    y, q, sa, am = fp8q.fp8_linear_rowwise(x, qw, sw)
    q2, sa2, am2 = fp8q.fp8_quantize_rows(x)
    y2 = fp8q.fp8_gemm_rowwise(q2, sa2, qw, sw)
    assert torch.equal(q, q2) and torch.equal(sa, sa2) and torch.equal(am, am2)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    # and the codes are the oracle's
    code = oracle.BF16 if dtype == "bf16" else oracle.FP16
    want_q, want_s, _ = oracle.quantize_rows(synth.bits(x.cpu()), code)
    assert np.array_equal(host(q), want_q) and np.array_equal(host(sa), want_s)


def test_linear_rowwise_m1_equals_per_tensor_linear():
    """With one token, per-token and per-tensor activation scaling coincide."""
    K, N = 4096, 1000
    x = synth.activation(1, K, seed=31, outliers=True).to(DEV)
    w = synth.normal((N, K), 0.02, "fp16", seed=32, device=DEV)
    qw, sw, _ = fp8q.fp8_quantize_act(w)
    say("linear_rowwise M=1 vs fp8_linear")
    y, q, sa, am = fp8q.fp8_linear_rowwise(x, qw, sw.expand(N).contiguous())
    y2, q2, s2, a2 = fp8q.fp8_linear(x, qw, sw)
    assert torch.equal(q, q2) and torch.equal(sa, s2) and torch.equal(am, a2)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_linear_rowwise_graph_replays():
    M, K, N = 2, 11008, 4096
    x = synth.activation(M, K, seed=41, outliers=True).to(DEV)
    w = synth.normal((N, K), 0.02, "fp16", seed=42, device=DEV)
    qw, sw, _ = fp8q.fp8_quantize_rows(w)
    x5 = synth.activation(512, K, seed=43, outliers=True).to(DEV)
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device=DEV),
            torch.empty((M, K), dtype=torch.uint8, device=DEV),
            torch.empty(M, device=DEV), torch.empty(M, device=DEV),
            torch.empty((512, N), dtype=torch.bfloat16, device=DEV),
            torch.empty((512, K), dtype=torch.uint8, device=DEV),
            torch.empty(512, device=DEV), torch.empty(512, device=DEV)]

    def calls():
        fp8q.fp8_linear_rowwise(x, qw, sw, *outs[:4])
        fp8q.fp8_linear_rowwise(x5, qw, sw, *outs[4:])

    say("linear_rowwise graph")
    calls()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        calls()
    for rep in range(3):
        for o in outs:
            o.view(torch.uint8).fill_(0x7f)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w_ in zip(outs, want):
            assert torch.equal(o.view(torch.uint8), w_.view(torch.uint8)), f"replay {rep}"
    del g


@pytest.mark.parametrize("M", [1, 512])
@pytest.mark.parametrize("K,N", [(K, N) for _, K, N in synth.LLAMA7B_LINEARS])
def test_full_size_llama_shapes_dense(M, K, N):
    """fp8_linear_rowwise on the Llama-7B linear shapes as the benchmark calls
    it (weights quantized per channel on the GPU, activations per token with
    outlier channels): every per-channel weight code and scale and every
    activation code and scale bit-exact; outputs within tolerance of the
    oracle on every element at M = 1, on 32 seeded rows x all N plus 32
    seeded columns x all M at M = 512."""
    seed = synth.seed_for("rowwise-full", M, K, N)
    x = synth.activation(M, K, seed=seed, outliers=True, device=DEV)
    w = synth.normal((N, K), 0.02, "fp16", seed=seed + 1, device=DEV)
    say("rowwise full", M, K, N)
    qw, sw, _ = fp8q.fp8_quantize_rows(w)
    y, q, sa, _ = fp8q.fp8_linear_rowwise(x, qw, sw)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(seed))
    oqw, osw, _ = oracle.quantize_rows(synth.bits(w.cpu()), oracle.FP16)
    assert np.array_equal(host(qw), oqw) and np.array_equal(host(sw), osw)
    oqa, osa, _ = oracle.quantize_rows(synth.bits(x.cpu()), oracle.BF16)
    assert np.array_equal(host(q), oqa) and np.array_equal(host(sa), osa)
    ms, ns = dense_sample(M, N, rng)
    ref, ab = oracle.gemm_fp8_rowwise_ref(oqa, osa, oqw, osw, ms, ns)
    out = oracle.bf16_decode(host(y)[ms, ns]).astype(np.float64)
    assert_within(out, ref, ab, f"rowwise M={M} {K}->{N}", "bf16")
