"""GPU parity of delayed scaling with an amax history (fp8_quantize_act_delayed,
fp8_linear_delayed) against the oracle, call by call.

Every call is compared bit-exactly: codes, the scale used, the amax, and after
the sequence the history ring and the state (next scale, position, and the
accumulators back at 0).  Magnitudes change from call to call, so later calls
saturate and the window maximum moves; the history is short (wraps) and long.
Covers the single-workgroup quantizer (n <= 32768), the grid-stride one (its
last workgroup publishes the call), the fused decode linear (M <= 2) and the
two-launch linear, and HIP-graph replays (each replay is one more call).
Full Llama-7B shapes at M = 1 and 512 with a history of 1024: three calls,
outputs of the last within tolerance of the oracle on every element at M = 1,
on 32 seeded rows x all N plus 32 seeded columns x all M at M = 512.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_quantized_gemm_amd import fp8q, synth
from gpu_helpers import DEV, assert_within, dense_sample, host, say

pytestmark = pytest.mark.gpu

MAGS = [1.0, 3.0, 0.25, 40.0, 0.5, 0.5, 2.0, 0.125]


def _inputs(M, K, dtype, seed):
    return [(synth.activation(M, K, seed=seed + t, dtype=dtype, outliers=True).to(torch.float32)
             * mag).to(torch.bfloat16 if dtype == "bf16" else torch.float16) for t, mag in
            enumerate(MAGS)]


def _check_state(ds: fp8q.DelayedScaling, od: oracle.DelayedScaling, what):
    assert np.array_equal(host(ds.history), od.history), f"{what}: history"
    st = host(ds.state).view(np.uint32)
    assert st[0] == od.state[0] and st[2] == od.state[2], f"{what}: next scale / position"
    assert st[4] == np.max(od.history).astype(np.float32).view(np.uint32), f"{what}: max(history)"
    acc = st.copy()
    acc[[0, 2, 4]] = 0
    assert np.all(acc == 0), f"{what}: accumulators not cleared at {np.nonzero(acc)[0]}"


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("M,K,L", [(1, 4096, 3), (4, 8192, 1024), (300, 5120, 3),
                                   (2048, 11008, 5), (3, 17, 2)])
def test_quantize_delayed_sequence(M, K, L, dtype):
    xs = _inputs(M, K, dtype, seed=synth.seed_for("dq", M, K, L, dtype))
    code = oracle.BF16 if dtype == "bf16" else oracle.FP16
    od = oracle.DelayedScaling(L)
    ds = fp8q.DelayedScaling(L, device=DEV)
    for t, x in enumerate(xs):
        want_q, want_s, want_a = od.quantize(synth.bits(x).ravel(), code)
        say("quantize delayed", dtype, M, K, L, "call", t)
        q, s, a = fp8q.fp8_quantize_act_delayed(x.to(DEV), ds)
        assert np.array_equal(host(q).ravel(), want_q), f"call {t}: codes"
        assert host(s)[0] == np.float32(want_s) and host(a)[0] == np.float32(want_a), f"call {t}"
    _check_state(ds, od, f"{M}x{K} L={L}")


@pytest.mark.parametrize("M,K,N", [(1, 4096, 4096), (2, 11008, 300), (1, 32752, 64),
                                   (16, 4096, 1000), (512, 4096, 300)])
def test_linear_delayed_sequence(M, K, N):
    L = 4
    xs = _inputs(M, K, "bf16", seed=synth.seed_for("dl", M, K, N))
    w = synth.normal((N, K), 0.02, "fp16", seed=synth.seed_for("dlw", M, K, N), device=DEV)
    qw, sw, _ = fp8q.fp8_quantize_act(w)
    od = oracle.DelayedScaling(L)
    ds = fp8q.DelayedScaling(L, device=DEV)
    for t, x in enumerate(xs):
        want_q, want_s, want_a = od.quantize(synth.bits(x).ravel(), oracle.BF16)
        say("linear delayed", M, K, N, "call", t)
        y, q, s, a = fp8q.fp8_linear_delayed(x.to(DEV), qw, sw, ds)
        assert np.array_equal(host(q).ravel(), want_q), f"call {t}: codes"
        assert host(s)[0] == np.float32(want_s) and host(a)[0] == np.float32(want_a), f"call {t}"
        y2 = fp8q.fp8_gemm(q, s, qw, sw)                      # the GEMM on the same codes
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), f"call {t}: y"
    _check_state(ds, od, f"linear {M}x{K}x{N}")


def test_linear_delayed_fp16_and_two_states_independent():
    K, N = 4096, 512
    w = synth.normal((N, K), 0.02, "fp16", seed=7, device=DEV)
    qw, sw, _ = fp8q.fp8_quantize_act(w)
    xa = _inputs(1, K, "fp16", seed=70)
    xb = _inputs(2, K, "fp16", seed=80)
    oa, ob = oracle.DelayedScaling(8), oracle.DelayedScaling(2)
    da, db = fp8q.DelayedScaling(8, device=DEV), fp8q.DelayedScaling(2, device=DEV)
    for t in range(len(MAGS)):
        for x, od, ds, tag in ((xa[t], oa, da, "a"), (xb[t], ob, db, "b")):
            want_q, want_s, _ = od.quantize(synth.bits(x).ravel(), oracle.FP16)
            say("linear delayed fp16", tag, "call", t)
            y, q, s, _ = fp8q.fp8_linear_delayed(x.to(DEV), qw, sw, ds)
            assert np.array_equal(host(q).ravel(), want_q) and host(s)[0] == np.float32(want_s)
    _check_state(da, oa, "state a")
    _check_state(db, ob, "state b")


@pytest.mark.parametrize("M,K,N", [(1, 4096, 4096), (300, 5120, 256)])
def test_delayed_graph_replays_advance_the_history(M, K, N):
    """A captured call replayed R times is R more calls: the scale of each
    replay follows the oracle's sequence on the same input."""
    L, R = 3, 4
    x = (synth.activation(M, K, seed=91, outliers=True).to(torch.float32) * 5.0).to(torch.bfloat16)
    w = synth.normal((N, K), 0.02, "fp16", seed=92, device=DEV)
    qw, sw, _ = fp8q.fp8_quantize_act(w)
    xd = x.to(DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    q = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    s = torch.empty(1, device=DEV)
    a = torch.empty(1, device=DEV)
    ds = fp8q.DelayedScaling(L, device=DEV)
    od = oracle.DelayedScaling(L)
    # warm-up call on the capture stream (one call), then capture one call
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    say("delayed graph", M, K, N)
    with torch.cuda.stream(side):
        fp8q.fp8_linear_delayed(xd, qw, sw, ds, y, q, s, a)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    od.quantize(synth.bits(x).ravel(), oracle.BF16)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp8q.fp8_linear_delayed(xd, qw, sw, ds, y, q, s, a)
    # capture records without running: the state is unchanged
    _check_state(ds, od, "after capture")
    for rep in range(R):
        want_q, want_s, want_a = od.quantize(synth.bits(x).ravel(), oracle.BF16)
        q.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(q).ravel(), want_q), f"replay {rep}: codes"
        assert host(s)[0] == np.float32(want_s) and host(a)[0] == np.float32(want_a), f"replay {rep}"
        y2 = fp8q.fp8_gemm(q, s, qw, sw)
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), f"replay {rep}: y"
    _check_state(ds, od, "after replays")
    del g


@pytest.mark.parametrize("M", [1, 512])
@pytest.mark.parametrize("K,N", [(K, N) for _, K, N in synth.LLAMA7B_LINEARS])
def test_full_size_llama_shapes_sequence(M, K, N):
    """fp8_linear_delayed on the Llama-7B linear shapes with the benchmark's
    history length (1024): three calls with rising magnitudes, so the third
    saturates against the second's amax.  Codes, scale and amax bit-exact on
    every call; outputs of the last call within tolerance (dense_sample)."""
    seed = synth.seed_for("delayed-full", M, K, N)
    w = synth.normal((N, K), 0.02, "fp16", seed=seed + 1)
    oqw, osw, _ = oracle.quantize(synth.bits(w).ravel(), oracle.FP16)   # offline, by the oracle
    oqw = oqw.reshape(N, K)
    qw = torch.from_numpy(oqw).to(DEV)
    sw = torch.tensor([osw], dtype=torch.float32, device=DEV)
    od = oracle.DelayedScaling(1024)
    ds = fp8q.DelayedScaling(1024, device=DEV)
    for t, mag in enumerate((1.0, 0.5, 4.0)):
        x = (synth.activation(M, K, seed=seed + 10 + t, outliers=M > 16).to(torch.float32)
             * mag).to(torch.bfloat16)
        want_q, want_s, want_a = od.quantize(synth.bits(x).ravel(), oracle.BF16)
        say("delayed full", M, K, N, "call", t)
        y, q, s, a = fp8q.fp8_linear_delayed(x.to(DEV), qw, sw, ds)
        assert np.array_equal(host(q).ravel(), want_q), f"call {t}: codes"
        assert host(s)[0] == np.float32(want_s) and host(a)[0] == np.float32(want_a), f"call {t}"
    rng = np.random.Generator(np.random.PCG64(seed))
    ms, ns = dense_sample(M, N, rng)
    ref, ab = oracle.gemm_fp8_ref(want_q.reshape(M, K), want_s, oqw, osw, ms, ns)
    out = oracle.bf16_decode(host(y)[ms, ns]).astype(np.float64)
    assert_within(out, ref, ab, f"delayed M={M} {K}->{N}", "bf16")


def _spike_sequence(M, K, dtype, seed):
    """Calls that drive x / s beyond the binary32 range under a small delayed
    scale: the history first holds an amax of exactly 1.0 (scale 1/448), then
    inputs carry spikes whose quotient x * (1/s) overflows (bf16: 1e36,
    -3e38, a lone 3e38 among N(0,1) values; both dtypes: +-inf; fp16 also its
    largest finite value 65504), with calls of amax 1.0 in between so that
    the scale drops back to 1/448 before each spike (history length 1).  The
    infinite spike comes last, so no call quantizes with an infinite scale
    except the oracle-checked state it leaves."""
    td = torch.bfloat16 if dtype == "bf16" else torch.float16
    rng = np.random.Generator(np.random.PCG64(seed))

    def unit():                                  # N(0,1) clipped, amax exactly 1.0
        v = np.clip(rng.standard_normal((M, K)).astype(np.float32) * 0.3, -0.99, 0.99)
        v.flat[rng.integers(M * K)] = 1.0
        return v

    def spiked(vals):
        v = rng.standard_normal((M, K)).astype(np.float32)
        idx = rng.choice(M * K, len(vals), replace=False)
        for i, s in zip(idx, vals):
            v.flat[i] = s
        return v

    if dtype == "bf16":
        spikes = [[1e36, -1e36, 5e37], [-3e38], [3e38], [np.inf, -np.inf, 1e36]]
    else:
        spikes = [[65504.0, -65504.0], [np.inf], [-np.inf, 65504.0]]
    seq = [unit()]
    for sp in spikes:
        seq += [spiked(sp), unit()]
    seq.pop()                                    # end on the infinite spike
    return [torch.from_numpy(v).to(td) for v in seq]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("path,M,K,N", [("one workgroup", 1, 4096, 0),
                                        ("grid-stride", 64, 4096, 0),
                                        ("fused decode", 1, 4096, 512),
                                        ("fused decode", 2, 11008, 300),
                                        ("two-launch linear", 24, 4096, 300)])
def test_delayed_overflowing_quotients_saturate(path, M, K, N, dtype):
    """Codes of spikes whose quotient overflows binary32 saturate to +-448
    (0x7E / 0xFE) as the oracle's IEEE quotient does, never the NaN code; the
    scale, amax, ring and state follow the oracle call by call, and the
    linear's output equals the GEMM on the same codes."""
    xs = _spike_sequence(M, K, dtype, seed=synth.seed_for("ds-spike", path, M, K, dtype))
    code = oracle.BF16 if dtype == "bf16" else oracle.FP16
    od = oracle.DelayedScaling(1)
    ds = fp8q.DelayedScaling(1, device=DEV)
    if N:
        w = synth.normal((N, K), 0.02, "fp16", seed=synth.seed_for("ds-spike-w", N, K), device=DEV)
        qw, sw, _ = fp8q.fp8_quantize_act(w)
    saturated = 0
    for t, x in enumerate(xs):
        want_q, want_s, want_a = od.quantize(synth.bits(x).ravel(), code)
        say("delayed spike", path, dtype, M, K, N, "call", t)
        if N:
            y, q, s, a = fp8q.fp8_linear_delayed(x.to(DEV), qw, sw, ds)
        else:
            q, s, a = fp8q.fp8_quantize_act_delayed(x.to(DEV), ds)
        got = host(q).ravel()
        assert not np.any((got & 0x7F) == 0x7F), f"call {t}: NaN code"
        assert np.array_equal(got, want_q), f"call {t}: codes"
        assert host(s)[0] == np.float32(want_s), f"call {t}: scale"
        assert host(a)[0] == np.float32(want_a), f"call {t}: amax"
        saturated += int(np.count_nonzero((want_q & 0x7F) == 0x7E))
        if N:
            y2 = fp8q.fp8_gemm(q, s, qw, sw)
            assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), f"call {t}: y"
        _check_state(ds, od, f"{path} call {t}")
    assert saturated > 0
