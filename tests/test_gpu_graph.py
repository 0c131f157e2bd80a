"""The library's calls captured into a HIP graph (how bench.py times them):
every replay must reproduce the eager results bit-exactly.  Between replays
the outputs are overwritten eagerly and the device is synchronized, so a
replay that skipped or reordered work, or a captured memory operation that
misbehaves on later replays, shows up as a mismatch.  Covers each launch
pattern of the path: the fused decode linear (M = 1), the one-launch
quantizing GEMV (M = 4, 8, 16, with one to three tiles per workgroup), the
partial-maxima quantizer + MFMA GEMV (M = 4 on the down projection) and
+ tile GEMM (M = 512), the
stand-alone quantizer's atomic path (its amax is cleared by a kernel, not a
memset), and both NestedFP modes."""
import pytest
import torch

from fp8_quantized_gemm_amd import fp8q, synth
from gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _weights(N, K, seed):
    w = synth.normal((N, K), 0.02, "fp16", seed=seed, device=DEV)
    qw, sw, _ = fp8q.fp8_quantize_act(w)
    return w, qw, sw


def _check_graph(calls, outs):
    """Run `calls` eagerly, capture them, then replay REPLAYS times with the
    outputs scrambled before each replay; every replay equals the eager run."""
    calls()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        calls()
    for rep in range(REPLAYS):
        for o in outs:                            # eager work between replays
            if o.dtype in (torch.uint8,):
                o.fill_(0x55)
            else:
                o.view(torch.uint8).fill_(0x7f)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o.view(torch.uint8), w.view(torch.uint8)), f"replay {rep}"
    del g


@pytest.mark.parametrize("M,K,N", [(1, 4096, 4096), (4, 4096, 12288), (4, 11008, 4096),
                                   (8, 4096, 4096), (16, 4096, 22016),
                                   (512, 4096, 12288), (512, 11008, 4096)])
def test_fp8_linear_graph_replays(M, K, N):
    _, qw, sw = _weights(N, K, seed=synth.seed_for("graph-w", M, K, N))
    x = synth.activation(M, K, seed=synth.seed_for("graph-x", M, K, N), outliers=M > 16, device=DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    q = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    s = torch.empty(1, dtype=torch.float32, device=DEV)
    a = torch.empty(1, dtype=torch.float32, device=DEV)
    say("graph fp8_linear", M, K, N)
    _check_graph(lambda: fp8q.fp8_linear(x, qw, sw, y, q, s, a), [y, q, s, a])


def test_quantize_atomic_path_and_gemm_graph_replays():
    M, K, N = 300, 5120, 2048          # 1.5 M elements: init kernel + atomic amax + quantize
    _, qw, sw = _weights(N, K, seed=11)
    x = synth.activation(M, K, seed=12, outliers=True, device=DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    q = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    s = torch.empty(1, dtype=torch.float32, device=DEV)
    a = torch.empty(1, dtype=torch.float32, device=DEV)

    def calls():
        fp8q.fp8_quantize_act(x, q, s, a)
        fp8q.fp8_gemm(q, s, qw, sw, y)

    say("graph quantize + gemm", M, K, N)
    _check_graph(calls, [y, q, s, a])


@pytest.mark.parametrize("M,K,N", [(1, 4096, 12288), (256, 4096, 4096)])
def test_nested_modes_graph_replays(M, K, N):
    w = synth.normal((N, K), 0.02, "fp16", seed=synth.seed_for("graph-n", M, K, N), device=DEV)
    hi, lo = fp8q.nested_split(w)
    a16 = synth.activation(M, K, seed=synth.seed_for("graph-a", M, K, N), dtype="fp16", device=DEV)
    y16 = torch.empty((M, N), dtype=torch.float16, device=DEV)
    y8 = torch.empty((M, N), dtype=torch.float16, device=DEV)
    q = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    s = torch.empty(1, dtype=torch.float32, device=DEV)
    a = torch.empty(1, dtype=torch.float32, device=DEV)

    def calls():
        fp8q.nested_gemm_fp16(a16, hi, lo, y16)
        fp8q.nested_linear_fp8(a16, hi, y8, q, s, a)

    say("graph nested", M, K, N)
    _check_graph(calls, [y16, y8, q, s, a])
