"""GPU parity of the FP8 KV-cache quantizer (fp8_quantize_kv) against the
oracle: codes, per-head scales and amax bit-exact, on the one-launch path
(heads of at most 32768 elements, held in registers) and the three-launch path
(heads split over several workgroups, partial maxima kept in the code buffer),
whose last pass is token-major for 256..2048 vectors of 8 elements per token
(257 x 32 x 128, 1024 x 40 x 64, 512 x 40 x 80) and head-major otherwise
(4096 x 8 x 128, 300 x 64 x 512); GQA-sized and MHA-sized head counts, head
dimensions 8..512 (80: not a power of two), bf16 and fp16, outlier channels
and an all-zero head."""
import numpy as np
import pytest
import torch

import oracle
from fp8_quantized_gemm_amd import fp8q, synth
from gpu_helpers import DEV, host, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("T,H,D", [(1, 32, 128), (17, 8, 128), (256, 32, 128), (257, 32, 128),
                                   (4096, 8, 128), (3, 4, 8), (1024, 40, 64), (100, 1, 16),
                                   (512, 40, 80), (300, 64, 512), (4099, 16, 128)])
def test_quantize_kv_bit_exact(T, H, D, dtype):
    x = synth.activation(T, H * D, seed=synth.seed_for("gkv", T, H, D, dtype), dtype=dtype,
                         outliers=True).reshape(T, H, D)
    if H > 2:
        x[:, 1, :] = 0.0                       # an all-zero head: scale 1, codes 0
    code = oracle.BF16 if dtype == "bf16" else oracle.FP16
    want_q, want_s, want_a = oracle.quantize_kv(synth.bits(x), code)
    say("quantize_kv", dtype, T, H, D)
    q, s, a = fp8q.fp8_quantize_kv(x.to(DEV))
    assert np.array_equal(host(q), want_q)
    assert np.array_equal(host(s).view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(host(a).view(np.uint32), want_a.view(np.uint32))


@pytest.mark.parametrize("T,H,D", [(2048, 8, 128), (2047, 32, 128)])
def test_quantize_kv_graph_replays(T, H, D):
    x = synth.activation(T, H * D, seed=3, outliers=True).reshape(T, H, D).to(DEV)
    q = torch.empty((T, H, D), dtype=torch.uint8, device=DEV)
    s = torch.empty(H, device=DEV)
    a = torch.empty(H, device=DEV)
    fp8q.fp8_quantize_kv(x, q, s, a)
    torch.cuda.synchronize()
    want = [t.clone() for t in (q, s, a)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fp8q.fp8_quantize_kv(x, q, s, a)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("quantize_kv graph", T, H, D)
    with torch.cuda.graph(g):
        fp8q.fp8_quantize_kv(x, q, s, a)
    for rep in range(3):
        for t in (q, s, a):
            t.view(torch.uint8).fill_(0x7f)      # outputs scrambled between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, w in zip((q, s, a), want):
            assert torch.equal(t.view(torch.uint8), w.view(torch.uint8)), f"replay {rep}"
    del g
