"""Pins for the oracle's FP8 KV-cache quantizer (CPU only).

A K or V block x[T, H, D] gets one scale per head h (over all tokens and the
head dimension).  What fixes it here:
- head h equals the library-routine quantizer (numpy max, binary32 division,
  torch's float8_e4m3fn cast) applied to numpy's gather x[:, h, :];
- heads that are copies of head 0 times 2^e give identical codes and scales
  exactly 2^e apart, so a head / token index slip fails;
- one head is the per-tensor quantizer of the whole block.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_quantized_gemm_amd import synth


def _lib_quantize(v: np.ndarray):
    amax = np.float32(np.max(np.abs(v)))
    s = amax / np.float32(448.0) if amax > 0 else np.float32(1.0)
    t = (v / s).astype(np.float32)
    assert np.all(np.abs(t) < 464.0)
    return torch.from_numpy(t.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy(), s, amax


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("T,H,D", [(1, 4, 16), (7, 3, 32), (64, 8, 128)])
def test_heads_match_library_quantizer(T, H, D, dtype):
    x = synth.activation(T, H * D, seed=synth.seed_for("kv", T, H, D, dtype), dtype=dtype,
                         outliers=True).reshape(T, H, D)
    code = oracle.BF16 if dtype == "bf16" else oracle.FP16
    q, s, a = oracle.quantize_kv(synth.bits(x), code)
    v = x.to(torch.float32).numpy()
    for h in range(H):
        qh, sh, ah = _lib_quantize(v[:, h, :].ravel())
        assert np.array_equal(q[:, h, :].ravel(), qh), f"head {h}"
        assert s[h] == sh and a[h] == ah


def test_heads_two_to_the_e_apart():
    T, H, D = 9, 5, 64
    base = synth.activation(T, D, seed=3, outliers=True).to(torch.float32)
    e = [0, 4, -3, 7, -6]
    x = torch.stack([base * float(2.0 ** k) for k in e], dim=1).to(torch.bfloat16)   # [T, H, D]
    q, s, a = oracle.quantize_kv(synth.bits(x), oracle.BF16)
    for h, k in enumerate(e):
        assert np.array_equal(q[:, h, :], q[:, 0, :])
        assert s[h] == np.float32(s[0] * 2.0 ** k) and a[h] == np.float32(a[0] * 2.0 ** k)


def test_one_head_is_the_per_tensor_quantizer():
    x = synth.activation(33, 128, seed=5, outliers=True).reshape(33, 1, 128)
    q, s, a = oracle.quantize_kv(synth.bits(x), oracle.BF16)
    qt, st, at = oracle.quantize(synth.bits(x).ravel(), oracle.BF16)
    assert np.array_equal(q.ravel(), qt) and (s[0], a[0]) == (st, at)
