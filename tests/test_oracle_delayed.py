"""Pins for the oracle's delayed scaling with an amax history (CPU only).

The page on a 7B model on an RTX 4060 (§6.1) asks that the amax history be at
least 1024 long.  The oracle keeps a ring of the last L amax values; what fixes
it here, independently of the ring:
- the scale of call t is the closed form max(amax of calls t-L .. t-1) / 448
  (1 for the first call), computed from the list of earlier tensors with numpy;
- the codes are the library cast (torch's float8_e4m3fn) of fl32(x / s)
  clamped to +-448, so values beyond 448 s saturate;
- amax is numpy's max |x|.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_quantized_gemm_amd import synth


def _lib_codes(v: np.ndarray, s: np.float32) -> np.ndarray:
    t = np.clip((v / s).astype(np.float32), -448.0, 448.0)
    return torch.from_numpy(t.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _window_scale(amaxes, t, L):
    past = amaxes[max(0, t - L):t]
    if not past:
        return np.float32(1.0)
    m = np.float32(max(past))
    return m / np.float32(448.0) if m > 0 else np.float32(1.0)


@pytest.mark.parametrize("L,calls", [(1, 6), (3, 9), (1024, 12)])
def test_scales_follow_the_window_closed_form(L, calls):
    d = oracle.DelayedScaling(L)
    # magnitudes that rise, fall and jump, so the window maximum changes
    mags = [1.0, 3.0, 0.25, 40.0, 0.5, 0.5, 2.0, 0.125, 8.0, 1.0, 16.0, 0.01][:calls]
    amaxes = []
    for t, mag in enumerate(mags):
        x = (synth.activation(4, 256, seed=100 + t, outliers=True).to(torch.float32) * mag
             ).to(torch.bfloat16)
        v = x.to(torch.float32).numpy().ravel()
        q, s, a = d.quantize(synth.bits(x).ravel(), oracle.BF16)
        want_s = _window_scale(amaxes, t, L)
        assert np.float32(s) == want_s, f"call {t}"
        assert np.float32(a) == np.float32(np.max(np.abs(v)))
        assert np.array_equal(q, _lib_codes(v, want_s)), f"call {t}"
        amaxes.append(float(a))
        assert d.position == (t + 1) % L


def test_large_tensor_after_small_history_saturates():
    d = oracle.DelayedScaling(16)
    small = synth.activation(1, 512, seed=1).to(torch.float32)
    d.quantize(synth.bits((small * 0.01).to(torch.bfloat16)).ravel(), oracle.BF16)
    big = (small * 10.0).to(torch.bfloat16)
    q, s, a = d.quantize(synth.bits(big).ravel(), oracle.BF16)
    v = big.to(torch.float32).numpy().ravel()
    over = np.abs(v / np.float32(s)) > 448.0
    assert over.sum() > 100                              # most elements saturate
    assert np.all((q[over] & 0x7F) == 0x7E)              # +-448
    assert np.array_equal(q, _lib_codes(v, np.float32(s)))
    # the next call already uses the large amax
    assert d.next_scale == np.float32(a) / np.float32(448.0)


def test_zero_tensors_keep_unit_scale_and_fp16_input():
    d = oracle.DelayedScaling(4)
    z = np.zeros(64, np.uint16)
    for _ in range(3):
        q, s, a = d.quantize(z, oracle.FP16)
        assert s == 1.0 and a == 0.0 and np.all(q == 0)
    w = synth.normal((8, 64), 0.02, "fp16", seed=5)
    q, s, a = d.quantize(synth.bits(w).ravel(), oracle.FP16)
    assert s == 1.0                                     # history held only zeros
    assert np.array_equal(q, _lib_codes(w.to(torch.float32).numpy().ravel(), np.float32(1.0)))
    q2, s2, _ = d.quantize(synth.bits(w).ravel(), oracle.FP16)
    assert np.float32(s2) == np.float32(a) / np.float32(448.0)
    # with the scale of its own amax, the delayed codes equal the current-scaling codes
    qc, sc, _ = oracle.quantize(synth.bits(w).ravel(), oracle.FP16)
    assert s2 == sc and np.array_equal(q2, qc)
