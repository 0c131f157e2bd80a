"""GPU parity of the E4M3 encoder and of fp8_quantize_act against the oracle:
codes, scale and amax must be bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from fp8_quantized_gemm_amd import fp8q, synth
from gpu_helpers import DEV, f32_bits, host, say

pytestmark = pytest.mark.gpu

CHUNK = 1 << 24


def _binades(e_lo, e_hi):
    """Every binary32 with magnitude in [2^e_lo, 2^e_hi)."""
    exps = np.arange(e_lo + 127, e_hi + 127, dtype=np.uint32)
    mant = np.arange(1 << 23, dtype=np.uint32)
    return ((exps[:, None] << 23) | mant[None, :]).ravel().view(np.float32)


def _check_encoder(v: np.ndarray, what: str):
    for i in range(0, v.size, CHUNK):
        c = np.ascontiguousarray(v[i:i + CHUNK])
        say("e4m3 encoder", what, i, c.size)
        got = host(fp8q.e4m3_encode_f32(torch.from_numpy(c).to(DEV)))
        want = oracle.e4m3_encode(c)
        if not np.array_equal(got, want):
            j = int(np.nonzero(got != want)[0][0])
            raise AssertionError(f"{what}: v={c[j]!r} ({f32_bits(c[j]):#010x}) gpu={got[j]:#04x} "
                                 f"oracle={want[j]:#04x}")


@pytest.mark.parametrize("e_lo,e_hi", [(-12, -5), (-1, 1), (7, 10)])
@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_encoder_exhaustive_binades(e_lo, e_hi, sign):
    """Every fp32 in the E4M3 subnormal range and first normal binades, around
    1.0 and at the top of the range (saturation), both signs."""
    _check_encoder(_binades(e_lo, e_hi) * np.float32(sign), f"[2^{e_lo},2^{e_hi}) x{sign}")


def test_encoder_specials_and_random():
    rng = np.random.Generator(np.random.PCG64(21))
    bits = rng.integers(0, 2**32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 448.0, -448.0, 464.0, 1e30, -1e30,
                         2.0**-149, -(2.0**-149), 2.0**-126, 3.4e38, 2.0**-10, -(2.0**-10)],
                        np.float32)
    # fp32 subnormals: a dense sample
    sub = (np.arange(0, 1 << 23, 97, dtype=np.uint32)).view(np.float32)
    _check_encoder(np.concatenate([specials, v, sub, -sub]), "specials+random")


def _quant_case(x: torch.Tensor, what: str, guard: int = 64):
    n = x.numel()
    code = oracle.BF16 if x.dtype == torch.bfloat16 else oracle.FP16
    xd = x.to(DEV)
    qbuf = torch.full((n + guard,), 0xAB, dtype=torch.uint8, device=DEV)
    sc = torch.full((2,), -7.0, dtype=torch.float32, device=DEV)
    am = torch.full((2,), 12345.0, dtype=torch.float32, device=DEV)
    say("quantize", what, n, x.dtype)
    fp8q.fp8_quantize_act(xd, qbuf[:n].view(x.shape), sc[:1], am[:1])
    q = host(qbuf)
    s, a = host(sc), host(am)
    wq, ws, wa = oracle.quantize(synth.bits(x).ravel(), code)
    assert f32_bits(a[0]) == f32_bits(wa), f"{what}: amax {a[0]} vs {wa}"
    assert f32_bits(s[0]) == f32_bits(ws), f"{what}: scale {s[0]} vs {ws}"
    if not np.array_equal(q[:n], wq):
        j = int(np.nonzero(q[:n] != wq)[0][0])
        raise AssertionError(f"{what}: code {j}: gpu {q[j]:#04x} oracle {wq[j]:#04x}")
    assert np.all(q[n:] == 0xAB), f"{what}: wrote past the end"
    assert s[1] == -7.0 and a[1] == 12345.0
    return q[:n]


SIZES = [1, 7, 8, 9, 1000, 4096, 4103, 32767, 32768, 32769, 8 * 11008, 98303, 98304, 98305,
         131071, 131072, 131073, 1_000_003]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_quantize_sizes(n, dtype):
    x = synth.activation(1, n, seed=synth.seed_for("qs", n, dtype), dtype=dtype).view(-1)
    _quant_case(x, f"n={n}")


@pytest.mark.parametrize("M,K", [(2048, 4096), (2048, 11008), (1024, 25600), (16, 25600)])
def test_quantize_full_size_with_outliers(M, K):
    x = synth.activation(M, K, seed=synth.seed_for("qo", M, K), outliers=True)
    _quant_case(x, f"outliers {M}x{K}")


def test_quantize_fp16_weights_full_size():
    w = synth.normal((4096, 4096), 0.02, "fp16", seed=synth.seed_for("w", 4096))
    _quant_case(w, "weights 4096x4096")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("n", [20_000, 70_000, 120_000])
def test_quantize_every_16bit_value_at_unit_scale(dtype, n):
    """All finite 16-bit values with |v| <= 448, plus 448 itself: amax = 448 so
    s = 1 and the codes are the plain encodings (small and large path)."""
    allv = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    t = synth.from_bits(allv, dtype).to(torch.float32).numpy()
    keep = allv[np.isfinite(t) & (np.abs(t) <= 448.0)]
    rng = np.random.Generator(np.random.PCG64(n))
    sel = np.resize(keep, n) if n > keep.size else rng.choice(keep, n, replace=False)
    b = sel.copy()
    b[0] = synth.bits(synth.from_bits(np.array([0], np.uint16), dtype) + 448.0)[0]
    _quant_case(synth.from_bits(b, dtype), f"unit-scale {dtype} n={n}")


def test_quantize_scaled_midpoints():
    """x = 2 * (every E4M3 midpoint and its bf16 neighbours); amax = 896 makes
    s = 2 exactly, so x/s lands exactly on the ties."""
    lo = oracle.e4m3_decode(np.arange(0x7E, dtype=np.uint8))
    hi = oracle.e4m3_decode(np.arange(1, 0x7F, dtype=np.uint8))
    mids = torch.from_numpy(((lo + hi) / 2 * 2).astype(np.float32)).to(torch.bfloat16)
    b = synth.bits(mids)
    vals = np.concatenate([b, b + 1, b - 1, b | 0x8000, (b + 1) | 0x8000]).astype(np.uint16)
    vals = np.concatenate([vals, synth.bits(torch.tensor([896.0], dtype=torch.bfloat16))])
    q = _quant_case(synth.from_bits(vals, "bf16"), "scaled midpoints")
    assert q[-1] == 0x7E


@pytest.mark.parametrize("n", [5, 50_000, 150_000])
def test_quantize_zero_and_constant(n):
    _quant_case(torch.zeros(n, dtype=torch.bfloat16), f"zeros n={n}")
    _quant_case(-torch.zeros(n, dtype=torch.float16), f"neg zeros n={n}")
    _quant_case(torch.full((n,), -0.3, dtype=torch.bfloat16), f"const n={n}")
    tiny = torch.full((n,), 1e-30, dtype=torch.bfloat16)
    tiny[n // 2] = 1e-28
    _quant_case(tiny, f"tiny n={n}")


@pytest.mark.parametrize("n", [600, 40_000, 120_000])
@pytest.mark.parametrize("below", [False, True])
def test_quantize_scale_threshold(n, below):
    """The device divides by s with a reciprocal and an FMA correction for
    2^-80 <= s <= 2^120 and with IEEE division otherwise.  amax = 1.75 * 2^-72
    gives s = 2^-80 exactly (first path); one bf16 step lower gives the
    second.  The rest: random magnitudes over 40 binades below amax, both
    signs, +-0 and bf16 subnormals (codes must match the oracle's division)."""
    rng = np.random.Generator(np.random.PCG64(n + below))
    top = torch.tensor([1.75 * 2.0 ** -72], dtype=torch.bfloat16)
    tb = int(synth.bits(top)[0]) - (1 if below else 0)
    mag = 2.0 ** rng.uniform(-112, -72.5, n)
    vals = torch.from_numpy((mag * rng.choice([-1.0, 1.0], n)).astype(np.float32)).to(torch.bfloat16)
    b = synth.bits(vals).copy()
    b[:4] = [0x0000, 0x8000, 0x0001, 0x8003]           # +0, -0, subnormals
    b[n // 2] = tb
    _quant_case(synth.from_bits(b, "bf16"), f"threshold below={below} n={n}")


def test_quantize_deterministic_large_path():
    x = synth.activation(512, 11008, seed=3, outliers=True).to(DEV)
    say("quantize determinism")
    q1, s1, a1 = fp8q.fp8_quantize_act(x)
    q2, s2, a2 = fp8q.fp8_quantize_act(x)
    assert torch.equal(q1, q2) and torch.equal(s1, s2) and torch.equal(a1, a2)
