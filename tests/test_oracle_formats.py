"""Pins for the oracle's number formats (CPU only).

Each check compares the oracle with something other than itself: torch's and
numpy's own float8 / float16 / bfloat16 conversions (library routines), the
hand-worked encodings in tests/golden/e4m3_handpicked.txt, and invariants of
the format definitions (round trip, monotonicity, tie-to-even at every
midpoint).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _torch_e4m3_encode(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


ALL8 = np.arange(256, dtype=np.uint8)
ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def test_rounding_mode_is_nearest():
    assert oracle.lib.orc_rounding_is_nearest() == 1


# ----------------------------------------------------------------- E4M3 decode
def test_e4m3_decode_matches_torch_all_codes():
    ours = oracle.e4m3_decode(ALL8)
    lib = _torch_e4m3_decode(ALL8)
    nan_ours = np.isnan(ours)
    assert np.array_equal(nan_ours, np.isnan(lib))
    assert sorted(np.nonzero(nan_ours)[0].tolist()) == [0x7F, 0xFF]
    assert np.array_equal(ours[~nan_ours], lib[~nan_ours])
    # signed zero
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_e4m3_decode_monotone_and_bounds():
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    assert pos[0x7E] == 448.0
    assert pos[0x01] == 2.0 ** -9
    assert pos[0x08] == 2.0 ** -6
    neg = oracle.e4m3_decode(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos)


# ----------------------------------------------------------------- E4M3 encode
def test_e4m3_roundtrip_all_codes():
    vals = oracle.e4m3_decode(ALL8)
    ok = ~np.isnan(vals)
    back = oracle.e4m3_encode(vals[ok].astype(np.float32))
    assert np.array_equal(back, ALL8[ok])


def test_e4m3_every_midpoint_ties_to_even():
    for sign in (1.0, -1.0):
        codes = np.arange(0x7E, dtype=np.uint8)          # pairs (c, c+1), c+1 <= 0x7E
        lo = oracle.e4m3_decode(codes)
        hi = oracle.e4m3_decode(codes + 1)
        mid = ((lo + hi) / 2).astype(np.float32)          # 5 significant bits: exact
        assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
        even = np.where(codes % 2 == 0, codes, codes + 1).astype(np.uint8)
        sb = np.uint8(0x80) if sign < 0 else np.uint8(0)
        got = oracle.e4m3_encode(sign * mid)
        assert np.array_equal(got, even | sb)
        up = np.nextafter(mid, np.float32(np.inf))
        dn = np.nextafter(mid, np.float32(0))
        assert np.array_equal(oracle.e4m3_encode(sign * up), (codes + 1) | sb)
        assert np.array_equal(oracle.e4m3_encode(sign * dn), codes | sb)


def _golden_e4m3():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_handpicked.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            v, c = line.split()
            if v in ("inf", "-inf", "nan"):
                fv = float(v)
            else:
                fv = float.fromhex(v)
            rows.append((fv, int(c, 16)))
    return rows


def test_e4m3_handpicked_golden():
    rows = _golden_e4m3()
    assert len(rows) >= 20
    vals = np.array([r[0] for r in rows], np.float32)
    want = np.array([r[1] for r in rows], np.uint8)
    assert np.array_equal(oracle.e4m3_encode(vals), want)


def test_e4m3_encode_matches_torch_on_16bit_grids():
    # every finite bf16 and fp16 value with |v| <= 448 (torch does not saturate
    # above that, so saturation is pinned by the golden cases instead)
    for dt in (torch.bfloat16, torch.float16):
        t = torch.from_numpy(ALL16.view(np.int16).copy()).view(dt).to(torch.float32)
        v = t.numpy()
        keep = np.isfinite(v) & (np.abs(v) <= 448.0)
        v = v[keep]
        assert np.array_equal(oracle.e4m3_encode(v), _torch_e4m3_encode(v))


def test_e4m3_encode_matches_torch_on_random_f32():
    rng = np.random.Generator(np.random.PCG64(1234))
    # log-uniform magnitudes from 2^-14 to 448 with full 23-bit mantissas
    mag = np.exp2(rng.uniform(-14.0, math.log2(448.0), size=400_000)).astype(np.float32)
    sgn = np.where(rng.random(mag.size) < 0.5, -1.0, 1.0).astype(np.float32)
    v = (mag * sgn).astype(np.float32)
    v = v[np.abs(v) <= 448.0]
    assert np.array_equal(oracle.e4m3_encode(v), _torch_e4m3_encode(v))


# ----------------------------------------------------------------- E5M2
def test_e5m2_decode_is_fp16_of_upper_byte():
    ours = oracle.e5m2_decode(ALL8)
    as_half = (ALL8.astype(np.uint16) << 8).view(np.float16).astype(np.float64)
    lib = torch.from_numpy(ALL8.copy()).view(torch.float8_e5m2).to(torch.float64).numpy()
    for ref in (as_half, lib):
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(ours), nan)
        assert np.array_equal(ours[~nan], ref[~nan])


# ----------------------------------------------------------------- fp16
def test_f16_decode_all_patterns():
    ours = oracle.f16_decode(ALL16)
    lib = ALL16.view(np.float16).astype(np.float64)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(lib[~nan]))


def test_f16_encode_matches_numpy():
    rng = np.random.Generator(np.random.PCG64(7))
    bits = rng.integers(0, 2**32, size=500_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    # every fp16 midpoint and its neighbours
    h = np.arange(0x7BFF, dtype=np.uint16)
    a = h.view(np.float16).astype(np.float64)
    b = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mids = ((a + b) / 2).astype(np.float32)
    extra = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)),
                            np.nextafter(mids, np.float32(0)), -mids,
                            np.array([65504, 65519.996, 65520, 1e9, np.inf, -np.inf, 0.0, -0.0,
                                      2.0**-24, 2.0**-25, 2.0**-25 * 1.0000001, 2.0**-26],
                                     np.float32)])
    v = np.concatenate([v, extra]).astype(np.float32)
    ours = oracle.f16_encode(v)
    lib = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, lib)


# ----------------------------------------------------------------- bf16
def test_bf16_decode_all_patterns():
    ours = oracle.bf16_decode(ALL16)
    lib = torch.from_numpy(ALL16.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), lib[~nan].view(np.uint32))


def test_bf16_encode_matches_torch():
    rng = np.random.Generator(np.random.PCG64(8))
    bits = rng.integers(0, 2**32, size=500_000, dtype=np.uint64).astype(np.uint32)
    # plus every exact bf16 midpoint in a band of exponents, and its neighbours
    mant = np.arange(1 << 16, dtype=np.uint32)
    ties = (mant << 15) | 0x3F800000  # values in [1,2) with the tie bit pattern
    ties = (ties & 0xFFFF8000) | 0x8000
    v = np.concatenate([bits, ties, ties + 1, ties - 1]).astype(np.uint32).view(np.float32)
    v = v[~np.isnan(v)]
    ours = oracle.bf16_encode(v)
    lib = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, lib)
    assert oracle.bf16_encode(np.array([np.nan], np.float32))[0] == 0x7FC0


# ----------------------------------------------------------------- mutation check
@pytest.mark.parametrize("bad_code", [0x77, 0x7E])
def test_pins_detect_fnuz_variant(bad_code):
    """The FNUZ variant (bias 8, max 240) would decode 0x77 / 0x7E differently;
    make sure the pins above tell the two apart."""
    fnuz = {0x77: 2.0 ** (14 - 8) * 1.875, 0x7E: 2.0 ** (15 - 8) * 1.75}
    assert oracle.e4m3_decode(np.array([bad_code], np.uint8))[0] != fnuz[bad_code]
