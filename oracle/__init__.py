"""Python face of the fp8q oracle (plain C in ``oracle.c``, loaded with ctypes).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the product path.  It shares
no code with the HIP library.

All arrays are numpy arrays; 16-bit floating-point tensors travel as their
uint16 bit patterns, FP8 tensors as uint8 codes.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

BF16 = 0
FP16 = 1

_c = ctypes
_p = _c.c_void_p
_i64 = _c.c_int64


def _load():
    if not os.path.exists(_LIB_PATH):
        from . import build as _build  # noqa: WPS433 (build on first use)
        _build.build()
    lib = _c.CDLL(_LIB_PATH)
    sig = {
        "orc_bf16_decode": (_c.c_float, [_c.c_uint16]),
        "orc_bf16_encode": (_c.c_uint16, [_c.c_float]),
        "orc_f16_decode": (_c.c_double, [_c.c_uint16]),
        "orc_f16_encode": (_c.c_uint16, [_c.c_float]),
        "orc_e4m3_decode": (_c.c_double, [_c.c_uint8]),
        "orc_e4m3_encode": (_c.c_uint8, [_c.c_float]),
        "orc_e5m2_decode": (_c.c_double, [_c.c_uint8]),
        "orc_amax": (_c.c_float, [_p, _c.c_int, _i64]),
        "orc_scale_from_amax": (_c.c_float, [_c.c_float]),
        "orc_quantize_with_scale": (None, [_p, _c.c_int, _i64, _c.c_float, _p]),
        "orc_quantize": (None, [_p, _c.c_int, _i64, _p, _p, _p]),
        "orc_quantize_rows": (None, [_p, _c.c_int, _i64, _i64, _p, _p, _p]),
        "orc_quantize_delayed": (None, [_p, _c.c_int, _i64, _p, _p, _p, _p, _i64, _p]),
        "orc_quantize_kv": (None, [_p, _c.c_int, _i64, _i64, _i64, _p, _p, _p]),
        "orc_nested_split_e4m3": (_i64, [_p, _p, _p, _i64]),
        "orc_nested_rebuild_e4m3": (None, [_p, _p, _p, _i64]),
        "orc_gemm_fp8_f32_fp16out": (None, [_p, _c.c_float, _p, _c.c_float, _i64, _i64, _i64,
                                            _p, _c.c_int]),
        "orc_gemm_fp8_rowwise_ref": (None, [_p, _p, _p, _p, _i64, _i64, _i64,
                                            _p, _p, _i64, _p, _p]),
        "orc_gemm_fp8_rowwise_f32": (None, [_p, _p, _p, _p, _i64, _i64, _i64, _p, _c.c_int]),
        "orc_nested_split": (None, [_p, _p, _p, _i64]),
        "orc_nested_rebuild": (None, [_p, _p, _p, _i64]),
        "orc_gemm_fp8_ref": (None, [_p, _c.c_float, _p, _c.c_float, _i64, _i64, _i64,
                                    _p, _p, _i64, _p, _p]),
        "orc_nested_fp16_ref": (None, [_p, _p, _p, _i64, _i64, _i64, _p, _p, _i64, _p, _p]),
        "orc_nested_fp8_ref": (None, [_p, _c.c_float, _p, _i64, _i64, _i64,
                                      _p, _p, _i64, _p, _p]),
        "orc_gemm_fp8_f32": (None, [_p, _c.c_float, _p, _c.c_float, _i64, _i64, _i64,
                                    _p, _c.c_int]),
        "orc_nested_fp16_f32": (None, [_p, _p, _p, _i64, _i64, _i64, _p, _c.c_int]),
        "orc_nested_fp8_f32": (None, [_p, _c.c_float, _p, _i64, _i64, _i64, _p, _c.c_int]),
        "orc_rounding_is_nearest": (_c.c_int, []),
        "orc_set_ref_threads": (None, [_c.c_int]),
        "orc_e4m3_encode_array": (None, [_p, _p, _i64]),
        "orc_e4m3_decode_array": (None, [_p, _p, _i64]),
        "orc_e5m2_decode_array": (None, [_p, _p, _i64]),
        "orc_f16_decode_array": (None, [_p, _p, _i64]),
        "orc_f16_encode_array": (None, [_p, _p, _i64]),
        "orc_bf16_decode_array": (None, [_p, _p, _i64]),
        "orc_bf16_encode_array": (None, [_p, _p, _i64]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def set_ref_threads(n: int):
    """Threads the fp64 checkers may use (they split the list of (m, n) pairs)."""
    lib.orc_set_ref_threads(int(n))


set_ref_threads(max(1, min(16, len(os.sched_getaffinity(0)))))


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(_p)


def _c_arr(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- codecs
def e4m3_encode(v) -> np.ndarray:
    """binary32 values -> E4M3 codes (RNE, saturating to +-448, NaN -> 0x7F|s)."""
    v = _c_arr(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib.orc_e4m3_encode_array(_ptr(v), _ptr(out), v.size)
    return out


def e4m3_decode(c) -> np.ndarray:
    c = _c_arr(c, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib.orc_e4m3_decode_array(_ptr(c), _ptr(out), c.size)
    return out


def e5m2_decode(c) -> np.ndarray:
    c = _c_arr(c, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib.orc_e5m2_decode_array(_ptr(c), _ptr(out), c.size)
    return out


def f16_decode(h) -> np.ndarray:
    h = _c_arr(h, np.uint16)
    out = np.empty(h.shape, np.float64)
    lib.orc_f16_decode_array(_ptr(h), _ptr(out), h.size)
    return out


def f16_encode(v) -> np.ndarray:
    v = _c_arr(v, np.float32)
    out = np.empty(v.shape, np.uint16)
    lib.orc_f16_encode_array(_ptr(v), _ptr(out), v.size)
    return out


def bf16_decode(b) -> np.ndarray:
    b = _c_arr(b, np.uint16)
    out = np.empty(b.shape, np.float32)
    lib.orc_bf16_decode_array(_ptr(b), _ptr(out), b.size)
    return out


def bf16_encode(v) -> np.ndarray:
    v = _c_arr(v, np.float32)
    out = np.empty(v.shape, np.uint16)
    lib.orc_bf16_encode_array(_ptr(v), _ptr(out), v.size)
    return out


# ---------------------------------------------------------------- quantizer
def amax(x_bits, dtype: int) -> float:
    x = _c_arr(x_bits, np.uint16)
    return float(lib.orc_amax(_ptr(x), dtype, x.size))


def scale_from_amax(a: float) -> float:
    return float(lib.orc_scale_from_amax(a))


def quantize_with_scale(x_bits, dtype: int, s: float) -> np.ndarray:
    x = _c_arr(x_bits, np.uint16)
    q = np.empty(x.shape, np.uint8)
    lib.orc_quantize_with_scale(_ptr(x), dtype, x.size, s, _ptr(q))
    return q


def quantize(x_bits, dtype: int):
    """Returns (codes, scale, amax) for a bf16/fp16 tensor given as uint16 bits."""
    x = _c_arr(x_bits, np.uint16)
    q = np.empty(x.shape, np.uint8)
    s = np.zeros(1, np.float32)
    a = np.zeros(1, np.float32)
    lib.orc_quantize(_ptr(x), dtype, x.size, _ptr(q), _ptr(s), _ptr(a))
    return q, float(s[0]), float(a[0])


def quantize_rows(x_bits, dtype: int):
    """Per-row quantization of a [rows, cols] bf16/fp16 matrix (uint16 bits):
    returns (codes [rows, cols], scale float32 [rows], amax float32 [rows])."""
    x = _c_arr(x_bits, np.uint16)
    assert x.ndim == 2
    rows, cols = x.shape
    q = np.empty(x.shape, np.uint8)
    s = np.zeros(rows, np.float32)
    a = np.zeros(rows, np.float32)
    lib.orc_quantize_rows(_ptr(x), dtype, rows, cols, _ptr(q), _ptr(s), _ptr(a))
    return q, s, a


def quantize_kv(x_bits, dtype: int):
    """Per-head quantization of a K or V block [T, H, D] (uint16 bits): returns
    (codes [T, H, D], scale float32 [H], amax float32 [H])."""
    x = _c_arr(x_bits, np.uint16)
    assert x.ndim == 3
    T, H, D = x.shape
    q = np.empty(x.shape, np.uint8)
    s = np.zeros(H, np.float32)
    a = np.zeros(H, np.float32)
    lib.orc_quantize_kv(_ptr(x), dtype, T, H, D, _ptr(q), _ptr(s), _ptr(a))
    return q, s, a


class DelayedScaling:
    """Delayed scaling with an amax history of `length` calls (state kept on
    the host): each call quantizes with the scale the earlier calls' amax
    history gives (1 before any call), then records its own amax."""

    def __init__(self, length: int):
        assert length >= 1
        self.history = np.zeros(length, np.float32)
        self.state = np.zeros(4, np.uint32)          # [next scale bits, 0, position, 0]

    @property
    def next_scale(self) -> float:
        return float(self.state[:1].view(np.float32)[0])

    @property
    def position(self) -> int:
        return int(self.state[2])

    def quantize(self, x_bits, dtype: int):
        """Returns (codes, scale used, amax of x) and advances the history."""
        x = _c_arr(x_bits, np.uint16)
        q = np.empty(x.shape, np.uint8)
        s = np.zeros(1, np.float32)
        a = np.zeros(1, np.float32)
        lib.orc_quantize_delayed(_ptr(x), dtype, x.size, _ptr(q), _ptr(s), _ptr(a),
                                 _ptr(self.history), self.history.size, _ptr(self.state))
        return q, float(s[0]), float(a[0])


# ---------------------------------------------------------------- NestedFP
def nested_split(w_bits):
    w = _c_arr(w_bits, np.uint16)
    hi = np.empty(w.shape, np.uint8)
    lo = np.empty(w.shape, np.uint8)
    lib.orc_nested_split(_ptr(w), _ptr(hi), _ptr(lo), w.size)
    return hi, lo


def nested_rebuild(hi, lo):
    hi = _c_arr(hi, np.uint8)
    lo = _c_arr(lo, np.uint8)
    assert hi.shape == lo.shape
    w = np.empty(hi.shape, np.uint16)
    lib.orc_nested_rebuild(_ptr(hi), _ptr(lo), _ptr(w), hi.size)
    return w


def nested_split_e4m3(w_bits):
    """E4M3 upper-byte split: returns (hi, lo, number of words outside the FP8
    mode's range |w| < 1.875)."""
    w = _c_arr(w_bits, np.uint16)
    hi = np.empty(w.shape, np.uint8)
    lo = np.empty(w.shape, np.uint8)
    bad = lib.orc_nested_split_e4m3(_ptr(w), _ptr(hi), _ptr(lo), w.size)
    return hi, lo, int(bad)


def nested_rebuild_e4m3(hi, lo):
    hi = _c_arr(hi, np.uint8)
    lo = _c_arr(lo, np.uint8)
    assert hi.shape == lo.shape
    w = np.empty(hi.shape, np.uint16)
    lib.orc_nested_rebuild_e4m3(_ptr(hi), _ptr(lo), _ptr(w), hi.size)
    return w


NESTED_E4M3_SCALE = 2.0 ** -8      # weight scale of the E4M3 upper byte


def gemm_fp8_f32_fp16out(qa, sa, qw, sw, nthreads=None):
    """The fp32-accumulating E4M3 x E4M3 GEMM with fp16 output:
    y = fp16(acc * fl32(sa * sw)); returns fp16 bits [M,N]."""
    qa = _c_arr(qa, np.uint8)
    qw = _c_arr(qw, np.uint8)
    M, K = qa.shape
    N, _ = qw.shape
    y = np.empty((M, N), np.uint16)
    lib.orc_gemm_fp8_f32_fp16out(_ptr(qa), sa, _ptr(qw), sw, M, N, K, _ptr(y),
                                 nthreads or default_threads())
    return y


# ---------------------------------------------------------------- GEMM checkers
def _pairs(M, N, ms, ns):
    if ms is None:
        mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        ms, ns = mm.ravel(), nn.ravel()
    ms = _c_arr(ms, np.int64)
    ns = _c_arr(ns, np.int64)
    assert ms.shape == ns.shape
    assert ms.size == 0 or (ms.min() >= 0 and ms.max() < M and ns.min() >= 0 and ns.max() < N)
    return ms, ns


def gemm_fp8_ref(qa, sa, qw, sw, ms=None, ns=None):
    """fp64 (ref, absref) of the FP8 GEMM at (ms[i], ns[i]) (all of [M,N] if None)."""
    qa = _c_arr(qa, np.uint8)
    qw = _c_arr(qw, np.uint8)
    M, K = qa.shape
    N, K2 = qw.shape
    assert K == K2
    ms, ns = _pairs(M, N, ms, ns)
    ref = np.empty(ms.size, np.float64)
    ab = np.empty(ms.size, np.float64)
    lib.orc_gemm_fp8_ref(_ptr(qa), sa, _ptr(qw), sw, M, N, K, _ptr(ms), _ptr(ns), ms.size,
                         _ptr(ref), _ptr(ab))
    return ref, ab


def nested_fp16_ref(a16, hi, lo, ms=None, ns=None):
    a16 = _c_arr(a16, np.uint16)
    hi = _c_arr(hi, np.uint8)
    lo = _c_arr(lo, np.uint8)
    M, K = a16.shape
    N, K2 = hi.shape
    assert K == K2 and lo.shape == hi.shape
    ms, ns = _pairs(M, N, ms, ns)
    ref = np.empty(ms.size, np.float64)
    ab = np.empty(ms.size, np.float64)
    lib.orc_nested_fp16_ref(_ptr(a16), _ptr(hi), _ptr(lo), M, N, K, _ptr(ms), _ptr(ns),
                            ms.size, _ptr(ref), _ptr(ab))
    return ref, ab


def nested_fp8_ref(qa, sa, hi, ms=None, ns=None):
    qa = _c_arr(qa, np.uint8)
    hi = _c_arr(hi, np.uint8)
    M, K = qa.shape
    N, K2 = hi.shape
    assert K == K2
    ms, ns = _pairs(M, N, ms, ns)
    ref = np.empty(ms.size, np.float64)
    ab = np.empty(ms.size, np.float64)
    lib.orc_nested_fp8_ref(_ptr(qa), sa, _ptr(hi), M, N, K, _ptr(ms), _ptr(ns), ms.size,
                           _ptr(ref), _ptr(ab))
    return ref, ab


def gemm_fp8_rowwise_ref(qa, sa, qw, sw, ms=None, ns=None):
    """fp64 (ref, absref) of the FP8 GEMM with scales sa[M] per activation row
    and sw[N] per weight row, at (ms[i], ns[i]) (all of [M,N] if None)."""
    qa = _c_arr(qa, np.uint8)
    qw = _c_arr(qw, np.uint8)
    M, K = qa.shape
    N, K2 = qw.shape
    assert K == K2
    sa = _c_arr(sa, np.float32)
    sw = _c_arr(sw, np.float32)
    assert sa.shape == (M,) and sw.shape == (N,)
    ms, ns = _pairs(M, N, ms, ns)
    ref = np.empty(ms.size, np.float64)
    ab = np.empty(ms.size, np.float64)
    lib.orc_gemm_fp8_rowwise_ref(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), M, N, K, _ptr(ms),
                                 _ptr(ns), ms.size, _ptr(ref), _ptr(ab))
    return ref, ab


def gemm_fp8_rowwise_f32(qa, sa, qw, sw, nthreads=None):
    """The plain fp32-accumulating FP8 GEMM with scales sa[M] and sw[N]:
    y[m,n] = bf16(acc * fl32(sa[m] * sw[n])); returns bf16 bits [M,N]."""
    qa = _c_arr(qa, np.uint8)
    qw = _c_arr(qw, np.uint8)
    M, K = qa.shape
    N, _ = qw.shape
    sa = _c_arr(sa, np.float32)
    sw = _c_arr(sw, np.float32)
    assert sa.shape == (M,) and sw.shape == (N,)
    y = np.empty((M, N), np.uint16)
    lib.orc_gemm_fp8_rowwise_f32(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), M, N, K, _ptr(y),
                                 nthreads or default_threads())
    return y


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def gemm_fp8_f32(qa, sa, qw, sw, nthreads=None):
    """The plain fp32-accumulating FP8 GEMM; returns bf16 bits [M,N]."""
    qa = _c_arr(qa, np.uint8)
    qw = _c_arr(qw, np.uint8)
    M, K = qa.shape
    N, _ = qw.shape
    y = np.empty((M, N), np.uint16)
    lib.orc_gemm_fp8_f32(_ptr(qa), sa, _ptr(qw), sw, M, N, K, _ptr(y),
                         nthreads or default_threads())
    return y


def nested_fp16_f32(a16, hi, lo, nthreads=None):
    a16 = _c_arr(a16, np.uint16)
    hi = _c_arr(hi, np.uint8)
    lo = _c_arr(lo, np.uint8)
    M, K = a16.shape
    N, _ = hi.shape
    y = np.empty((M, N), np.uint16)
    lib.orc_nested_fp16_f32(_ptr(a16), _ptr(hi), _ptr(lo), M, N, K, _ptr(y),
                            nthreads or default_threads())
    return y


def nested_fp8_f32(qa, sa, hi, nthreads=None):
    qa = _c_arr(qa, np.uint8)
    hi = _c_arr(hi, np.uint8)
    M, K = qa.shape
    N, _ = hi.shape
    y = np.empty((M, N), np.uint16)
    lib.orc_nested_fp8_f32(_ptr(qa), sa, _ptr(hi), M, N, K, _ptr(y),
                           nthreads or default_threads())
    return y


# ---------------------------------------------------------------- tolerance
TOL_REL = 2e-3
TOL_ABS = 1e-6

# (stored mantissa bits, minimum normal exponent) of the GEMM output formats
_OUT_FORMATS = {"bf16": (7, -126), "fp16": (10, -14), "exact": None}


def half_ulp(v, out_format: str) -> np.ndarray:
    """Half a unit in the last place of `out_format` at magnitude |v|."""
    fmt = _OUT_FORMATS[out_format]
    v = np.abs(np.asarray(v, np.float64))
    if fmt is None:
        return np.zeros_like(v)
    p, emin = fmt
    _, e2 = np.frexp(v)                      # v = m * 2^e2, m in [0.5, 1)
    e = np.where(v == 0, emin, np.maximum(e2 - 1, emin))
    return np.ldexp(1.0, e - p - 1)


def within_tolerance(out, ref, absref, out_format: str = "exact"):
    """Per-element GEMM acceptance: |out - ref| <= 2e-3 * sum|a*b| + 1e-6, plus
    half an ulp of the output format at max(|out|, |ref|).

    The 2e-3 * sum|a*b| + 1e-6 bound covers the fp32 accumulation; the output
    is then rounded once to bf16 (FP8 GEMM) or fp16 (NestedFP), which on its
    own moves a value by up to half an ulp.  Where one product dominates a
    short sum (|y| close to sum|a*b|), that rounding alone exceeds
    2e-3 * sum|a*b|, so the bound is applied before the output rounding.
    """
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    mag = np.maximum(np.abs(out), np.abs(ref))
    return np.abs(out - ref) <= TOL_REL * absref + TOL_ABS + half_ulp(mag, out_format)
