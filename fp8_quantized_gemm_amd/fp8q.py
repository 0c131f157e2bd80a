"""ctypes binding of libfp8q (the C ABI in include/fp8q.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libfp8q.so.  torch supplies device memory (output tensors are
allocated with torch when not given) and the stream (torch's current stream
on the tensors' device).  There is no fallback: if the library is missing or
a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FP8Q_LIB", os.path.join(_HERE, "libfp8q.so"))

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libfp8q.so not found at {LIB_PATH}; build it with "
        "`python -m fp8_quantized_gemm_amd.build` (hipcc, gfx950)")

lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i = ctypes.c_int

_SIGS = {
    "fp8q_abi_version": (_i, []),
    "fp8q_status_str": (ctypes.c_char_p, [_i]),
    "fp8q_last_error": (ctypes.c_char_p, []),
    "fp8_quantize_act": (_i, [_p, _i, _i64, _p, _p, _p, _p]),
    "fp8_gemm": (_i, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _p]),
    "fp8_linear": (_i, [_p, _i, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p]),
    "nested_split": (_i, [_p, _p, _p, _i64, _p]),
    "nested_rebuild_fp16": (_i, [_p, _p, _p, _i64, _p]),
    "nested_gemm_fp16": (_i, [_p, _p, _p, _p, _i64, _i64, _i64, _p]),
    "nested_gemm_fp8": (_i, [_p, _p, _p, _p, _i64, _i64, _i64, _p]),
    "nested_linear_fp8": (_i, [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p]),
    "fp8q_e4m3_encode_f32": (_i, [_p, _p, _i64, _p]),
    "fp8_quantize_rows": (_i, [_p, _i, _i64, _i64, _p, _p, _p, _p]),
    "fp8_gemm_rowwise": (_i, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _p]),
    "fp8_linear_rowwise": (_i, [_p, _i, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p]),
    "fp8_quantize_act_delayed": (_i, [_p, _i, _i64, _p, _p, _p, _p, _i64, _p, _p]),
    "fp8_quantize_kv": (_i, [_p, _i, _i64, _i64, _i64, _p, _p, _p, _p]),
    "nested_split_e4m3": (_i, [_p, _p, _p, _i64, _p, _p]),
    "nested_rebuild_e4m3": (_i, [_p, _p, _p, _i64, _p]),
    "nested_gemm_fp16_e4m3": (_i, [_p, _p, _p, _p, _i64, _i64, _i64, _p]),
    "nested_gemm_fp8_e4m3": (_i, [_p, _p, _p, _p, _i64, _i64, _i64, _p]),
    "nested_linear_fp8_e4m3": (_i, [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p]),
    "fp8_linear_delayed": (_i, [_p, _i, _p, _p, _p, _p, _p, _p, _p, _i64, _p, _i64, _i64, _i64,
                                _p]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

ABI_VERSION = 3
# words of the delayed-scaling state (FP8Q_DELAYED_STATE_WORDS)
DELAYED_STATE_WORDS = 288
if lib.fp8q_abi_version() != ABI_VERSION:
    raise ImportError(f"libfp8q ABI {lib.fp8q_abi_version()} != binding ABI {ABI_VERSION}")

BF16 = 0
FP16 = 1


class Fp8qError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib.fp8q_status_str(status).decode()
        last = lib.fp8q_last_error().decode()
        super().__init__(f"{fn}: {msg} (status {status})" + (f": {last}" if last else ""))


def abi_version() -> int:
    return int(lib.fp8q_abi_version())


def _check(fn: str, status: int):
    if status != 0:
        raise Fp8qError(fn, status)


def _stream(t: torch.Tensor):
    return _p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.device.index != torch.cuda.current_device():
        # the library launches on the current device
        raise ValueError(f"{name} is on {t.device}, the current device is "
                         f"cuda:{torch.cuda.current_device()}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return _p(t.data_ptr())


def _scalar(t: torch.Tensor, name: str):
    if t.numel() != 1:
        raise ValueError(f"{name} must hold exactly one float32")
    return _dev(t, name, torch.float32)


def fp8_quantize_act(x: torch.Tensor, q: torch.Tensor | None = None,
                     scale: torch.Tensor | None = None, amax: torch.Tensor | None = None):
    """E4M3 codes, scale = amax/448 and amax of a bf16/fp16 tensor (any shape).

    Returns (q uint8 like x, scale float32[1], amax float32[1]); all on x's device.
    """
    if x.dtype == torch.bfloat16:
        code = BF16
    elif x.dtype == torch.float16:
        code = FP16
    else:
        raise TypeError(f"x must be bfloat16 or float16, got {x.dtype}")
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    if amax is None:
        amax = torch.empty(1, dtype=torch.float32, device=x.device)
    if q.numel() != x.numel():
        raise ValueError("q must have as many elements as x")
    _check("fp8_quantize_act", lib.fp8_quantize_act(
        _dev(x, "x"), code, x.numel(), _dev(q, "q", torch.uint8), _scalar(scale, "scale"),
        _scalar(amax, "amax"), _stream(x)))
    return q, scale, amax


def _mnk(a: torch.Tensor, w: torch.Tensor):
    if a.dim() != 2 or w.dim() != 2 or a.shape[1] != w.shape[1]:
        raise ValueError(f"expected a[M,K] and w[N,K], got {tuple(a.shape)} and {tuple(w.shape)}")
    return a.shape[0], w.shape[0], a.shape[1]


def fp8_gemm(qa: torch.Tensor, sa: torch.Tensor, qw: torch.Tensor, sw: torch.Tensor,
             y: torch.Tensor | None = None) -> torch.Tensor:
    """y[M,N] bf16 = (qa[M,K] . qw[N,K]^T) * sa * sw, E4M3 operands, fp32 accumulation."""
    M, N, K = _mnk(qa, qw)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=qa.device)
    _check("fp8_gemm", lib.fp8_gemm(
        _dev(qa, "qa", torch.uint8), _scalar(sa, "sa"), _dev(qw, "qw", torch.uint8),
        _scalar(sw, "sw"), _dev(y, "y", torch.bfloat16, (M, N)), M, N, K, _stream(qa)))
    return y


def fp8_linear(x: torch.Tensor, qw: torch.Tensor, sw: torch.Tensor,
               y: torch.Tensor | None = None, q: torch.Tensor | None = None,
               scale: torch.Tensor | None = None, amax: torch.Tensor | None = None):
    """One FP8 linear layer: quantize x[M,K] (bf16/fp16) per tensor, then
    y[M,N] bf16 = (q . qw^T) * scale * sw.  Returns (y, q, scale, amax)."""
    if x.dtype == torch.bfloat16:
        code = BF16
    elif x.dtype == torch.float16:
        code = FP16
    else:
        raise TypeError(f"x must be bfloat16 or float16, got {x.dtype}")
    M, N, K = _mnk(x, qw)
    dev = x.device
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=dev)
    if amax is None:
        amax = torch.empty(1, dtype=torch.float32, device=dev)
    _check("fp8_linear", lib.fp8_linear(
        _dev(x, "x"), code, _dev(qw, "qw", torch.uint8), _scalar(sw, "sw"),
        _dev(y, "y", torch.bfloat16, (M, N)), _dev(q, "q", torch.uint8, (M, K)),
        _scalar(scale, "scale"), _scalar(amax, "amax"), M, N, K, _stream(x)))
    return y, q, scale, amax


def _vector(t: torch.Tensor, name: str, n: int):
    if t.numel() != n:
        raise ValueError(f"{name} must hold {n} float32 values, got {t.numel()}")
    return _dev(t, name, torch.float32)


def _dtype_code(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return BF16
    if x.dtype == torch.float16:
        return FP16
    raise TypeError(f"x must be bfloat16 or float16, got {x.dtype}")


def fp8_quantize_rows(x: torch.Tensor, q: torch.Tensor | None = None,
                      scale: torch.Tensor | None = None, amax: torch.Tensor | None = None):
    """One E4M3 scale per row of x[rows, cols] (bf16/fp16): per-token activation
    or per-channel weight scales.  Returns (q uint8 [rows, cols], scale float32
    [rows], amax float32 [rows])."""
    code = _dtype_code(x)
    if x.dim() != 2:
        raise ValueError(f"x must be 2-D [rows, cols], got {tuple(x.shape)}")
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(rows, dtype=torch.float32, device=x.device)
    if amax is None:
        amax = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check("fp8_quantize_rows", lib.fp8_quantize_rows(
        _dev(x, "x"), code, rows, cols, _dev(q, "q", torch.uint8, (rows, cols)),
        _vector(scale, "scale", rows), _vector(amax, "amax", rows), _stream(x)))
    return q, scale, amax


def fp8_gemm_rowwise(qa: torch.Tensor, sa: torch.Tensor, qw: torch.Tensor, sw: torch.Tensor,
                     y: torch.Tensor | None = None) -> torch.Tensor:
    """y[M,N] bf16 = (qa . qw^T)[m,n] * fl32(sa[m] * sw[n]): per-token activation
    and per-channel weight scales, fp32 accumulation."""
    M, N, K = _mnk(qa, qw)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=qa.device)
    _check("fp8_gemm_rowwise", lib.fp8_gemm_rowwise(
        _dev(qa, "qa", torch.uint8), _vector(sa, "sa", M), _dev(qw, "qw", torch.uint8),
        _vector(sw, "sw", N), _dev(y, "y", torch.bfloat16, (M, N)), M, N, K, _stream(qa)))
    return y


def fp8_linear_rowwise(x: torch.Tensor, qw: torch.Tensor, sw: torch.Tensor,
                       y: torch.Tensor | None = None, q: torch.Tensor | None = None,
                       sa: torch.Tensor | None = None, amax: torch.Tensor | None = None):
    """fp8_quantize_rows on x[M,K], then fp8_gemm_rowwise with the per-channel
    weight scales sw[N].  Returns (y, q, sa, amax)."""
    code = _dtype_code(x)
    M, N, K = _mnk(x, qw)
    dev = x.device
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=dev)
    if sa is None:
        sa = torch.empty(M, dtype=torch.float32, device=dev)
    if amax is None:
        amax = torch.empty(M, dtype=torch.float32, device=dev)
    _check("fp8_linear_rowwise", lib.fp8_linear_rowwise(
        _dev(x, "x"), code, _dev(qw, "qw", torch.uint8), _vector(sw, "sw", N),
        _dev(y, "y", torch.bfloat16, (M, N)), _dev(q, "q", torch.uint8, (M, K)),
        _vector(sa, "sa", M), _vector(amax, "amax", M), M, N, K, _stream(x)))
    return y, q, sa, amax


def fp8_quantize_kv(x: torch.Tensor, q: torch.Tensor | None = None,
                    scale: torch.Tensor | None = None, amax: torch.Tensor | None = None):
    """FP8 KV cache: E4M3 codes of a K or V block x[T, H, D] (bf16/fp16) with one
    scale per head.  Returns (q uint8 [T, H, D], scale float32 [H], amax float32 [H])."""
    code = _dtype_code(x)
    if x.dim() != 3:
        raise ValueError(f"x must be [tokens, heads, head_dim], got {tuple(x.shape)}")
    T, H, D = x.shape
    if q is None:
        q = torch.empty((T, H, D), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(H, dtype=torch.float32, device=x.device)
    if amax is None:
        amax = torch.empty(H, dtype=torch.float32, device=x.device)
    _check("fp8_quantize_kv", lib.fp8_quantize_kv(
        _dev(x, "x"), code, T, H, D, _dev(q, "q", torch.uint8, (T, H, D)),
        _vector(scale, "scale", H), _vector(amax, "amax", H), _stream(x)))
    return q, scale, amax


class DelayedScaling:
    """Device state of delayed scaling for one tensor: the amax of its last
    `length` quantizations (zeros at first) and the scale the next one uses.
    Use one object per tensor and issue its calls on one stream."""

    def __init__(self, length: int = 1024, device="cuda"):
        if length < 1:
            raise ValueError("the amax history needs at least one entry")
        self.history = torch.zeros(length, dtype=torch.float32, device=device)
        self.state = torch.zeros(DELAYED_STATE_WORDS, dtype=torch.int32, device=device)

    def _args(self):
        return (_dev(self.history, "history", torch.float32), self.history.numel(),
                _dev(self.state, "state", torch.int32, (DELAYED_STATE_WORDS,)))

    @property
    def next_scale(self) -> float:
        """The scale the next call will use (1.0 before any history)."""
        s = float(self.state[:1].view(torch.float32).item())
        return s if s > 0 else 1.0

    @property
    def position(self) -> int:
        return int(self.state[2].item())


def fp8_quantize_act_delayed(x: torch.Tensor, ds: DelayedScaling, q: torch.Tensor | None = None,
                             scale: torch.Tensor | None = None,
                             amax: torch.Tensor | None = None):
    """fp8_quantize_act with delayed scaling: codes with the scale of ds's amax
    history, then x's amax recorded in it.  Returns (q, scale used, amax of x)."""
    code = _dtype_code(x)
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    if amax is None:
        amax = torch.empty(1, dtype=torch.float32, device=x.device)
    if q.numel() != x.numel():
        raise ValueError("q must have as many elements as x")
    _check("fp8_quantize_act_delayed", lib.fp8_quantize_act_delayed(
        _dev(x, "x"), code, x.numel(), _dev(q, "q", torch.uint8), _scalar(scale, "scale"),
        _scalar(amax, "amax"), *ds._args(), _stream(x)))
    return q, scale, amax


def fp8_linear_delayed(x: torch.Tensor, qw: torch.Tensor, sw: torch.Tensor, ds: DelayedScaling,
                       y: torch.Tensor | None = None, q: torch.Tensor | None = None,
                       scale: torch.Tensor | None = None, amax: torch.Tensor | None = None):
    """fp8_linear with delayed activation scaling (ds holds the amax history).
    Returns (y, q, scale used, amax of x)."""
    code = _dtype_code(x)
    M, N, K = _mnk(x, qw)
    dev = x.device
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=dev)
    if amax is None:
        amax = torch.empty(1, dtype=torch.float32, device=dev)
    hist, hlen, state = ds._args()
    _check("fp8_linear_delayed", lib.fp8_linear_delayed(
        _dev(x, "x"), code, _dev(qw, "qw", torch.uint8), _scalar(sw, "sw"),
        _dev(y, "y", torch.bfloat16, (M, N)), _dev(q, "q", torch.uint8, (M, K)),
        _scalar(scale, "scale"), _scalar(amax, "amax"), hist, hlen, state, M, N, K, _stream(x)))
    return y, q, scale, amax


def nested_split(w: torch.Tensor, hi: torch.Tensor | None = None,
                 lo: torch.Tensor | None = None):
    """NestedFP byte planes of an fp16 tensor: (hi, lo) uint8 of w's shape."""
    if hi is None:
        hi = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    if lo is None:
        lo = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    if hi.numel() != w.numel() or lo.numel() != w.numel():
        raise ValueError("hi and lo must have as many elements as w")
    _check("nested_split", lib.nested_split(
        _dev(w, "w", torch.float16), _dev(hi, "hi", torch.uint8), _dev(lo, "lo", torch.uint8),
        w.numel(), _stream(w)))
    return hi, lo


def nested_rebuild_fp16(hi: torch.Tensor, lo: torch.Tensor,
                        w: torch.Tensor | None = None) -> torch.Tensor:
    """fp16 tensor with words (hi << 8) | lo."""
    if hi.shape != lo.shape:
        raise ValueError("hi and lo must have the same shape")
    if w is None:
        w = torch.empty(hi.shape, dtype=torch.float16, device=hi.device)
    _check("nested_rebuild_fp16", lib.nested_rebuild_fp16(
        _dev(hi, "hi", torch.uint8), _dev(lo, "lo", torch.uint8),
        _dev(w, "w", torch.float16, hi.shape), hi.numel(), _stream(hi)))
    return w


def nested_gemm_fp16(a: torch.Tensor, hi: torch.Tensor, lo: torch.Tensor,
                     y: torch.Tensor | None = None) -> torch.Tensor:
    """NestedFP FP16 mode: y[M,N] fp16 = a[M,K] . fp16((hi<<8)|lo)[N,K]^T."""
    M, N, K = _mnk(a, hi)
    if lo.shape != hi.shape:
        raise ValueError("hi and lo must have the same shape")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=a.device)
    _check("nested_gemm_fp16", lib.nested_gemm_fp16(
        _dev(a, "a", torch.float16), _dev(hi, "hi", torch.uint8), _dev(lo, "lo", torch.uint8),
        _dev(y, "y", torch.float16, (M, N)), M, N, K, _stream(a)))
    return y


def nested_gemm_fp8(qa: torch.Tensor, sa: torch.Tensor, hi: torch.Tensor,
                    y: torch.Tensor | None = None) -> torch.Tensor:
    """NestedFP FP8 mode: y[M,N] fp16 = (qa . E5M2(hi)^T) * sa."""
    M, N, K = _mnk(qa, hi)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=qa.device)
    _check("nested_gemm_fp8", lib.nested_gemm_fp8(
        _dev(qa, "qa", torch.uint8), _scalar(sa, "sa"), _dev(hi, "hi", torch.uint8),
        _dev(y, "y", torch.float16, (M, N)), M, N, K, _stream(qa)))
    return y


def nested_linear_fp8(a: torch.Tensor, hi: torch.Tensor, y: torch.Tensor | None = None,
                      q: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                      amax: torch.Tensor | None = None):
    """One NestedFP FP8-mode linear layer: quantize a[M,K] (fp16) per tensor,
    then y[M,N] fp16 = (q . E5M2(hi)^T) * scale.  Returns (y, q, scale, amax)."""
    if a.dtype != torch.float16:
        raise TypeError(f"a must be float16, got {a.dtype}")
    M, N, K = _mnk(a, hi)
    dev = a.device
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=dev)
    if amax is None:
        amax = torch.empty(1, dtype=torch.float32, device=dev)
    _check("nested_linear_fp8", lib.nested_linear_fp8(
        _dev(a, "a", torch.float16), _dev(hi, "hi", torch.uint8),
        _dev(y, "y", torch.float16, (M, N)), _dev(q, "q", torch.uint8, (M, K)),
        _scalar(scale, "scale"), _scalar(amax, "amax"), M, N, K, _stream(a)))
    return y, q, scale, amax


def nested_split_e4m3(w: torch.Tensor, hi: torch.Tensor | None = None,
                      lo: torch.Tensor | None = None):
    """NestedFP planes with an E4M3 upper byte: hi = sign | bits 13..7 (the E4M3
    code of w * 2^8 when |w| < 2), lo = bit 14 | bits 6..0.  Returns (hi, lo,
    out_of_range), the last an int64 device tensor counting the words outside
    the FP8 mode's range |w| < 1.875."""
    if hi is None:
        hi = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    if lo is None:
        lo = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    if hi.numel() != w.numel() or lo.numel() != w.numel():
        raise ValueError("hi and lo must have as many elements as w")
    bad = torch.zeros(1, dtype=torch.int64, device=w.device)
    _check("nested_split_e4m3", lib.nested_split_e4m3(
        _dev(w, "w", torch.float16), _dev(hi, "hi", torch.uint8), _dev(lo, "lo", torch.uint8),
        w.numel(), _dev(bad, "out_of_range", torch.int64), _stream(w)))
    return hi, lo, bad


def nested_rebuild_e4m3(hi: torch.Tensor, lo: torch.Tensor,
                        w: torch.Tensor | None = None) -> torch.Tensor:
    """fp16 words rebuilt from the E4M3-split planes."""
    if hi.shape != lo.shape:
        raise ValueError("hi and lo must have the same shape")
    if w is None:
        w = torch.empty(hi.shape, dtype=torch.float16, device=hi.device)
    _check("nested_rebuild_e4m3", lib.nested_rebuild_e4m3(
        _dev(hi, "hi", torch.uint8), _dev(lo, "lo", torch.uint8),
        _dev(w, "w", torch.float16, hi.shape), hi.numel(), _stream(hi)))
    return w


def nested_gemm_fp16_e4m3(a: torch.Tensor, hi: torch.Tensor, lo: torch.Tensor,
                          y: torch.Tensor | None = None) -> torch.Tensor:
    """NestedFP FP16 mode on E4M3-split planes: y fp16 = a . rebuilt(hi, lo)^T."""
    M, N, K = _mnk(a, hi)
    if lo.shape != hi.shape:
        raise ValueError("hi and lo must have the same shape")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=a.device)
    _check("nested_gemm_fp16_e4m3", lib.nested_gemm_fp16_e4m3(
        _dev(a, "a", torch.float16), _dev(hi, "hi", torch.uint8), _dev(lo, "lo", torch.uint8),
        _dev(y, "y", torch.float16, (M, N)), M, N, K, _stream(a)))
    return y


def nested_gemm_fp8_e4m3(qa: torch.Tensor, sa: torch.Tensor, hi: torch.Tensor,
                         y: torch.Tensor | None = None) -> torch.Tensor:
    """NestedFP FP8 mode on E4M3-split planes: y fp16 = (qa . E4M3(hi)^T) * sa * 2^-8."""
    M, N, K = _mnk(qa, hi)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=qa.device)
    _check("nested_gemm_fp8_e4m3", lib.nested_gemm_fp8_e4m3(
        _dev(qa, "qa", torch.uint8), _scalar(sa, "sa"), _dev(hi, "hi", torch.uint8),
        _dev(y, "y", torch.float16, (M, N)), M, N, K, _stream(qa)))
    return y


def nested_linear_fp8_e4m3(a: torch.Tensor, hi: torch.Tensor, y: torch.Tensor | None = None,
                           q: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                           amax: torch.Tensor | None = None):
    """nested_linear_fp8 on E4M3-split planes.  Returns (y, q, scale, amax)."""
    if a.dtype != torch.float16:
        raise TypeError(f"a must be float16, got {a.dtype}")
    M, N, K = _mnk(a, hi)
    dev = a.device
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=dev)
    if amax is None:
        amax = torch.empty(1, dtype=torch.float32, device=dev)
    _check("nested_linear_fp8_e4m3", lib.nested_linear_fp8_e4m3(
        _dev(a, "a", torch.float16), _dev(hi, "hi", torch.uint8),
        _dev(y, "y", torch.float16, (M, N)), _dev(q, "q", torch.uint8, (M, K)),
        _scalar(scale, "scale"), _scalar(amax, "amax"), M, N, K, _stream(a)))
    return y, q, scale, amax


def e4m3_encode_f32(v: torch.Tensor, q: torch.Tensor | None = None) -> torch.Tensor:
    """The device E4M3 encoder on float32 values (for exhaustive checks)."""
    if q is None:
        q = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    _check("fp8q_e4m3_encode_f32", lib.fp8q_e4m3_encode_f32(
        _dev(v, "v", torch.float32), _dev(q, "q", torch.uint8, v.shape), v.numel(), _stream(v)))
    return q
