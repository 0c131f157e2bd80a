"""fp8_quantized_gemm_amd: FP8 E4M3 per-tensor-scaled linear layers and the
NestedFP dual-precision GEMM for AMD MI355X (gfx950).

The compute lives in ``libfp8q.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/fp8q.h``).  ``fp8_quantized_gemm_amd.fp8q`` is the thin
ctypes binding with the same entry-point names; importing any of those names
from this package loads the library and raises if it has not been built.
"""
_API = (
    # per-tensor FP8 linear: quantizer, GEMM, quantize + GEMM
    "fp8_quantize_act", "fp8_gemm", "fp8_linear",
    # per-token activation / per-channel weight scales
    "fp8_quantize_rows", "fp8_gemm_rowwise", "fp8_linear_rowwise",
    # delayed scaling with an amax history
    "DelayedScaling", "fp8_quantize_act_delayed", "fp8_linear_delayed",
    # FP8 KV-cache quantizer (one scale per head)
    "fp8_quantize_kv",
    # NestedFP: byte split, FP16 and FP8 modes
    "nested_split", "nested_rebuild_fp16", "nested_gemm_fp16", "nested_gemm_fp8",
    "nested_linear_fp8",
    # NestedFP with an E4M3 upper byte
    "nested_split_e4m3", "nested_rebuild_e4m3", "nested_gemm_fp16_e4m3",
    "nested_gemm_fp8_e4m3", "nested_linear_fp8_e4m3",
    # the device E4M3 encoder on fp32 values, the ABI version, the error type
    "e4m3_encode_f32", "abi_version", "Fp8qError",
)

__all__ = list(_API)


def __getattr__(name):
    if name in _API:
        from . import fp8q  # loads libfp8q.so; raises loudly if it is missing
        return getattr(fp8q, name)
    raise AttributeError(name)
