"""The C ABI library loads, exports every function include/fp8q.h declares, and
rejects invalid arguments on the host before any HIP call (CPU only: none of
these calls reaches the GPU)."""
import ctypes
import os
import re

import pytest

from fp8_quantized_gemm_amd import fp8q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DTYPE = 0, 1, 2, 3, 4
ERR_OVERLAP = 7

P16 = ctypes.c_void_p(0x1000)      # aligned, never dereferenced: validation fails first
P17 = ctypes.c_void_p(0x1001)
NULL = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ["fp8_quantize_act", "fp8_gemm", "fp8_linear", "nested_split", "nested_rebuild_fp16",
                 "nested_gemm_fp16", "nested_gemm_fp8", "nested_linear_fp8", "fp8q_abi_version",
                 "fp8q_status_str", "fp8q_last_error", "fp8q_e4m3_encode_f32",
                 "fp8_quantize_rows", "fp8_gemm_rowwise", "fp8_linear_rowwise",
                 "fp8_quantize_act_delayed", "fp8_linear_delayed", "fp8_quantize_kv",
                 "nested_split_e4m3", "nested_rebuild_e4m3", "nested_gemm_fp16_e4m3",
                 "nested_gemm_fp8_e4m3", "nested_linear_fp8_e4m3"]:
        assert want in names


def test_library_exports_every_declared_symbol():
    for name in declared_functions():
        assert hasattr(fp8q.lib, name), name


def test_no_internal_symbols_exported():
    out = os.popen(f"nm -D --defined-only {fp8q.LIB_PATH}").read()
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert exported == set(declared_functions())


def _header_define(name):
    m = re.search(r"^#define\s+" + name + r"\s+(\d+)", open(HEADER).read(), flags=re.M)
    assert m, name
    return int(m.group(1))


def test_version_and_status_strings():
    assert fp8q.lib.fp8q_abi_version() == _header_define("FP8Q_ABI_VERSION") == 3
    assert fp8q.DELAYED_STATE_WORDS == _header_define("FP8Q_DELAYED_STATE_WORDS")
    for s in range(8):
        assert fp8q.lib.fp8q_status_str(s)
    assert fp8q.lib.fp8q_status_str(99) == b"unknown status"


GEMM_SIG = [P16, P16, P16, P16, P16]


@pytest.mark.parametrize("fn,args,status", [
    # fp8_quantize_act(x, dtype, n, q, scale, amax, stream)
    ("fp8_quantize_act", [NULL, 0, 8, P16, P16, P16, NULL], ERR_NULL),
    ("fp8_quantize_act", [P16, 0, 8, NULL, P16, P16, NULL], ERR_NULL),
    ("fp8_quantize_act", [P16, 0, 8, P16, NULL, P16, NULL], ERR_NULL),
    ("fp8_quantize_act", [P16, 0, 8, P16, P16, NULL, NULL], ERR_NULL),
    ("fp8_quantize_act", [P16, 2, 8, P16, P16, P16, NULL], ERR_DTYPE),
    ("fp8_quantize_act", [P16, -1, 8, P16, P16, P16, NULL], ERR_DTYPE),
    ("fp8_quantize_act", [P16, 0, 0, P16, P16, P16, NULL], ERR_SHAPE),
    ("fp8_quantize_act", [P16, 1, -5, P16, P16, P16, NULL], ERR_SHAPE),
    ("fp8_quantize_act", [P17, 0, 8, P16, P16, P16, NULL], ERR_ALIGN),
    ("fp8_quantize_act", [P16, 0, 8, P17, P16, P16, NULL], ERR_ALIGN),
    ("fp8_quantize_act", [P16, 0, 8, P16, ctypes.c_void_p(0x1002), P16, NULL], ERR_ALIGN),
    # fp8_gemm(qa, sa, qw, sw, y, M, N, K, stream)
    ("fp8_gemm", [NULL, P16, P16, P16, P16, 1, 1, 16, NULL], ERR_NULL),
    ("fp8_gemm", [P16, NULL, P16, P16, P16, 1, 1, 16, NULL], ERR_NULL),
    ("fp8_gemm", [P16, P16, NULL, P16, P16, 1, 1, 16, NULL], ERR_NULL),
    ("fp8_gemm", [P16, P16, P16, NULL, P16, 1, 1, 16, NULL], ERR_NULL),
    ("fp8_gemm", [P16, P16, P16, P16, NULL, 1, 1, 16, NULL], ERR_NULL),
    ("fp8_gemm", [P16, P16, P16, P16, P16, 0, 1, 16, NULL], ERR_SHAPE),
    ("fp8_gemm", [P16, P16, P16, P16, P16, 1, 0, 16, NULL], ERR_SHAPE),
    ("fp8_gemm", [P16, P16, P16, P16, P16, 1, 1, 0, NULL], ERR_SHAPE),
    ("fp8_gemm", [P16, P16, P16, P16, P16, 1, 1, 8, NULL], ERR_SHAPE),
    ("fp8_gemm", [P16, P16, P16, P16, P16, 1, 1, 40, NULL], ERR_SHAPE),
    ("fp8_gemm", [P16, P16, P16, P16, P16, 2**31, 1, 16, NULL], ERR_SHAPE),
    ("fp8_gemm", [P16, P16, P16, P16, P16, 1, 2**31, 16, NULL], ERR_SHAPE),
    ("fp8_gemm", [P16, P16, P16, P16, P16, 1, 1, 2**31 + 16, NULL], ERR_SHAPE),
    ("fp8_gemm", [P16, P16, P16, P16, P16, 1, 1, 2**22 + 16, NULL], ERR_SHAPE),
    ("fp8_gemm", [P17, P16, P16, P16, P16, 1, 1, 16, NULL], ERR_ALIGN),
    ("fp8_gemm", [P16, P16, P17, P16, P16, 1, 1, 16, NULL], ERR_ALIGN),
    ("fp8_gemm", [P16, P16, P16, P16, P17, 1, 1, 16, NULL], ERR_ALIGN),
    ("fp8_gemm", [P16, P17, P16, P16, P16, 1, 1, 16, NULL], ERR_ALIGN),
    # fp8_linear(x, dtype, qw, sw, y, q, scale, amax, M, N, K, stream)
    ("fp8_linear", [NULL, 0, P16, P16, P16, P16, P16, P16, 1, 1, 16, NULL], ERR_NULL),
    ("fp8_linear", [P16, 0, P16, P16, P16, NULL, P16, P16, 1, 1, 16, NULL], ERR_NULL),
    ("fp8_linear", [P16, 0, P16, P16, P16, P16, P16, NULL, 1, 1, 16, NULL], ERR_NULL),
    ("fp8_linear", [P16, 3, P16, P16, P16, P16, P16, P16, 1, 1, 16, NULL], ERR_DTYPE),
    ("fp8_linear", [P16, 0, P16, P16, P16, P16, P16, P16, 1, 1, 24, NULL], ERR_SHAPE),
    ("fp8_linear", [P16, 1, P16, P16, P16, P16, P16, P16, 0, 1, 16, NULL], ERR_SHAPE),
    ("fp8_linear", [P16, 0, P16, P16, P16, P17, P16, P16, 1, 1, 16, NULL], ERR_ALIGN),
    ("fp8_linear", [P17, 0, P16, P16, P16, P16, P16, P16, 1, 1, 16, NULL], ERR_ALIGN),
    # nested_split(w, hi, lo, n, stream) / nested_rebuild_fp16(hi, lo, w, n, stream)
    ("nested_split", [NULL, P16, P16, 8, NULL], ERR_NULL),
    ("nested_split", [P16, P16, P16, 0, NULL], ERR_SHAPE),
    ("nested_split", [P16, P17, P16, 8, NULL], ERR_ALIGN),
    ("nested_rebuild_fp16", [P16, NULL, P16, 8, NULL], ERR_NULL),
    ("nested_rebuild_fp16", [P16, P16, P16, -1, NULL], ERR_SHAPE),
    ("nested_rebuild_fp16", [P16, P16, P17, 8, NULL], ERR_ALIGN),
    # nested_gemm_fp16(a, hi, lo, y, M, N, K, stream)
    ("nested_gemm_fp16", [P16, P16, NULL, P16, 1, 1, 16, NULL], ERR_NULL),
    ("nested_gemm_fp16", [P16, P16, P16, P16, 1, 1, 24, NULL], ERR_SHAPE),
    ("nested_gemm_fp16", [P16, P16, P16, P17, 1, 1, 16, NULL], ERR_ALIGN),
    # nested_gemm_fp8(qa, sa, hi, y, M, N, K, stream)
    ("nested_gemm_fp8", [P16, NULL, P16, P16, 1, 1, 16, NULL], ERR_NULL),
    ("nested_gemm_fp8", [P16, P16, P16, P16, -3, 1, 16, NULL], ERR_SHAPE),
    ("nested_gemm_fp8", [P16, P16, P17, P16, 1, 1, 16, NULL], ERR_ALIGN),
    # nested_linear_fp8(a, hi, y, q, scale, amax, M, N, K, stream)
    ("nested_linear_fp8", [NULL, P16, P16, P16, P16, P16, 1, 1, 16, NULL], ERR_NULL),
    ("nested_linear_fp8", [P16, P16, P16, P16, P16, NULL, 1, 1, 16, NULL], ERR_NULL),
    ("nested_linear_fp8", [P16, P16, P16, P16, P16, P16, 1, 1, 24, NULL], ERR_SHAPE),
    ("nested_linear_fp8", [P16, P16, P16, P16, P16, P16, 1, 0, 16, NULL], ERR_SHAPE),
    ("nested_linear_fp8", [P16, P17, P16, P16, P16, P16, 1, 1, 16, NULL], ERR_ALIGN),
    ("nested_linear_fp8", [P16, P16, P16, P16, ctypes.c_void_p(0x1002), P16, 1, 1, 16, NULL],
     ERR_ALIGN),
    # fp8_quantize_rows(x, dtype, rows, cols, q, scale, amax, stream)
    ("fp8_quantize_rows", [NULL, 0, 1, 16, P16, P16, P16, NULL], ERR_NULL),
    ("fp8_quantize_rows", [P16, 0, 1, 16, P16, NULL, P16, NULL], ERR_NULL),
    ("fp8_quantize_rows", [P16, 2, 1, 16, P16, P16, P16, NULL], ERR_DTYPE),
    ("fp8_quantize_rows", [P16, 0, 0, 16, P16, P16, P16, NULL], ERR_SHAPE),
    ("fp8_quantize_rows", [P16, 0, 1, 8, P16, P16, P16, NULL], ERR_SHAPE),
    ("fp8_quantize_rows", [P16, 0, 1, 24, P16, P16, P16, NULL], ERR_SHAPE),
    ("fp8_quantize_rows", [P16, 0, 2**31, 16, P16, P16, P16, NULL], ERR_SHAPE),
    ("fp8_quantize_rows", [P16, 0, 1, 2**22 + 16, P16, P16, P16, NULL], ERR_SHAPE),
    ("fp8_quantize_rows", [P17, 0, 1, 16, P16, P16, P16, NULL], ERR_ALIGN),
    ("fp8_quantize_rows", [P16, 1, 1, 16, P16, P16, ctypes.c_void_p(0x1002), NULL], ERR_ALIGN),
    # fp8_gemm_rowwise(qa, sa, qw, sw, y, M, N, K, stream)
    ("fp8_gemm_rowwise", [P16, P16, P16, NULL, P16, 1, 1, 16, NULL], ERR_NULL),
    ("fp8_gemm_rowwise", [P16, P16, P16, P16, P16, 1, 1, 40, NULL], ERR_SHAPE),
    ("fp8_gemm_rowwise", [P16, P16, P16, P16, P16, 0, 1, 16, NULL], ERR_SHAPE),
    ("fp8_gemm_rowwise", [P16, P16, P16, P16, P17, 1, 1, 16, NULL], ERR_ALIGN),
    ("fp8_gemm_rowwise", [P16, ctypes.c_void_p(0x1002), P16, P16, P16, 1, 1, 16, NULL], ERR_ALIGN),
    # fp8_linear_rowwise(x, dtype, qw, sw, y, q, sa, amax, M, N, K, stream)
    ("fp8_linear_rowwise", [P16, 0, P16, P16, P16, P16, NULL, P16, 1, 1, 16, NULL], ERR_NULL),
    ("fp8_linear_rowwise", [P16, 5, P16, P16, P16, P16, P16, P16, 1, 1, 16, NULL], ERR_DTYPE),
    ("fp8_linear_rowwise", [P16, 0, P16, P16, P16, P16, P16, P16, 1, 1, 8, NULL], ERR_SHAPE),
    ("fp8_linear_rowwise", [P16, 0, P16, P16, P16, P17, P16, P16, 1, 1, 16, NULL], ERR_ALIGN),
    # fp8_quantize_act_delayed(x, dtype, n, q, scale, amax, history, L, state, stream)
    ("fp8_quantize_act_delayed", [P16, 0, 8, P16, P16, P16, NULL, 4, P16, NULL], ERR_NULL),
    ("fp8_quantize_act_delayed", [P16, 0, 8, P16, P16, P16, P16, 4, NULL, NULL], ERR_NULL),
    ("fp8_quantize_act_delayed", [P16, 9, 8, P16, P16, P16, P16, 4, P16, NULL], ERR_DTYPE),
    ("fp8_quantize_act_delayed", [P16, 0, 0, P16, P16, P16, P16, 4, P16, NULL], ERR_SHAPE),
    ("fp8_quantize_act_delayed", [P16, 0, 8, P16, P16, P16, P16, 0, P16, NULL], ERR_SHAPE),
    ("fp8_quantize_act_delayed", [P16, 0, 8, P16, P16, P16, P16, 2**24 + 1, P16, NULL], ERR_SHAPE),
    ("fp8_quantize_act_delayed", [P16, 0, 8, P16, P16, P16, P16, 4, ctypes.c_void_p(0x1004), NULL],
     ERR_ALIGN),
    ("fp8_quantize_act_delayed", [P16, 0, 8, P16, P16, P16, ctypes.c_void_p(0x1002), 4, P16, NULL],
     ERR_ALIGN),
    # fp8_linear_delayed(x, dtype, qw, sw, y, q, scale, amax, history, L, state, M, N, K, stream)
    ("fp8_linear_delayed", [P16, 0, P16, P16, P16, P16, P16, P16, NULL, 4, P16, 1, 1, 16, NULL],
     ERR_NULL),
    ("fp8_linear_delayed", [P16, 0, P16, P16, P16, P16, P16, P16, P16, 4, P16, 1, 1, 24, NULL],
     ERR_SHAPE),
    ("fp8_linear_delayed", [P16, 0, P16, P16, P16, P16, P16, P16, P16, -1, P16, 1, 1, 16, NULL],
     ERR_SHAPE),
    ("fp8_linear_delayed", [P16, 1, P16, P16, P16, P17, P16, P16, P16, 4, P16, 1, 1, 16, NULL],
     ERR_ALIGN),
    # fp8_quantize_kv(x, dtype, tokens, heads, head_dim, q, scale, amax, stream)
    ("fp8_quantize_kv", [P16, 0, 1, 1, 8, P16, NULL, P16, NULL], ERR_NULL),
    ("fp8_quantize_kv", [P16, 3, 1, 1, 8, P16, P16, P16, NULL], ERR_DTYPE),
    ("fp8_quantize_kv", [P16, 0, 0, 1, 8, P16, P16, P16, NULL], ERR_SHAPE),
    ("fp8_quantize_kv", [P16, 0, 1, 0, 8, P16, P16, P16, NULL], ERR_SHAPE),
    ("fp8_quantize_kv", [P16, 0, 1, 1, 12, P16, P16, P16, NULL], ERR_SHAPE),
    ("fp8_quantize_kv", [P16, 0, 1, 1, 4, P16, P16, P16, NULL], ERR_SHAPE),
    ("fp8_quantize_kv", [P16, 0, 2**40, 2, 8, P16, P16, P16, NULL], ERR_SHAPE),
    ("fp8_quantize_kv", [P16, 0, 1, 1, 8, P17, P16, P16, NULL], ERR_ALIGN),
    # nested_split_e4m3(w, hi, lo, n, out_of_range, stream) and the E4M3-split calls
    ("nested_split_e4m3", [P16, NULL, P16, 8, NULL, NULL], ERR_NULL),
    ("nested_split_e4m3", [P16, P16, P16, 0, NULL, NULL], ERR_SHAPE),
    ("nested_split_e4m3", [P16, P16, P16, 8, ctypes.c_void_p(0x1004), NULL], ERR_ALIGN),
    ("nested_rebuild_e4m3", [P16, P16, P17, 8, NULL], ERR_ALIGN),
    ("nested_gemm_fp16_e4m3", [P16, P16, P16, P16, 1, 1, 24, NULL], ERR_SHAPE),
    ("nested_gemm_fp8_e4m3", [P16, NULL, P16, P16, 1, 1, 16, NULL], ERR_NULL),
    ("nested_linear_fp8_e4m3", [P16, P16, P16, P16, P16, P16, 1, 0, 16, NULL], ERR_SHAPE),
    # fp8q_e4m3_encode_f32(v, q, n, stream)
    ("fp8q_e4m3_encode_f32", [NULL, P16, 4, NULL], ERR_NULL),
    ("fp8q_e4m3_encode_f32", [P16, P16, 0, NULL], ERR_SHAPE),
    ("fp8q_e4m3_encode_f32", [P16, P17, 4, NULL], ERR_ALIGN),
])
def test_validation_before_any_hip_call(fn, args, status):
    assert getattr(fp8q.lib, fn)(*args) == status


# Distinct, aligned, never dereferenced base addresses 64 KiB apart.
def _at(region, offset=0):
    return ctypes.c_void_p(0x100000 + region * 0x10000 + offset)


A, B, C, D, E, F, G, H = (_at(i) for i in range(8))


@pytest.mark.parametrize("fn,args", [
    # fp8_quantize_act(x, dtype, n, q, scale, amax): q inside x, scale inside q, scale == amax
    ("fp8_quantize_act", [A, 0, 64, _at(0, 64), C, D, NULL]),
    ("fp8_quantize_act", [A, 0, 64, B, _at(1, 16), D, NULL]),
    ("fp8_quantize_act", [A, 0, 64, B, C, C, NULL]),
    ("fp8_quantize_act", [A, 1, 64, B, _at(0, 124), D, NULL]),
    # fp8_gemm(qa, sa, qw, sw, y, M, N, K): y over qa, over sw, over the last weight row
    ("fp8_gemm", [A, B, C, D, A, 1, 1, 16, NULL]),
    ("fp8_gemm", [A, B, C, D, D, 1, 1, 16, NULL]),
    ("fp8_gemm", [A, B, C, D, _at(2, 16 * 16), 2, 17, 16, NULL]),
    # fp8_linear(x, dtype, qw, sw, y, q, scale, amax, M, N, K): y == q, q over x,
    # y over the weights, amax == scale
    ("fp8_linear", [A, 0, C, D, B, B, E, F, 1, 1, 16, NULL]),
    ("fp8_linear", [A, 0, C, D, B, A, E, F, 1, 1, 16, NULL]),
    ("fp8_linear", [A, 0, C, D, C, G, E, F, 1, 1, 16, NULL]),
    ("fp8_linear", [A, 0, C, D, B, G, E, E, 1, 1, 16, NULL]),
    # fp8_quantize_kv(x, dtype, T, H, D, q, scale, amax): q over x, amax inside scale
    ("fp8_quantize_kv", [A, 0, 4, 2, 8, _at(0, 32), C, D, NULL]),
    ("fp8_quantize_kv", [A, 0, 4, 2, 8, B, C, _at(2, 4), NULL]),
    # fp8_quantize_act_delayed(x, dtype, n, q, scale, amax, history, L, state):
    # history over q, state == scale
    ("fp8_quantize_act_delayed", [A, 0, 64, B, C, D, _at(1, 32), 4, E, NULL]),
    ("fp8_quantize_act_delayed", [A, 0, 64, B, E, D, F, 4, E, NULL]),
    # the state's last words (FP8Q_DELAYED_STATE_WORDS of them) reach amax
    ("fp8_quantize_act_delayed", [A, 0, 64, B, C, E, F, 4, _at(3, 0x10000 - 512), NULL]),
    # fp8_linear_delayed(x, dtype, qw, sw, y, q, scale, amax, history, L, state, M, N, K):
    # history over y, state over x
    ("fp8_linear_delayed", [A, 0, C, D, B, E, F, G, B, 4, H, 1, 1, 16, NULL]),
    ("fp8_linear_delayed", [A, 0, C, D, B, E, F, G, H, 4, A, 1, 1, 16, NULL]),
    # fp8_quantize_rows(x, dtype, rows, cols, q, scale, amax): amax inside scale
    ("fp8_quantize_rows", [A, 0, 2, 16, B, C, _at(2, 4), NULL]),
    # fp8_gemm_rowwise(qa, sa, qw, sw, y, M, N, K): y over sw[N]
    ("fp8_gemm_rowwise", [A, B, C, D, _at(3, 32), 1, 16, 16, NULL]),
    # fp8_linear_rowwise(x, dtype, qw, sw, y, q, sa, amax, M, N, K): amax inside sa[M]
    ("fp8_linear_rowwise", [A, 0, C, D, B, E, F, _at(5, 4), 2, 1, 16, NULL]),
    # nested_split(w, hi, lo, n) / nested_rebuild_fp16(hi, lo, w, n)
    ("nested_split", [A, _at(0, 64), C, 64, NULL]),
    ("nested_split", [A, B, B, 64, NULL]),
    ("nested_rebuild_fp16", [A, B, _at(1, 48), 64, NULL]),
    ("nested_split_e4m3", [A, B, C, 64, _at(1, 8), NULL]),
    ("nested_rebuild_e4m3", [A, B, A, 64, NULL]),
    # nested_gemm_fp16(a, hi, lo, y, M, N, K) / nested_gemm_fp8(qa, sa, hi, y, M, N, K)
    ("nested_gemm_fp16", [A, B, C, A, 1, 1, 16, NULL]),
    ("nested_gemm_fp16_e4m3", [A, B, C, C, 1, 1, 16, NULL]),
    ("nested_gemm_fp8", [A, B, C, C, 1, 1, 16, NULL]),
    ("nested_gemm_fp8_e4m3", [A, B, C, B, 1, 1, 16, NULL]),
    # nested_linear_fp8(a, hi, y, q, scale, amax, M, N, K): q over a, y over hi
    ("nested_linear_fp8", [A, B, C, A, E, F, 1, 1, 16, NULL]),
    ("nested_linear_fp8_e4m3", [A, B, B, D, E, F, 1, 1, 16, NULL]),
    # fp8q_e4m3_encode_f32(v, q, n): codes over the values
    ("fp8q_e4m3_encode_f32", [A, _at(0, 16), 16, NULL]),
])
def test_overlapping_outputs_rejected_before_any_hip_call(fn, args):
    """An output sharing bytes with another buffer of the call is refused
    with FP8Q_ERR_OVERLAP; nothing is launched (the pointers are never
    dereferenced)."""
    assert getattr(fp8q.lib, fn)(*args) == ERR_OVERLAP


def test_binding_raises_on_cpu_tensors():
    import torch
    with pytest.raises(TypeError):
        fp8q.fp8_quantize_act(torch.zeros(8, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        fp8q.fp8_quantize_act(torch.zeros(8, dtype=torch.float32))


def test_error_type_carries_status():
    e = fp8q.Fp8qError("fp8_gemm", ERR_SHAPE)
    assert e.status == ERR_SHAPE and "size out of range" in str(e)


def test_package_exports_every_binding():
    """Every entry point of the binding is reachable from the package itself."""
    import fp8_quantized_gemm_amd as pkg

    public = {n for n in dir(fp8q) if not n.startswith("_") and callable(getattr(fp8q, n))
              and getattr(getattr(fp8q, n), "__module__", "") == fp8q.__name__}
    assert public <= set(pkg.__all__), sorted(public - set(pkg.__all__))
    for name in pkg.__all__:
        assert getattr(pkg, name) is getattr(fp8q, name)
