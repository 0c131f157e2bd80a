"""Shared helpers for the GPU parity tests (host-side marshalling only)."""
import sys

import numpy as np
import torch

import oracle
from fp8_quantized_gemm_amd import synth

DEV = "cuda:0"


def say(*args):
    """Name the case before a GPU step, flushed, so a fault report names it."""
    print("[case]", *args, flush=True)
    sys.stdout.flush()


def to_dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(DEV)


def to_dev_bits(b: np.ndarray, dtype: str) -> torch.Tensor:
    return synth.from_bits(b, dtype).to(DEV)


def scalar_dev(v: float) -> torch.Tensor:
    return torch.tensor([v], dtype=torch.float32, device=DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype in (torch.bfloat16, torch.float16):
        return synth.bits(t)
    return t.detach().cpu().numpy()


def f32_bits(v: float) -> int:
    return int(np.float32(v).view(np.uint32))


def oracle_quantize_rows(x_bits: np.ndarray, dtype_code: int, s: float) -> np.ndarray:
    return oracle.quantize_with_scale(x_bits, dtype_code, s)


def assert_within(out_vals: np.ndarray, ref: np.ndarray, ab: np.ndarray, what: str,
                  out_format: str):
    ok = oracle.within_tolerance(out_vals, ref, ab, out_format)
    if not np.all(ok):
        bad = np.nonzero(~ok)[0]
        i = bad[0]
        raise AssertionError(
            f"{what}: {bad.size}/{ok.size} outside tolerance; first at flat index {i}: "
            f"out={out_vals[i]!r} ref={ref[i]!r} absref={ab[i]!r}")


def dense_sample(M, N, rng, rows=32, cols=32):
    """Output positions checked against the oracle at full size: every element
    when M <= 16; otherwise `rows` seeded rows across all N plus `cols` seeded
    columns across all M.  Returns (ms, ns) flat index arrays."""
    if M <= 16:
        mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        return mm.ravel(), nn.ravel()
    r = np.sort(rng.choice(M, min(rows, M), replace=False))
    c = np.sort(rng.choice(N, min(cols, N), replace=False))
    ms = np.concatenate([np.repeat(r, N), np.tile(np.arange(M), c.size)])
    ns = np.concatenate([np.tile(np.arange(N), r.size), np.repeat(c, M)])
    return ms, ns
