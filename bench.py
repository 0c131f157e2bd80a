"""Benchmark of the FP8 linear-layer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-secondary] [--eager]

Workload (one "step"): the 32 layers of Llama-7B-shaped decode linears at
M = 1 token (fused QKV 4096->12288, O 4096->4096, gate+up 4096->22016,
down 11008->4096), each one a dynamic per-tensor E4M3 quantization of its bf16
activation followed by the FP8 GEMM against statically quantized E4M3 weights
(fp32 accumulation, bf16 output), issued as one fp8_linear call per linear
(a single fused kernel at M = 1).  The 128 weight matrices are distinct
(6.48 GB of FP8 codes), so every step streams them from HBM.

`value` is whole-step algorithmic HBM traffic divided by the step time
(GB/s): per linear N*K weight bytes + M*K code bytes + 2*M*N output bytes for
the GEMM and 3*M*K bytes for the quantizer.  Inputs are resident in HBM
before timing.  By default the 128 launches of a step are captured once into
a HIP graph and the timed steps are graph replays.  `roofline` reports the
decode kernel alone: its algorithmic bytes over its average duration,
measured with a HIP event pair around the timed region on the replay stream (the step
is the 128 launches of that one kernel, so device time over launch count is
its average launch duration, inter-launch gaps included).  `traffic` is
the HBM bytes per launch from hardware counters, read from the committed
counter summary when it was taken on the current kernel source.
`secondary` adds the prefill (M = 512, 2048: TFLOP/s of the tile GEMM) and
NestedFP figures; `cpu_baseline` times the oracle on a bounded sample.
Rank 0 prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0      # dense FP8 MFMA
FP16_PEAK_TFLOPS = 2500.0     # dense FP16 MFMA
LAYERS = 32
QWEN_LAYERS = 64
CFG1_COPIES = 64              # 64 x 16 MiB of weights: beyond the 256 MB last-level cache
METRIC = "FP8 linear: HBM GB/s @M=1 and TFLOP/s @M=512, % of MI355X peak"
PARTS = ("cfg1", "decode", "prefill", "delayed", "qwen", "rowwise", "kv", "nested")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--eager", action="store_true",
                   help="launch every kernel from Python instead of replaying the step as "
                        "one captured HIP graph")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="lower bound on the oracle's timed CPU work")
    p.add_argument("--only-prefill", action="store_true",
                   help="run only the prefill figures (M = 512, 2048) and print them: the "
                        "command that the prefill GEMM's rocprofv3 summaries are taken on")
    p.add_argument("--only", default="", metavar="PARTS",
                   help="run only these secondary figures (comma-separated: " +
                        ", ".join(PARTS) + ") and print them as one JSON line, without the "
                        "headline step: the commands the per-kernel rocprofv3 summaries "
                        "are taken on")
    p.add_argument("--copy-calibration-mib", type=int, default=0, metavar="MIB",
                   help="instead of the benchmark, run 5 launches of a plain elementwise "
                        "copy (read MIB MiB, write MIB MiB) so that HBM byte counters "
                        "can be calibrated against a kernel of known traffic")
    return p.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("linear.hip", "common.hpp"):
        with open(os.path.join(ROOT, "fp8_quantized_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(src_hash: str):
    """HBM traffic per GEMV launch from the committed counter summary, if it
    was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "rowk_f8_llama7b_decode_m1_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != src_hash:
        return None
    return d.get("traffic_bytes_per_launch")


class Model:
    """Device-resident weights and per-linear buffers of one decode workload."""

    def __init__(self, torch, fp8q, synth, M: int, dev: str, spec=None, layers: int = LAYERS,
                 sigma: float = 0.02, tag: str = "w", rowwise: bool = False):
        self.M = M
        self.linears = []
        for layer in range(layers):
            for name, K, N in (spec if spec is not None else synth.LLAMA7B_LINEARS):
                w = synth.normal((N, K), sigma, "fp16", seed=synth.seed_for(tag, layer, name),
                                 device=dev)
                # offline static quantization: one scale per tensor, or per
                # output channel
                qw, sw, _ = fp8q.fp8_quantize_rows(w) if rowwise else fp8q.fp8_quantize_act(w)
                del w
                self.linears.append(dict(layer=layer, name=name, K=K, N=N, qw=qw, sw=sw,
                                         rowwise=rowwise))
        for L in self.linears:
            K, N = L["K"], L["N"]
            L["x"] = synth.activation(M, K, seed=synth.seed_for("x", M, L["layer"], L["name"]),
                                      device=dev)
            L["q"] = torch.empty((M, K), dtype=torch.uint8, device=dev)
            L["sa"] = torch.empty(M if rowwise else 1, dtype=torch.float32, device=dev)
            L["amax"] = torch.empty(M if rowwise else 1, dtype=torch.float32, device=dev)
            L["y"] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()

    def gemm_bytes(self, L):
        M, K, N = self.M, L["K"], L["N"]
        return N * K + M * K + 2 * M * N

    def quant_bytes(self, L):
        return 3 * self.M * L["K"]

    def flops(self, L):
        return 2 * self.M * L["N"] * L["K"]


def linear_call(fp8q, L):
    fn = fp8q.fp8_linear_rowwise if L["rowwise"] else fp8q.fp8_linear
    fn(L["x"], L["qw"], L["sw"], L["y"], L["q"], L["sa"], L["amax"])


def delayed_call(fp8q, L):
    fp8q.fp8_linear_delayed(L["x"], L["qw"], L["sw"], L["ds"], L["y"], L["q"], L["sa"], L["amax"])


def gemm_call(fp8q, L):
    fn = fp8q.fp8_gemm_rowwise if L["rowwise"] else fp8q.fp8_gemm
    fn(L["q"], L["sa"], L["qw"], L["sw"], L["y"])


def run_step(fp8q, model, events=None, call=linear_call):
    """One pass over every linear (by default dynamic quantization + FP8 GEMM,
    fp8_linear).  With `events`, a HIP event pair brackets each call on its
    stream."""
    for i, L in enumerate(model.linears):
        if events is not None:
            events[i][0].record()
        call(fp8q, L)
        if events is not None:
            events[i][1].record()


def time_fn(torch, fn, steps, warmup, graph=True):
    """Time `steps` calls of fn() (one step each).  With `graph`, fn's launches
    are captured once into a HIP graph and the timed steps are replays.
    Returns (wall seconds per step, device seconds per step): the second from
    a HIP event pair recorded on the stream the work runs on (torch's current
    stream) around the whole timed region."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    g = None
    if graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()                             # warm on the capture stream
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                fn()
        torch.cuda.synchronize()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        if g is not None:
            g.replay()
        else:
            fn()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    return wall, e0.elapsed_time(e1) * 1e-3 / steps


def time_steps(torch, fp8q, model, steps, warmup, graph=True, call=linear_call):
    return time_fn(torch, lambda: run_step(fp8q, model, call=call), steps, warmup, graph)


def cpu_baseline(torch, synth, dev, seconds):
    """The oracle (quantize + fp32-accumulating GEMM) on a bounded sample of
    the same decode workload: layers 0..L-1, repeated until `seconds` pass."""
    import numpy as np
    import oracle

    threads = oracle.default_threads()
    work = []
    for layer in range(2):
        for name, K, N in synth.LLAMA7B_LINEARS:
            w = synth.normal((N, K), 0.02, "fp16", seed=synth.seed_for("w", layer, name), device=dev)
            wb = synth.bits(w).ravel()
            del w
            qw, sw, _ = oracle.quantize(wb, oracle.FP16)            # offline, untimed
            x = synth.activation(1, K, seed=synth.seed_for("x", 1, layer, name), device=dev)
            work.append((synth.bits(x).ravel(), qw.reshape(N, K), sw, K, N))
    done_bytes = 0
    passes = 0
    t0 = time.perf_counter()
    while True:
        for xb, qw, sw, K, N in work:
            qa, sa, _ = oracle.quantize(xb, oracle.BF16)
            oracle.gemm_fp8_f32(qa.reshape(1, K), sa, qw, sw, nthreads=threads)
            done_bytes += N * K + K + 2 * N + 3 * K
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(done_bytes / el / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"layers 0-1 of the 32 (8 linears, M=1), {passes} pass(es), "
                      f"{el:.1f} s of CPU work on {threads} threads of {host_cpu()} "
                      f"({os.cpu_count()} logical CPUs visible); same algorithmic bytes as "
                      f"the GPU metric"}


def host_cpu() -> str:
    """The host CPU's model name (Linux), for the record of the oracle's timing."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "an unknown CPU"


def with_activations(torch, synth, model1, M, dev, tag, outliers=False):
    """The weights of `model1` with fresh M-row activations and outputs."""
    mm = Model.__new__(Model)
    mm.M = M
    mm.linears = []
    for L in model1.linears:
        K, N = L["K"], L["N"]
        d = dict(L)
        d["x"] = synth.activation(M, K, seed=synth.seed_for(tag, M, L["layer"], L["name"]),
                                  outliers=outliers, device=dev)
        d["q"] = torch.empty((M, K), dtype=torch.uint8, device=dev)
        d["y"] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        if L["rowwise"]:
            d["sa"] = torch.empty(M, dtype=torch.float32, device=dev)
            d["amax"] = torch.empty(M, dtype=torch.float32, device=dev)
        mm.linears.append(d)
    return mm


def decode_figures(torch, fp8q, mm, graph=True, call=linear_call):
    dt, _ = time_steps(torch, fp8q, mm, steps=5, warmup=2, graph=graph, call=call)
    byts = sum(mm.gemm_bytes(L) + mm.quant_bytes(L) for L in mm.linears)
    return {"GB_per_s": round(byts / dt / 1e9, 1),
            "frac_hbm": round(byts / dt / 1e9 / HBM_PEAK_GBS, 4),
            "ms_per_step": round(dt * 1e3, 3)}


def prefill_figures(torch, fp8q, mm, graph=True, call=linear_call):
    dt, _ = time_steps(torch, fp8q, mm, steps=3, warmup=1, graph=graph, call=call)
    # the GEMM alone, on the codes and scales the timed steps left behind
    _, gdev = time_steps(torch, fp8q, mm, steps=3, warmup=1, graph=graph, call=gemm_call)
    fl = sum(mm.flops(L) for L in mm.linears)
    return {"TFLOP_per_s": round(fl / dt / 1e12, 1),
            "frac_fp8_mfma": round(fl / dt / 1e12 / FP8_PEAK_TFLOPS, 4),
            "gemm_only_TFLOP_per_s": round(fl / gdev / 1e12, 1),
            "ms_per_step": round(dt * 1e3, 3)}


def single_linear_figure(torch, fp8q, synth, dev, graph=True):
    """The single 4096 -> 4096 linear at M = 1 (fp16 N(0, 0.02) weights
    quantized per tensor, bf16 N(0, 1) activation quantized per call):
    one fp8_linear call on each of CFG1_COPIES distinct weight copies per step,
    so every call reads its 16 MiB of codes from HBM rather than from the
    256 MB last-level cache."""
    K = N = 4096
    mm = Model.__new__(Model)
    mm.M = 1
    mm.linears = []
    for c in range(CFG1_COPIES):
        w = synth.normal((N, K), 0.02, "fp16", seed=synth.seed_for("cfg1-w", c), device=dev)
        qw, sw, _ = fp8q.fp8_quantize_act(w)
        del w
        mm.linears.append(dict(layer=c, name="single", K=K, N=N, qw=qw, sw=sw, rowwise=False,
                               x=synth.activation(1, K, seed=synth.seed_for("cfg1-x", c),
                                                  device=dev),
                               q=torch.empty((1, K), dtype=torch.uint8, device=dev),
                               sa=torch.empty(1, dtype=torch.float32, device=dev),
                               amax=torch.empty(1, dtype=torch.float32, device=dev),
                               y=torch.empty((1, N), dtype=torch.bfloat16, device=dev)))
    torch.cuda.synchronize()
    dt, dev_dt = time_steps(torch, fp8q, mm, steps=10, warmup=3, graph=graph)
    byts = sum(mm.gemm_bytes(L) + mm.quant_bytes(L) for L in mm.linears)
    per_launch = dev_dt / len(mm.linears)
    return {"GB_per_s": round(byts / dt / 1e9, 1),
            "frac_hbm": round(byts / dt / 1e9 / HBM_PEAK_GBS, 4),
            "us_per_linear": round(per_launch * 1e6, 3),
            "algorithmic_bytes_per_linear": byts // len(mm.linears),
            "weight_copies": CFG1_COPIES}


def secondary(torch, fp8q, synth, model1, dev, parts=PARTS, graph=True):
    """The single-linear, prefill, M = 4/8 decode, delayed scaling, Qwen-32B,
    per-token/per-channel, KV-cache and NestedFP figures (a few steps each)."""
    out = {}
    if "cfg1" in parts:
        out["single_4096x4096_m1"] = single_linear_figure(torch, fp8q, synth, dev, graph)
        progress("single linear done")
    # decode at M = 4, 8 on the same weights (activations re-drawn)
    for M in ((4, 8) if "decode" in parts else ()):
        out[f"decode_m{M}"] = decode_figures(torch, fp8q, with_activations(torch, synth, model1, M,
                                                                           dev, "x"), graph)
        progress(f"decode M={M} done")
    # prefill M = 512, 2048 (activations with 0.1% outlier channels x50)
    for M in ((512, 2048) if "prefill" in parts else ()):
        mm = with_activations(torch, synth, model1, M, dev, "xp", outliers=True)
        out[f"prefill_m{M}"] = prefill_figures(torch, fp8q, mm, graph)
        progress(f"prefill M={M} done")
        del mm
    # delayed scaling (amax history of 1024 per linear) on the same 32 layers:
    # the activation is quantized in one pass with the history's scale
    if "delayed" in parts:
        for L in model1.linears:
            L["ds"] = fp8q.DelayedScaling(1024, device=dev)
        out["delayed_decode_m1"] = decode_figures(torch, fp8q, model1, graph, call=delayed_call)
        mm = with_activations(torch, synth, model1, 512, dev, "xp", outliers=True)
        out["delayed_prefill_m512"] = prefill_figures(torch, fp8q, mm, graph, call=delayed_call)
        progress("delayed scaling done")
        del mm
        for L in model1.linears:
            del L["ds"]
    # Qwen-32B linears (weights N(0, 0.015)) on all 64 layers: 31.2 GB of E4M3
    # weights, cold in HBM on every step; decode M = 1, 16, prefill M = 1024
    if "qwen" in parts:
        mq = Model(torch, fp8q, synth, M=1, dev=dev, spec=synth.QWEN32B_LINEARS,
                   layers=QWEN_LAYERS, sigma=0.015, tag="wq")
        progress("qwen-32b model built")
        out["qwen32b_decode_m1"] = dict(decode_figures(torch, fp8q, mq, graph), layers=QWEN_LAYERS)
        out["qwen32b_decode_m16"] = dict(decode_figures(
            torch, fp8q, with_activations(torch, synth, mq, 16, dev, "xq"), graph),
            layers=QWEN_LAYERS)
        out["qwen32b_prefill_m1024"] = dict(prefill_figures(
            torch, fp8q, with_activations(torch, synth, mq, 1024, dev, "xqp"), graph),
            layers=QWEN_LAYERS)
        progress("qwen-32b done")
        del mq
    # per-token activation and per-channel weight scales (fp8_linear_rowwise)
    # on all 32 Llama-7B layers: 6.48 GB of E4M3 weights, cold in HBM on every step
    if "rowwise" in parts:
        mr = Model(torch, fp8q, synth, M=1, dev=dev, layers=LAYERS, tag="w", rowwise=True)
        out["rowwise_decode_m1"] = dict(decode_figures(torch, fp8q, mr, graph), layers=LAYERS)
        out["rowwise_prefill_m512"] = dict(prefill_figures(
            torch, fp8q, with_activations(torch, synth, mr, 512, dev, "xp", outliers=True), graph),
            layers=LAYERS)
        progress("per-token / per-channel done")
        del mr
    # FP8 KV cache: the K and V blocks of 8 layers, each 4096 tokens x 32 heads x
    # 128 (bf16, 32 MiB), one scale per head; a step quantizes all 16 blocks
    # (16 calls, one graph); algorithmic bytes 2 read + 1 written per element
    if "kv" in parts:
        blocks = [synth.activation(4096, 32 * 128, seed=77 + b, device=dev).reshape(4096, 32, 128)
                  for b in range(16)]
        outs = [(torch.empty((4096, 32, 128), dtype=torch.uint8, device=dev),
                 torch.empty(32, dtype=torch.float32, device=dev),
                 torch.empty(32, dtype=torch.float32, device=dev)) for _ in blocks]

        def kv_step():
            for x, (q, s, a) in zip(blocks, outs):
                fp8q.fp8_quantize_kv(x, q, s, a)

        dt, _ = time_fn(torch, kv_step, steps=10, warmup=2, graph=graph)
        byts = 3 * sum(x.numel() for x in blocks)
        out["kv_quantize_16x4096x32x128"] = {"GB_per_s": round(byts / dt / 1e9, 1),
                                             "frac_hbm": round(byts / dt / 1e9 / HBM_PEAK_GBS, 4),
                                             "us_per_block": round(dt * 1e6 / len(blocks), 2)}
        progress("kv cache done")
        del blocks, outs
    if "nested" not in parts:
        return out
    # NestedFP at M = 1 and 256 on all 32 layers of fp16 weights (hi/lo planes:
    # 12.95 GB, and as much again for the E4M3 upper-byte split), and at the
    # decode sizes M = 4, 8 of the GEMV path
    nested = []
    nested4 = []                       # planes of the E4M3 upper-byte split
    for layer in range(LAYERS):
        for name, K, N in synth.LLAMA7B_LINEARS:
            w = synth.normal((N, K), 0.02, "fp16", seed=synth.seed_for("w", layer, name), device=dev)
            hi, lo = fp8q.nested_split(w)
            hi4, lo4, _ = fp8q.nested_split_e4m3(w)
            del w
            nested.append((K, N, hi, lo))
            nested4.append((hi4, lo4))
    for M in (1, 4, 8, 256):
        bufs = []
        for K, N, hi, lo in nested:
            a = synth.activation(M, K, seed=synth.seed_for("a16", M, K, N), dtype="fp16", device=dev)
            bufs.append((a, torch.empty((M, K), dtype=torch.uint8, device=dev),
                         torch.empty(1, dtype=torch.float32, device=dev),
                         torch.empty(1, dtype=torch.float32, device=dev),
                         torch.empty((M, N), dtype=torch.float16, device=dev)))

        def step16():
            for (K, N, hi, lo), (a, q, s, am, y) in zip(nested, bufs):
                fp8q.nested_gemm_fp16(a, hi, lo, y)

        def step8():
            for (K, N, hi, lo), (a, q, s, am, y) in zip(nested, bufs):
                fp8q.nested_linear_fp8(a, hi, y, q, s, am)

        def step16e():
            for (K, N, _, _), (hi4, lo4), (a, q, s, am, y) in zip(nested, nested4, bufs):
                fp8q.nested_gemm_fp16_e4m3(a, hi4, lo4, y)

        def step8e():
            for (K, N, _, _), (hi4, _), (a, q, s, am, y) in zip(nested, nested4, bufs):
                fp8q.nested_linear_fp8_e4m3(a, hi4, y, q, s, am)

        for mode, fn, wbytes in (("fp16", step16, 2), ("fp8", step8, 1),
                                 ("fp16_e4m3split", step16e, 2), ("fp8_e4m3split", step8e, 1)):
            dt, _ = time_fn(torch, fn, steps=5, warmup=2, graph=graph)
            byts = sum(wbytes * N * K + 2 * M * K + 2 * M * N for K, N, _, _ in nested)
            if mode.startswith("fp8"):
                byts = sum(N * K + M * K + 2 * M * N + 3 * M * K for K, N, _, _ in nested)
            fl = sum(2 * M * N * K for K, N, _, _ in nested)
            peak = FP16_PEAK_TFLOPS if mode.startswith("fp16") else FP8_PEAK_TFLOPS
            out[f"nested_{mode}_m{M}"] = {"GB_per_s": round(byts / dt / 1e9, 1),
                                          "frac_hbm": round(byts / dt / 1e9 / HBM_PEAK_GBS, 4),
                                          "TFLOP_per_s": round(fl / dt / 1e12, 2),
                                          "frac_mfma": round(fl / dt / 1e12 / peak, 4),
                                          "layers": LAYERS}
            progress(f"nested {mode} M={M} done")
    return out


def progress(msg):
    """Phase marker on stderr (stdout carries only the JSON result line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def copy_calibration(torch, mib):
    """A plain copy kernel of known traffic (torch's elementwise bitwise_not on
    int32: reads and writes mib MiB per launch) for scaling byte counters."""
    n = mib * (1 << 20) // 4
    x = torch.arange(n, dtype=torch.int32, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(5):
        torch.bitwise_not(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_launch": n * 4,
                                           "bytes_written_per_launch": n * 4,
                                           "launches": 5}}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_calibration_mib > 0:
        copy_calibration(torch, args.copy_calibration_mib)
        return

    from fp8_quantized_gemm_amd import fp8q, synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    model = Model(torch, fp8q, synth, M=1, dev=dev)
    progress("decode model built (128 E4M3 weight matrices)")
    if args.only_prefill or args.only:
        parts = ("prefill",) if args.only_prefill else tuple(args.only.split(","))
        bad = [p for p in parts if p not in PARTS]
        if bad:
            print(f"unknown parts {bad}; choose from {PARTS}", file=sys.stderr)
            sys.exit(2)
        print(json.dumps({"secondary": secondary(torch, fp8q, synth, model, dev, parts=parts,
                                                 graph=not args.eager)}), flush=True)
        return
    graph = not args.eager
    dt, dev_step = time_steps(torch, fp8q, model, args.steps, args.warmup, graph=graph)
    step_bytes = sum(model.gemm_bytes(L) + model.quant_bytes(L) for L in model.linears)
    value = step_bytes / dt / 1e9
    # The step is the 128 launches of the decode kernel and nothing else, so
    # the event-timed device time of the timed region over its launch count is
    # that kernel's average launch duration (inter-launch gaps included).
    kern = dev_step / len(model.linears)
    progress(f"timed {args.steps} steps: {dt * 1e3:.3f} ms/step, {kern * 1e6:.2f} us/launch")
    launch_bytes = step_bytes / len(model.linears)
    achieved = launch_bytes / kern / 1e9
    src_hash = kernel_source_hash()
    traffic = load_traffic(src_hash)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic",
        "config": {"workload": "llama7b_decode_m1_32layers", "M": 1, "layers": LAYERS,
                   "linears_K_N": [[K, N] for _, K, N in synth.LLAMA7B_LINEARS],
                   "weights": "fp16 N(0,0.02) -> E4M3 per-tensor", "activations": "bf16 N(0,1)",
                   "frac_hbm_step": round(value / HBM_PEAK_GBS, 4),
                   "launch": "hip_graph_replay" if graph else "eager"},
        "roofline": {"bound": "hbm",
                     "kernel": "rowk_f8_kernel, fused quantize + FP8 GEMM (fp8_linear, M=1)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "avg_launch_us": round(kern * 1e6, 3),
                     "algorithmic_bytes_per_launch": int(launch_bytes),
                     "traffic": traffic, "kernel_source_hash": src_hash},
    }
    if not args.no_secondary:
        result["secondary"] = secondary(torch, fp8q, synth, model, dev)
        progress("secondary figures done")
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(torch, synth, dev, args.cpu_seconds)
        progress("cpu baseline done")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
