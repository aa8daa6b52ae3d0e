"""Benchmark of the FP8 linear-layer hot path on one MI355X.

Default workload (one "step"): the four Llama-3.1-8B-shaped fprop linear layers at M = 8192
tokens -- QKV 4096->6144, O 4096->4096, gate+up 4096->28672, down 14336->4096.  The step
re-quantizes the four bf16 weights (128x128 tiles, E4M3: the per-step scale recalibration) in
one batched launch, then for each layer quantizes the bf16 activation (1x128 blocks, E4M3) and
runs the block-scaled FP8 GEMM with fp32 accumulation and bf16 output.  Inputs are seeded synthetic bf16 tensors resident in
HBM before timing: activations N(0,1) with 1% of the channels scaled by 50, weights N(0,0.02).

value = sum of the GEMMs' 2*M*N*K over the step / step time (TFLOP/s, quantization included).
roofline: the dominant kernel (the block-scaled GEMM) -- algorithmic flops per launch (mean
over the four shapes) / mean launch duration measured with HIP events on the launch stream,
against the MI355X dense FP8 MFMA peak.  traffic: HBM bytes per launch (mean over the four
shapes) from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, calibrated on a plain copy;
null when the GEMM sources differ from the ones the counters were taken on.
cpu_baseline: the CPU oracle (C quantizer + NumPy fp64 GEMM) on the same step (all rows of all
four layers), on the host's cores.

Other workloads (--workload): llama8b-fprop-pow2 (the same step with power-of-2 scales, the
GEMM applying them as E8M0 block scales in the MFMA), quant-sweep (HBM-bound quantizer), moe
(grouped GEMM; --pow2 for power-of-2 scales), backward (delayed-scaled dgrad / wgrad),
backward-blockwise (dgrad + blockwise wgrad on columnwise-quantized operands; --pow2),
llama8b-fprop-qout (the GEMM quantizing its own output against GEMM + quantizer),
llama8b-fprop-mx (the same step in microscaling form: 32-element row blocks with E8M0 scale
bytes on X and W, the scales applied by the scaled MFMA), backward-mx (dgrad + wgrad in
microscaling form, operands quantized along rows or, transposed, along columns), kv-decode
(FP8 KV-cache write + grouped-query decode attention, Llama-3.1-8B attention shape), copy
(counter calibration).  Each prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
GEMM_COUNTERS = os.path.join(ROOT, "profiles", "gemm_kernel_llama8b_fprop_counters.txt")
GEMM_COUNTERS_POW2 = os.path.join(ROOT, "profiles", "gemm_kernel_pow2_llama8b_fprop_counters.txt")
GEMM_COUNTERS_MX = os.path.join(ROOT, "profiles", "gemm_kernel_mx_llama8b_fprop_counters.txt")
QUANT_COUNTERS = os.path.join(ROOT, "profiles", "quantize_kernels_sweep_counters.txt")
QUANT_SOURCES = [os.path.join(ROOT, "block_scaled_quantize_amd", "csrc", f)
                 for f in ("quantize.hip", "common.h")]
GEMM_SOURCES = [os.path.join(ROOT, "block_scaled_quantize_amd", "csrc", f)
                for f in ("gemm_impl.h", "gemm.hip", "gemm_fprop.hip", "gemm_fprop_pow2.hip",
                          "gemm_dgrad.hip", "gemm_wgrad.hip", "gemm_grouped.hip", "gemm_mx.hip",
                          "common.h")]

LAYERS_8B = [("qkv", 4096, 6144), ("o", 4096, 4096), ("gate_up", 4096, 28672), ("down", 14336, 4096)]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b-fprop",
                    choices=["llama8b-fprop", "llama8b-fprop-pow2", "quant-sweep", "moe", "backward",
                             "backward-blockwise", "llama8b-fprop-qout", "kv-decode", "copy", "stream",
                             "mfma-ceiling", "llama8b-fprop-mx", "backward-mx"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pow2", action="store_true",
                    help="moe, backward-blockwise: power-of-2 scales (E8M0 in the MFMA)")
    ap.add_argument("--mx", action="store_true",
                    help="moe: microscaling scales (32-element blocks, E8M0 bytes)")
    ap.add_argument("--tokens", type=int, default=8192)
    ap.add_argument("--kv-split", type=int, default=-1,
                    help="kv-decode: tokens per chunk of fp8_attention_decode_split (0: unsplit, "
                         "-1: the binding's choice for the batch)")
    ap.add_argument("--kv-batch", type=int, default=64, help="kv-decode: sequences")
    return ap.parse_args()


class EventTimer:
    """HIP events recorded on the stream the kernels are launched on."""

    def __init__(self):
        self.pairs = {}

    def time(self, key, fn):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        out = fn()
        e.record()
        self.pairs.setdefault(key, []).append((s, e))
        return out

    def mean_ms(self, key) -> float:
        v = [s.elapsed_time(e) for s, e in self.pairs.get(key, [])]
        return float(np.mean(v)) if v else float("nan")

    def total_ms(self, key) -> float:
        return float(sum(s.elapsed_time(e) for s, e in self.pairs.get(key, [])))


def measured_traffic(counter_file: str, sources) -> dict:
    """HBM bytes per launch from a committed counter summary (key = value lines), if it was
    taken on the current kernel sources (sha256 over the source files), else None."""
    import hashlib
    out = dict(bytes=None, algorithmic=None, source="none")
    try:
        kv = {}
        for line in open(counter_file):
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
        h = hashlib.sha256()
        for p in sources:
            with open(p, "rb") as f:
                h.update(f.read())
    except OSError:
        return out
    out["algorithmic"] = float(kv["mean_algorithmic_bytes_per_launch"])
    if kv.get("source_sha256") == h.hexdigest():
        out["bytes"] = float(kv["mean_hbm_bytes_per_launch"])
        out["source"] = os.path.relpath(counter_file, ROOT)
    else:
        out["source"] = "stale: kernel sources changed since the counters were taken"
    return out


def cpu_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# ----------------------------------------------------------------------------- matrix-core ceiling

def mfma_sustained(codes, shape: int = 0, launches: int = 20, steps: int = 1000) -> float:
    """TFLOP/s the matrix core sustains on register operands holding `codes` (16384 E4M3 bytes
    on the GPU: 8 operand sets of 64 lanes x 32 bytes) -- independent MFMAs in a loop, 512-thread
    workgroups (two waves per SIMD, as the GEMM tiles), one per CU (each takes 96 KiB of LDS), no
    memory traffic inside the loop (libfp8bs_bench.so).  shape 0: 16x16x128, 1: 32x32x64.  Mean
    over `launches` back-to-back launches of about a millisecond each, after 3 warm-up launches."""
    blib = ctypes.CDLL(os.path.join(ROOT, "block_scaled_quantize_amd", "libfp8bs_bench.so"))
    blib.fp8bs_bench_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    blib.fp8bs_bench_mfma.restype = ctypes.c_int
    codes = codes.contiguous()
    assert codes.dtype == torch.uint8 and codes.numel() == 16384 and codes.is_cuda
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cus * 512, dtype=torch.float32, device=codes.device)
    stream = torch.cuda.current_stream().cuda_stream

    def launch():
        rc = blib.fp8bs_bench_mfma(codes.data_ptr(), out.data_ptr(), shape, steps, cus, 96 * 1024,
                                   stream)
        if rc != 0:
            raise RuntimeError("fp8bs_bench_mfma failed")
    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(launches)]
    for a, b in ev:
        a.record()
        launch()
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    flops = 2.0 * cus * 8 * steps * 32 * 16 * 16 * 128
    return flops / ms / 1e9


def bench_mfma_ceiling(args):
    """The rate the matrix core sustains on register operands (no memory traffic): the practical
    ceiling of an FP8 GEMM with the same operand bits, against the 5.0 PFLOP/s dense peak (which
    assumes the peak shader clock).  Codes: those of the 8B fprop workload's gate_up layer
    (weights, normal(0, 0.02), 128x128 scales; activations with outlier channels, 1x128 scales),
    uniform random E4M3 codes of magnitude below 448, and zeros."""
    import block_scaled_quantize_amd as bsq
    import synth
    bsq.load()
    dev = torch.device("cuda", 0)
    w = synth.normal((64, 128), 0.02, 0, "bench/8b/gate_up/W").to(dev)
    x = synth.activations_with_outliers(64, 128, 0, "bench/8b/gate_up/X").to(dev)
    qw, _ = bsq.quantize_blockwise(w, bsq.E4M3, bsq.BLOCK_128x128, bsq.SCALE_FP32)
    qx, _ = bsq.quantize_blockwise(x, bsq.E4M3, bsq.BLOCK_1x128, bsq.SCALE_FP32)
    g = torch.Generator().manual_seed(0)
    rnd = (torch.randint(0, 0x7F, (16384,), generator=g, dtype=torch.int32) |
           (torch.randint(0, 2, (16384,), generator=g, dtype=torch.int32) << 7)).to(torch.uint8)
    sets = {"8b_gate_up_codes": torch.cat([qw.reshape(-1), qx.reshape(-1)]),
            "uniform_random_codes": rnd.to(dev),
            "zeros": torch.zeros(16384, dtype=torch.uint8, device=dev)}
    cases = {}
    for name, codes in sets.items():
        for shape, label in ((0, "16x16x128"), (1, "32x32x64")):
            tf = mfma_sustained(codes, shape, launches=max(args.steps, 10))
            cases[f"{name}/{label}"] = round(tf, 1)
            log(f"mfma {label} {name}: {tf:.0f} TFLOP/s")
    head = cases["8b_gate_up_codes/16x16x128"]
    return dict(metric="sustained FP8 MFMA TFLOP/s on register operands (matrix-core ceiling)",
                value=head, unit="TFLOP/s", n_gpus=1, steps=max(args.steps, 10), warmup=3,
                ms_per_step=None, higher_is_better=True, scaling="weak", vs_baseline=None,
                dtype="fp8e4m3 x fp8e4m3 -> fp32 acc", data="synthetic",
                config=dict(workload="mfma-ceiling", headline="8B gate_up codes, 16x16x128"),
                roofline=dict(bound="mfma", achieved=head, peak=FP8_PEAK_TFLOPS, unit="TFLOP/s",
                              frac=round(head / FP8_PEAK_TFLOPS, 4), traffic=None,
                              kernel="mfma_loop_kernel (libfp8bs_bench.so)"),
                cases=cases)


# ----------------------------------------------------------------------------- 8B fprop

def bench_llama8b(args, pow2: bool = False):
    """pow2: power-of-2 block scales (SCALE_POW2 quantization, fp8_gemm_blockscaled_pow2)."""
    import block_scaled_quantize_amd as bsq
    import synth
    bsq.load()
    mode = bsq.SCALE_POW2 if pow2 else bsq.SCALE_FP32
    M = args.tokens
    dev = torch.device("cuda", 0)
    layers = []
    log(f"generating inputs for M={M}")
    for name, k, n in LAYERS_8B:
        x = synth.activations_with_outliers(M, k, 0, f"bench/8b/{name}/X").to(dev)
        w = synth.normal((n, k), 0.02, 0, f"bench/8b/{name}/W").to(dev)
        layers.append(dict(
            name=name, K=k, N=n, x=x, w=w,
            qx=torch.empty((M, k), dtype=torch.uint8, device=dev),
            sx=torch.empty(bsq.scale_shape(M, k, bsq.BLOCK_1x128), dtype=torch.float32, device=dev),
            qw=torch.empty((n, k), dtype=torch.uint8, device=dev),
            sw=torch.empty(bsq.scale_shape(n, k, bsq.BLOCK_128x128), dtype=torch.float32, device=dev),
            y=torch.empty((M, n), dtype=torch.bfloat16, device=dev)))
    torch.cuda.synchronize()
    flops = sum(2.0 * M * L["N"] * L["K"] for L in layers)

    def qw_all():
        # every layer's weight re-quantized in one launch (the per-step recalibration)
        bsq.quantize_blockwise_batched([L["w"] for L in layers], [bsq.BLOCK_128x128] * len(layers),
                                       bsq.E4M3, mode, qs=[L["qw"] for L in layers],
                                       scale_invs=[L["sw"] for L in layers])

    def step(timer=None):
        if timer is None:
            qw_all()
        else:
            timer.time(("qw", "all"), qw_all)
        for L in layers:
            def qx():
                bsq.quantize_blockwise(L["x"], bsq.E4M3, bsq.BLOCK_1x128, mode, q=L["qx"],
                                       scale_inv=L["sx"])

            def mm():
                bsq.gemm_blockscaled(bsq.FPROP, L["qx"], bsq.E4M3, bsq.BLOCK_1x128, L["sx"], L["qw"],
                                     bsq.E4M3, bsq.BLOCK_128x128, L["sw"], c=L["y"], pow2=pow2)
            if timer is None:
                qx(); mm()
            else:
                timer.time(("qx", L["name"]), qx)
                timer.time(("gemm", L["name"]), mm)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")
    # whole-step timing (no per-kernel events inside)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    log(f"timed {args.steps} steps: {dt * 1e3:.3f} ms/step")
    # per-kernel durations (separate pass with events around every launch)
    timer = EventTimer()
    for _ in range(max(3, min(args.steps, 10))):
        step(timer)
    torch.cuda.synchronize()
    per_layer = {}
    gemm_ms, gemm_flops = [], []
    qw_ms = timer.mean_ms(("qw", "all"))
    w_bytes = sum(L["N"] * L["K"] * (2 + 1) + 4 * (L["N"] // 128) * (L["K"] // 128) for L in layers)
    q_bytes, q_ms = w_bytes, qw_ms
    for L in layers:
        g = timer.mean_ms(("gemm", L["name"]))
        f = 2.0 * M * L["N"] * L["K"]
        gemm_ms.append(g)
        gemm_flops.append(f)
        qx_ms = timer.mean_ms(("qx", L["name"]))
        xb = M * L["K"] * (2 + 1) + 4 * M * (L["K"] // 128)
        q_bytes += xb
        q_ms += qx_ms
        per_layer[L["name"]] = dict(gemm_us=round(g * 1e3, 2), gemm_tflops=round(f / g / 1e9, 1),
                                    quant_x_us=round(qx_ms * 1e3, 2), quant_x_gbps=round(xb / qx_ms / 1e6, 1))
    mean_launch_flops = float(np.mean(gemm_flops))
    mean_launch_ms = float(np.mean(gemm_ms))
    achieved = mean_launch_flops / mean_launch_ms / 1e9
    traffic = measured_traffic(GEMM_COUNTERS_POW2 if pow2 else GEMM_COUNTERS, GEMM_SOURCES)
    # the matrix core's own sustained rate on this workload's codes (gate_up weight and
    # activation codes in registers, no memory traffic): what the GEMM's clock allows
    gu = layers[2]
    ceiling = mfma_sustained(torch.cat([gu["qw"].reshape(-1)[:8192], gu["qx"].reshape(-1)[:8192]]))
    log(f"matrix core on the workload's codes: {ceiling:.0f} TFLOP/s")
    scales = "power-of-2 (E8M0 in the MFMA)" if pow2 else "fp32"
    result = dict(
        metric="block-scaled FP8 GEMM TFLOP/s (+quantize GB/s), % of MI355X FP8/HBM peak",
        value=round(flops / dt / 1e12, 2), unit="TFLOP/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=round(dt * 1e3, 4), higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype="fp8e4m3 x fp8e4m3 -> fp32 acc -> bf16",
        data="synthetic",
        config=dict(workload="llama3.1-8b-fprop-linear" + ("-pow2" if pow2 else ""), tokens=M,
                    layers="qkv 4096->6144, o 4096->4096, gate_up 4096->28672, down 14336->4096",
                    act_scales="1x128 E4M3", weight_scales="128x128 E4M3 (all four re-quantized every step in one launch)",
                    scale_values=scales, parallelism="single GPU"),
        roofline=dict(bound="mfma", achieved=round(achieved, 1), peak=FP8_PEAK_TFLOPS,
                      unit="TFLOP/s", frac=round(achieved / FP8_PEAK_TFLOPS, 4),
                      traffic=traffic["bytes"], traffic_unit="HBM bytes per launch",
                      traffic_algorithmic=traffic["algorithmic"], traffic_source=traffic["source"],
                      # the tile chooser takes the 256x256 tile for all four shapes
                      kernel="gemm_persistent_kernel<Cfg<256,256,2,4>,FPROP,E4M3,E4M3,%s>" % ("hw" if pow2 else "fold"),
                      per_launch_flops=mean_launch_flops, mean_launch_us=round(mean_launch_ms * 1e3, 2)),
        gemm_only_tflops=round(sum(gemm_flops) / sum(gemm_ms) / 1e9, 1),
        mfma_sustained=dict(tflops=round(ceiling, 1),
                            gemm_frac=round(achieved / ceiling, 4),
                            what="V_MFMA 16x16x128 E4M3 loop on register operands holding the "
                                 "gate_up layer's weight and activation codes, two waves per "
                                 "SIMD, no memory traffic (libfp8bs_bench.so): the rate the "
                                 "clock allows with these operand bits"),
        quant_gbps=round(q_bytes / q_ms / 1e6, 1),
        quant_hbm_frac=round(q_bytes / q_ms / 1e6 / HBM_PEAK_GBPS, 4),
        quant_weights=dict(us=round(qw_ms * 1e3, 2), gbps=round(w_bytes / qw_ms / 1e6, 1),
                           what="all four weights, 128x128 E4M3, one batched launch"),
        layers=per_layer,
    )
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_8b(layers, M, mode=mode)
    return result


def bench_llama8b_mx(args):
    """The 8B fprop step with microscaling (MXFP8) operands: every step quantizes all four W and,
    per layer, X into 32-element row blocks with E8M0 scale bytes (fp8_quantize_mx) and runs
    fp8_gemm_mx (the scales applied by the scaled MFMA).  Inputs as the default workload."""
    import block_scaled_quantize_amd as bsq
    import synth
    bsq.load()
    M = args.tokens
    dev = torch.device("cuda", 0)
    layers = []
    for name, k, n in LAYERS_8B:
        x = synth.activations_with_outliers(M, k, 0, f"bench/8b/{name}/X").to(dev)
        w = synth.normal((n, k), 0.02, 0, f"bench/8b/{name}/W").to(dev)
        layers.append(dict(
            name=name, K=k, N=n, x=x, w=w,
            qx=torch.empty((M, k), dtype=torch.uint8, device=dev),
            sx=torch.empty(bsq.mx_scale_shape(M, k), dtype=torch.uint8, device=dev),
            qw=torch.empty((n, k), dtype=torch.uint8, device=dev),
            sw=torch.empty(bsq.mx_scale_shape(n, k), dtype=torch.uint8, device=dev),
            y=torch.empty((M, n), dtype=torch.bfloat16, device=dev)))
    torch.cuda.synchronize()
    flops = sum(2.0 * M * L["N"] * L["K"] for L in layers)

    def step(timer=None):
        for L in layers:
            def qw():
                bsq.quantize_mx(L["w"], bsq.E4M3, q=L["qw"], scales=L["sw"])
            def qx():
                bsq.quantize_mx(L["x"], bsq.E4M3, q=L["qx"], scales=L["sx"])
            def mm():
                bsq.gemm_mx(L["qx"], L["sx"], L["qw"], L["sw"], c=L["y"])
            if timer is None:
                qw(); qx(); mm()
            else:
                timer.time(("qw", L["name"]), qw)
                timer.time(("qx", L["name"]), qx)
                timer.time(("gemm", L["name"]), mm)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    timer = EventTimer()
    for _ in range(max(3, min(args.steps, 10))):
        step(timer)
    torch.cuda.synchronize()
    per_layer, gemm_ms, gemm_flops = {}, [], []
    q_bytes, q_ms = 0.0, 0.0
    for L in layers:
        g = timer.mean_ms(("gemm", L["name"]))
        f = 2.0 * M * L["N"] * L["K"]
        gemm_ms.append(g)
        gemm_flops.append(f)
        xb = M * L["K"] * 3 + M * L["K"] / 32
        wb = L["N"] * L["K"] * 3 + L["N"] * L["K"] / 32
        qx_ms, qw_ms = timer.mean_ms(("qx", L["name"])), timer.mean_ms(("qw", L["name"]))
        q_bytes += xb + wb
        q_ms += qx_ms + qw_ms
        per_layer[L["name"]] = dict(gemm_us=round(g * 1e3, 2), gemm_tflops=round(f / g / 1e9, 1),
                                    quant_x_us=round(qx_ms * 1e3, 2), quant_w_us=round(qw_ms * 1e3, 2))
    mean_launch_flops = float(np.mean(gemm_flops))
    achieved = mean_launch_flops / float(np.mean(gemm_ms)) / 1e9
    traffic = measured_traffic(GEMM_COUNTERS_MX, GEMM_SOURCES)
    result = dict(
        metric="microscaling FP8 GEMM TFLOP/s (+quantize GB/s), % of MI355X FP8/HBM peak",
        value=round(flops / dt / 1e12, 2), unit="TFLOP/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=round(dt * 1e3, 4), higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype="fp8e4m3 x fp8e4m3 -> fp32 acc -> bf16",
        data="synthetic",
        config=dict(workload="llama3.1-8b-fprop-linear-mxfp8", tokens=M,
                    layers="qkv 4096->6144, o 4096->4096, gate_up 4096->28672, down 14336->4096",
                    scales="E8M0 bytes, one per 32 K elements of every row of X and W (all four W "
                           "and every X re-quantized each step)", parallelism="single GPU"),
        roofline=dict(bound="mfma", achieved=round(achieved, 1), peak=FP8_PEAK_TFLOPS,
                      unit="TFLOP/s", frac=round(achieved / FP8_PEAK_TFLOPS, 4),
                      traffic=traffic["bytes"], traffic_unit="HBM bytes per launch",
                      traffic_algorithmic=traffic["algorithmic"], traffic_source=traffic["source"],
                      kernel="gemm_persistent_kernel<Cfg<256,256,2,4>,FPROP,E4M3,E4M3,mx>",
                      per_launch_flops=mean_launch_flops,
                      mean_launch_us=round(float(np.mean(gemm_ms)) * 1e3, 2)),
        gemm_only_tflops=round(sum(gemm_flops) / sum(gemm_ms) / 1e9, 1),
        quant_gbps=round(q_bytes / q_ms / 1e6, 1),
        quant_hbm_frac=round(q_bytes / q_ms / 1e6 / HBM_PEAK_GBPS, 4),
        layers=per_layer)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_8b_mx(layers, M)
    return result


def cpu_baseline_8b_mx(layers, M, rows: int = 1024, min_seconds: float = 10.0):
    """The oracle on a bounded sample of the microscaling step: `rows` token rows of each layer's
    activation and the full weights quantized into 32-element blocks, dequantized and multiplied
    in fp64, repeated until min_seconds have passed.  TFLOP/s of the GEMM flops done."""
    import oracle
    oracle.build()
    rows = min(rows, M)
    host = [(L["x"][:rows].cpu().contiguous().view(torch.int16).numpy().view(np.uint16),
             L["w"].cpu().contiguous().view(torch.int16).numpy().view(np.uint16), L) for L in layers]
    t0 = time.perf_counter()
    flops, reps = 0.0, 0
    while reps == 0 or time.perf_counter() - t0 < min_seconds:
        for xs, ws, L in host:
            qx, sx = oracle.quantize_mx(xs, oracle.E4M3)
            qw, sw = oracle.quantize_mx(ws, oracle.E4M3)
            oracle.gemm_mx(qx, oracle.E4M3, sx, qw, oracle.E4M3, sw)
            flops += 2.0 * rows * L["N"] * L["K"]
        reps += 1
    dt = time.perf_counter() - t0
    blas = blas_threads()
    return dict(value=round(flops / dt / 1e12, 5), unit="TFLOP/s", cores=max(cpu_cores(), blas),
                kind="oracle",
                sample=f"{rows} of {M} token rows per layer (all four layers, full weights "
                       f"re-quantized) x {reps} repetitions, {dt:.1f} s; C oracle threads "
                       f"{cpu_cores()}, BLAS threads {blas}")


def cpu_baseline_8b(layers, M, rows: int | None = None, min_seconds: float = 10.0, mode: int = 0):
    """The oracle on the same step (by default all M rows; `rows` bounds the sample): quantize
    the activation rows (1x128) and the full weight (128x128), dequantize and multiply in fp64;
    the step is repeated until min_seconds have passed.  TFLOP/s of the GEMM flops done."""
    import oracle
    oracle.build()
    rows = M if rows is None else min(rows, M)
    host = [(L["x"][:rows].cpu().contiguous().view(torch.int16).numpy().view(np.uint16),
             L["w"].cpu().contiguous().view(torch.int16).numpy().view(np.uint16), L) for L in layers]
    t0 = time.perf_counter()
    flops, reps = 0.0, 0
    while reps == 0 or time.perf_counter() - t0 < min_seconds:
        for xs, ws, L in host:
            qx, sx = oracle.quantize_blockwise(xs, oracle.E4M3, oracle.BLOCK_1x128, mode)
            qw, sw = oracle.quantize_blockwise(ws, oracle.E4M3, oracle.BLOCK_128x128, mode)
            oracle.gemm(oracle.FPROP, qx, oracle.E4M3, oracle.BLOCK_1x128, sx, qw, oracle.E4M3,
                        oracle.BLOCK_128x128, sw)
            flops += 2.0 * rows * L["N"] * L["K"]
        reps += 1
    dt = time.perf_counter() - t0
    blas = blas_threads()
    return dict(value=round(flops / dt / 1e12, 5), unit="TFLOP/s", cores=max(cpu_cores(), blas),
                kind="oracle",
                sample=f"{rows} of {M} token rows per layer (all four layers, full weights "
                       f"re-quantized) x {reps} repetitions, {dt:.1f} s; C oracle threads "
                       f"{cpu_cores()}, BLAS threads {blas}")


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:  # pragma: no cover - optional dependency
        return 1


# ----------------------------------------------------------------------------- quantizer sweep

SWEEP_SHAPES = [(4096, 4096), (32768, 4096), (131072, 4096), (1152, 14336), (9344, 14336),
                (37504, 14336)]


def bench_quant_sweep(args):
    """HBM-bound quantizer on Student-t(3) bf16 tensors of 16M / 128M / 512M elements (rows of
    4096 or 14336), 1x128 and 128x128 E4M3, fp32 and power-of-2 scales.  Buffers rotate over
    more than 512 MiB so that the 256 MiB last-level cache does not serve the inputs."""
    import block_scaled_quantize_amd as bsq
    import synth
    bsq.load()
    dev = torch.device("cuda", 0)
    cases = {}
    for rows, cols in SWEEP_SHAPES:
        n = rows * cols
        nbuf = max(1, -(-(600 << 20) // (3 * n)))
        log(f"sweep {rows}x{cols}: {nbuf} rotating buffers")
        base = synth.student_t((rows, cols), 3.0, 0, f"bench/sweep/{rows}x{cols}").to(dev)
        xs = [base] + [base.roll(i, 0) for i in range(1, nbuf)]
        for gran in (bsq.BLOCK_1x128, bsq.BLOCK_128x128):
            qs = [torch.empty((rows, cols), dtype=torch.uint8, device=dev) for _ in range(nbuf)]
            ss = [torch.empty(bsq.scale_shape(rows, cols, gran), dtype=torch.float32, device=dev)
                  for _ in range(nbuf)]
            for mode in (bsq.SCALE_FP32, bsq.SCALE_POW2):
                def run(i):
                    bsq.quantize_blockwise(xs[i % nbuf], bsq.E4M3, gran, mode, q=qs[i % nbuf],
                                           scale_inv=ss[i % nbuf])
                for i in range(args.warmup):
                    run(i)
                torch.cuda.synchronize()
                iters = max(args.steps, 10)
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(iters)]
                for i in range(iters):
                    ev[i][0].record()
                    run(i)
                    ev[i][1].record()
                torch.cuda.synchronize()
                ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
                nb = ss[0].numel() * 4
                byts = 3.0 * n + nb
                key = f"{rows}x{cols}/{'1x128' if gran == 0 else '128x128'}/{'fp32' if mode == 0 else 'pow2'}"
                cases[key] = dict(us=round(ms * 1e3, 2), gbps=round(byts / ms / 1e6, 1),
                                  hbm_frac=round(byts / ms / 1e6 / HBM_PEAK_GBPS, 4), bytes=byts)
                log(f"  {key}: {ms * 1e3:.1f} us, {byts / ms / 1e6:.0f} GB/s")
            del qs, ss
        del xs, base
        torch.cuda.empty_cache()
    head = cases["131072x4096/1x128/fp32"]
    traffic = measured_traffic(QUANT_COUNTERS, QUANT_SOURCES)
    res = dict(metric="quantize GB/s (bf16 -> E4M3 codes + scales), % of MI355X HBM peak",
               value=head["gbps"], unit="GB/s", n_gpus=1, steps=max(args.steps, 10),
               warmup=args.warmup, ms_per_step=head["us"] / 1e3, higher_is_better=True,
               scaling="weak", vs_baseline=None, dtype="bf16 -> u8 (E4M3) + fp32 scales",
               data="synthetic",
               config=dict(workload="quantizer-sweep", headline="131072x4096 1x128 fp32-scale",
                           distribution="Student-t(3)"),
               roofline=dict(bound="hbm", achieved=head["gbps"], peak=HBM_PEAK_GBPS, unit="GB/s",
                             frac=head["hbm_frac"], traffic=traffic["bytes"],
                             traffic_unit="HBM bytes per launch",
                             traffic_algorithmic=traffic["algorithmic"],
                             traffic_source=traffic["source"],
                             kernel="quant_1x128_rows_kernel<E4M3,fp32,non-temporal stores>",
                             per_launch_bytes=head["bytes"], mean_launch_us=head["us"]),
               cases=cases)
    if not args.no_cpu_baseline:
        import oracle
        oracle.build()
        x = synth.student_t((4096, 4096), 3.0, 0, "bench/sweep/4096x4096")
        xb = x.contiguous().view(torch.int16).numpy().view(np.uint16)
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 10.0:
            oracle.quantize_blockwise(xb, oracle.E4M3, oracle.BLOCK_1x128, oracle.SCALE_FP32)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        res["cpu_baseline"] = dict(value=round((3.0 * xb.size + 4 * xb.size / 128) / dt / 1e9, 3),
                                   unit="GB/s", cores=cpu_cores(), kind="oracle",
                                   sample=f"4096x4096 1x128 fp32, {reps} repetitions in {dt * reps:.1f} s")
    return res


# ----------------------------------------------------------------------------- streaming ceiling

STREAM_VARIANTS = {0: "one-shot, 16 el/lane", 1: "one-shot, 2x16 el/lane", 2: "one-shot, 4x16 el/lane",
                   3: "2048 workgroups striding", 4: "4096 workgroups striding",
                   5: "one-shot, non-temporal loads", 6: "one-shot, non-temporal stores",
                   7: "one-shot, non-temporal loads and stores",
                   8: "32-row x 128-column tiles (the short-row quantizer's geometry)"}


def bench_stream(args):
    """The rate this GPU streams the quantizers' traffic at: plain kernels that read 2 bytes and
    write 1 byte per element (libfp8bs_bench.so: grid shapes, non-temporal accesses, the
    short-row quantizer's tile geometry), next to the 1x128 quantizer
    on the same buffers (bf16 [rows, 4096] of 16M / 128M / 512M elements, rotating over more
    than 512 MiB so that the last-level cache does not serve the inputs).  value = the best
    streaming rate on the 512M-element tensor; quantizer_vs_stream = the quantizer's rate over
    that ceiling."""
    import ctypes
    import block_scaled_quantize_amd as bsq
    import synth
    bsq.load()
    blib = ctypes.CDLL(os.path.join(ROOT, "block_scaled_quantize_amd", "libfp8bs_bench.so"))
    blib.fp8bs_bench_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_void_p]
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream().cuda_stream
    cases = {}
    iters = max(args.steps, 10)

    def timed(run):
        for i in range(args.warmup):
            run(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters)]
        for i in range(iters):
            ev[i][0].record()
            run(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev]))

    for rows in (4096, 32768, 131072):
        cols = 4096
        n = rows * cols
        nbuf = max(1, -(-(600 << 20) // (3 * n)))
        base = synth.student_t((rows, cols), 3.0, 0, f"bench/sweep/{rows}x{cols}").to(dev)
        xs = [base] + [base.roll(i, 0) for i in range(1, nbuf)]
        ys = [torch.empty((rows, cols), dtype=torch.uint8, device=dev) for _ in range(nbuf)]
        ss = [torch.empty(bsq.scale_shape(rows, cols, bsq.BLOCK_1x128), dtype=torch.float32,
                          device=dev) for _ in range(nbuf)]
        entry = {}
        for v, what in STREAM_VARIANTS.items():
            def run(i, v=v):
                rc = blib.fp8bs_bench_stream(xs[i % nbuf].data_ptr(), n, ys[i % nbuf].data_ptr(), v,
                                             stream)
                assert rc == 0
            ms = timed(run)
            entry[what] = round(3.0 * n / ms / 1e6, 1)
        qbytes = 3.0 * n + 4.0 * n / 128
        qms = timed(lambda i: bsq.quantize_blockwise(xs[i % nbuf], bsq.E4M3, bsq.BLOCK_1x128,
                                                     q=ys[i % nbuf], scale_inv=ss[i % nbuf]))
        best = max(entry.values())
        cases[f"{rows}x{cols}"] = dict(stream_gbps=entry, best_stream_gbps=best,
                                       quant_1x128_gbps=round(qbytes / qms / 1e6, 1),
                                       quant_vs_stream=round(qbytes / qms / 1e6 / best, 4))
        log(f"stream {rows}x{cols}: {entry}; quantizer {qbytes / qms / 1e6:.0f} GB/s")
        del xs, ys, ss, base
        torch.cuda.empty_cache()
    head = cases["131072x4096"]
    return dict(metric="streaming GB/s at the quantizers' traffic (2 B read + 1 B written per "
                       "element), % of MI355X HBM peak",
                value=head["best_stream_gbps"], unit="GB/s", n_gpus=1, steps=iters,
                warmup=args.warmup, ms_per_step=None, higher_is_better=True, scaling="weak",
                vs_baseline=None, dtype="bf16 -> u8", data="synthetic",
                config=dict(workload="stream-ceiling", headline="131072x4096 (512M elements)"),
                roofline=dict(bound="hbm", achieved=head["best_stream_gbps"], peak=HBM_PEAK_GBPS,
                              unit="GB/s", frac=round(head["best_stream_gbps"] / HBM_PEAK_GBPS, 4),
                              traffic=None, kernel="stream kernels (libfp8bs_bench.so)"),
                quantizer_vs_stream=head["quant_vs_stream"], cases=cases)


# ----------------------------------------------------------------------------- MoE grouped

def bench_moe(args):
    """Grouped FP8 GEMM of a Qwen3-30B-A3B-shaped MoE layer: 128 experts, 16384 tokens routed
    top-8 with Zipf(1.1) popularity (131072 rows sorted by expert); gate/up 2048 -> 1536 and
    down 768 -> 2048 per expert, 1x128 activation / 128x128 weight E4M3 scales, bf16 out.
    --pow2: power-of-2 scales applied by the MFMA; --mx: microscaling (32-element blocks with
    E8M0 bytes on the activations and every expert's weights, fp8_grouped_gemm_mx)."""
    import block_scaled_quantize_amd as bsq
    import synth
    bsq.load()
    dev = torch.device("cuda", 0)
    mx = getattr(args, "mx", False)
    counts = synth.moe_routing(16384, 128, 8, 1.1, 0)
    off = torch.from_numpy(synth.offsets_from_counts(counts)).to(dev)
    T = int(counts.sum())
    out = {}
    total_flops, total_ms = 0.0, 0.0
    for name, K, N in (("gate_up", 2048, 1536), ("down", 768, 2048)):
        x = synth.normal((T, K), 1.0, 0, f"bench/moe/{name}/X").to(dev)
        mode = bsq.SCALE_POW2 if args.pow2 else bsq.SCALE_FP32
        if mx:
            qx, sx = bsq.quantize_mx(x, bsq.E4M3)
        else:
            qx, sx = bsq.quantize_blockwise(x, bsq.E4M3, bsq.BLOCK_1x128, mode)
        del x
        qw = torch.empty((128, N, K), dtype=torch.uint8, device=dev)
        if mx:
            sw = torch.empty((128,) + bsq.mx_scale_shape(N, K), dtype=torch.uint8, device=dev)
        else:
            sw = torch.empty((128, N // 128, K // 128), dtype=torch.float32, device=dev)
        for e in range(128):
            w = synth.normal((N, K), 0.02, 0, f"bench/moe/{name}/W{e}").to(dev)
            if mx:
                bsq.quantize_mx(w, bsq.E4M3, q=qw[e], scales=sw[e])
            else:
                bsq.quantize_blockwise(w, bsq.E4M3, bsq.BLOCK_128x128, mode, q=qw[e], scale_inv=sw[e])
        c = torch.empty((T, N), dtype=torch.bfloat16, device=dev)

        def run():
            if mx:
                bsq.grouped_gemm_mx(off, qx, sx, qw, sw, c=c)
            else:
                bsq.grouped_gemm(off, qx, sx, qw, sw, c=c, pow2=args.pow2)
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        iters = max(args.steps, 5)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        for a, b in ev:
            a.record()
            run()
            b.record()
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        flops = 2.0 * T * N * K
        if mx:
            byts = T * K + 128 * N * K + 2 * T * N + T * K / 32 + 128 * N * K / 32
        else:
            byts = T * K + 128 * N * K + 2 * T * N + 4 * T * K / 128 + 4 * 128 * (N // 128) * (K // 128)
        t_mfma = flops / (FP8_PEAK_TFLOPS * 1e12)
        t_hbm = byts / (HBM_PEAK_GBPS * 1e9)
        bound = "mfma" if t_mfma >= t_hbm else "hbm"
        out[name] = dict(us=round(ms * 1e3, 1), tflops=round(flops / ms / 1e9, 1), gbps=round(byts / ms / 1e6, 1),
                         bound=bound, frac_of_binding_roofline=round(max(t_mfma, t_hbm) / (ms / 1e3), 4))
        total_flops += flops
        total_ms += ms
        log(f"moe {name}: {ms * 1e3:.1f} us {flops / ms / 1e9:.0f} TFLOP/s ({bound}-bound)")
        del qx, sx, qw, sw, c
        torch.cuda.empty_cache()
    gu = out["gate_up"]
    return dict(metric="grouped block-scaled FP8 GEMM TFLOP/s (MoE experts)",
                value=round(total_flops / total_ms / 1e9, 1), unit="TFLOP/s", n_gpus=1,
                steps=max(args.steps, 5), warmup=args.warmup, ms_per_step=round(total_ms, 4),
                higher_is_better=True, scaling="weak", vs_baseline=None,
                dtype="fp8e4m3 x fp8e4m3 -> fp32 acc -> bf16", data="synthetic",
                config=dict(workload="qwen3-30b-a3b-moe-experts" + ("-mxfp8" if mx else "-pow2" if args.pow2 else ""),
                            experts=128, tokens=16384, topk=8,
                            routing="Zipf(1.1)", rows=T),
                roofline=dict(bound=gu["bound"], achieved=gu["tflops"], peak=FP8_PEAK_TFLOPS,
                              unit="TFLOP/s", frac=round(gu["tflops"] / FP8_PEAK_TFLOPS, 4),
                              traffic=None,
                              kernel="grouped_gemm_kernel<Cfg<256,256,2,4>,E4M3,E4M3,%s>"
                                     % ("mx" if mx else "hw" if args.pow2 else "fold")),
                layers=out)


# ----------------------------------------------------------------------------- backward

def bench_backward(args):
    """8B-shaped backward linear layers with per-tensor delayed scaling (history 16, max,
    margin 0): X and W in E4M3, dY ~ N(0, 1e-3) in E5M2; per layer one delayed quantization of
    each tensor, dgrad dX = dY . W and wgrad dW = dY^T . X.  Steps draw fresh X and dY."""
    import block_scaled_quantize_amd as bsq
    import synth
    bsq.load()
    dev = torch.device("cuda", 0)
    M = args.tokens
    layers = []
    for name, k, n in LAYERS_8B:
        L = dict(name=name, K=k, N=n,
                 x=synth.activations_with_outliers(M, k, 0, f"bench/bwd/{name}/X").to(dev),
                 w=synth.normal((n, k), 0.02, 0, f"bench/bwd/{name}/W").to(dev),
                 dy=synth.normal((M, n), 1e-3, 0, f"bench/bwd/{name}/dY").to(dev),
                 sx=bsq.DelayedState(16), sw=bsq.DelayedState(16), sdy=bsq.DelayedState(16),
                 dx=torch.empty((M, k), dtype=torch.bfloat16, device=dev),
                 dw=torch.empty((n, k), dtype=torch.bfloat16, device=dev))
        layers.append(L)
    flops = sum(4.0 * M * L["N"] * L["K"] for L in layers)

    def step(t=None):
        def run(key, fn):
            return fn() if t is None else t.time(key, fn)
        for L in layers:
            n = L["name"]
            qx, six = run(n + "/qx", lambda: bsq.quantize_delayed(L["x"], bsq.E4M3, L["sx"]))
            qw, siw = run(n + "/qw", lambda: bsq.quantize_delayed(L["w"], bsq.E4M3, L["sw"]))
            qdy, sidy = run(n + "/qdy", lambda: bsq.quantize_delayed(L["dy"], bsq.E5M2, L["sdy"]))
            run(n + "/dgrad", lambda: bsq.gemm_blockscaled(
                bsq.DGRAD, qdy, bsq.E5M2, bsq.PER_TENSOR, sidy, qw, bsq.E4M3, bsq.PER_TENSOR,
                siw, c=L["dx"]))
            run(n + "/wgrad", lambda: bsq.gemm_blockscaled(
                bsq.WGRAD, qdy, bsq.E5M2, bsq.PER_TENSOR, sidy, qx, bsq.E4M3, bsq.PER_TENSOR,
                six, c=L["dw"]))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    # every launch with HIP events on its stream: the GEMMs (per-tensor scales on both operands)
    # and the delayed quantizer (cast + finalize of one tensor per event pair)
    timer = EventTimer()
    for _ in range(max(3, min(args.steps, 10))):
        step(timer)
    torch.cuda.synchronize()
    per_layer, gemm_ms, q_ms, q_bytes = {}, 0.0, 0.0, 0.0
    for L in layers:
        n, f1 = L["name"], 2.0 * M * L["N"] * L["K"]
        dg, wg = timer.mean_ms(n + "/dgrad"), timer.mean_ms(n + "/wgrad")
        gemm_ms += dg + wg
        quant = {}
        for key, numel in (("qx", M * L["K"]), ("qw", L["N"] * L["K"]), ("qdy", M * L["N"])):
            ms = timer.mean_ms(n + "/" + key)
            nbytes = 3.0 * numel          # 2 B read + 1 B written per element (state: 68 B)
            q_ms += ms
            q_bytes += nbytes
            quant[key + "_us"] = round(ms * 1e3, 2)
            quant[key + "_gbps"] = round(nbytes / ms / 1e6, 1)
        per_layer[n] = dict(dgrad_us=round(dg * 1e3, 2), dgrad_tflops=round(f1 / dg / 1e9, 1),
                            wgrad_us=round(wg * 1e3, 2), wgrad_tflops=round(f1 / wg / 1e9, 1),
                            **quant)
    achieved = flops / gemm_ms / 1e9
    return dict(metric="block-scaled FP8 GEMM TFLOP/s, backward (dgrad + wgrad, delayed scaling)",
                value=round(flops / dt / 1e12, 2), unit="TFLOP/s", n_gpus=1, steps=args.steps,
                warmup=args.warmup, ms_per_step=round(dt * 1e3, 4), higher_is_better=True,
                scaling="weak", vs_baseline=None, dtype="fp8e5m2 x fp8e4m3 -> fp32 acc -> bf16",
                data="synthetic",
                config=dict(workload="llama3.1-8b-backward-linear", tokens=M,
                            scaling="per-tensor delayed, history 16, max, margin 0"),
                roofline=dict(bound="mfma", achieved=round(achieved, 1), peak=FP8_PEAK_TFLOPS,
                              unit="TFLOP/s", frac=round(achieved / FP8_PEAK_TFLOPS, 4),
                              traffic=None,
                              kernel="gemm_persistent_kernel<Cfg<256,256,2,4>,DGRAD|WGRAD,E5M2,E4M3,tensor>",
                              mean_launch_us=round(gemm_ms / (2 * len(layers)) * 1e3, 2)),
                delayed_quant=dict(bound="hbm", achieved_gbps=round(q_bytes / q_ms / 1e6, 1),
                                   peak_gbps=HBM_PEAK_GBPS,
                                   frac=round(q_bytes / q_ms / 1e6 / HBM_PEAK_GBPS, 4),
                                   us_per_step=round(q_ms * 1e3, 1),
                                   what="delayed_cast_kernel + delayed_finalize_kernel per tensor "
                                        "(X, W E4M3; dY E5M2), 3 B per element"),
                layers=per_layer)


def bench_backward_blockwise(args):
    """8B-shaped backward linear layers in the block recipe ("NVIDIA NeMo RL ...", section "El
    avance técnico"; E4M3 gradients).  Per layer and step: dY quantized 1x128 along out-features
    (dgrad operand) and columnwise over tokens (wgrad operand, transposed) in one pass
    (fp8_quantize_1x128_and_columnwise_t), X quantized columnwise over tokens (transposed), W
    re-quantized 128x128; dgrad dX = dY . W (128x128 weight tiles), wgrad dW = dY^T . X (1x128
    scales on both operands).  --pow2: power-of-2 scales everywhere."""
    import block_scaled_quantize_amd as bsq
    import synth
    bsq.load()
    dev = torch.device("cuda", 0)
    M = args.tokens
    mode = bsq.SCALE_POW2 if args.pow2 else bsq.SCALE_FP32
    E4, B1, B128 = bsq.E4M3, bsq.BLOCK_1x128, bsq.BLOCK_128x128
    layers = []
    for name, k, n in LAYERS_8B:
        layers.append(dict(
            name=name, K=k, N=n,
            x=synth.activations_with_outliers(M, k, 0, f"bench/bwdb/{name}/X").to(dev),
            w=synth.normal((n, k), 0.02, 0, f"bench/bwdb/{name}/W").to(dev),
            dy=synth.normal((M, n), 1e-3, 0, f"bench/bwdb/{name}/dY").to(dev),
            dx=torch.empty((M, k), dtype=torch.bfloat16, device=dev),
            dw=torch.empty((n, k), dtype=torch.bfloat16, device=dev)))
    torch.cuda.synchronize()
    flops = sum(4.0 * M * L["N"] * L["K"] for L in layers)
    timer = EventTimer()

    def step(t=None):
        def run(key, fn):
            return fn() if t is None else t.time((key, L["name"]), fn)
        for L in layers:
            qdy, sdy, dyt, sdyt = run("q_dy", lambda: bsq.quantize_1x128_and_columnwise_t(
                L["dy"], E4, mode))
            qw, sw = run("q_w", lambda: bsq.quantize_blockwise(L["w"], E4, B128, mode))
            xt, sxt = run("q_xT", lambda: bsq.quantize_columnwise_t(L["x"], E4, mode))
            run("dgrad", lambda: bsq.gemm_blockscaled(bsq.DGRAD, qdy, E4, B1, sdy, qw, E4, B128, sw,
                                                      c=L["dx"], pow2=args.pow2))
            run("wgrad", lambda: bsq.gemm_blockscaled(bsq.FPROP, dyt, E4, B1, sdyt, xt, E4, B1, sxt,
                                                      c=L["dw"], pow2=args.pow2))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    for _ in range(max(3, min(args.steps, 10))):
        step(timer)
    torch.cuda.synchronize()
    per = {}
    for L in layers:
        f = 2.0 * M * L["N"] * L["K"]
        d = {}
        for key in ("dgrad", "wgrad"):
            ms = timer.mean_ms((key, L["name"]))
            d[f"{key}_us"] = round(ms * 1e3, 2)
            d[f"{key}_tflops"] = round(f / ms / 1e9, 1)
        # dY: 2 B read, 1 B of row codes and 1 B of transposed codes per element
        for key, byts in (("q_dy", 4.0 * M * L["N"]), ("q_xT", 3.0 * M * L["K"])):
            ms = timer.mean_ms((key, L["name"]))
            d[f"{key}_us"] = round(ms * 1e3, 2)
            d[f"{key}_gbps"] = round(byts / ms / 1e6, 1)
        per[L["name"]] = d
    wg_ms = [timer.mean_ms(("wgrad", L["name"])) for L in layers]
    wg_f = [2.0 * M * L["N"] * L["K"] for L in layers]
    achieved = float(np.mean(wg_f)) / float(np.mean(wg_ms)) / 1e9
    return dict(metric="block-scaled FP8 GEMM TFLOP/s, backward (dgrad + blockwise wgrad)",
                value=round(flops / dt / 1e12, 2), unit="TFLOP/s", n_gpus=1, steps=args.steps,
                warmup=args.warmup, ms_per_step=round(dt * 1e3, 4), higher_is_better=True,
                scaling="weak", vs_baseline=None, dtype="fp8e4m3 x fp8e4m3 -> fp32 acc -> bf16",
                data="synthetic",
                config=dict(workload="llama3.1-8b-backward-blockwise" + ("-pow2" if args.pow2 else ""),
                            tokens=M, scaling="dY 1x128 (dgrad) and dY^T columnwise 128x1 (wgrad) "
                            "in one pass, X^T columnwise 128x1 (wgrad), W 128x128"),
                roofline=dict(bound="mfma", achieved=round(achieved, 1), peak=FP8_PEAK_TFLOPS,
                              unit="TFLOP/s", frac=round(achieved / FP8_PEAK_TFLOPS, 4),
                              traffic=None,
                              kernel="gemm_persistent_kernel<Cfg<256,256,2,4>,FPROP,E4M3,E4M3,%s> (wgrad)"
                                     % ("hw-rows" if args.pow2 else "fold-rows"),
                              mean_launch_us=round(float(np.mean(wg_ms)) * 1e3, 2)),
                layers=per)


def bench_backward_mx(args):
    """8B-shaped backward linear layers in microscaling form (32-element blocks with E8M0 scale
    bytes).  Per layer and step: dY quantized along out-features (the dgrad A operand) and along
    tokens with transposed codes (wgrad A) in one pass (fp8_quantize_mx_and_columnwise_t), X
    along tokens transposed (wgrad B), W along out-features transposed (dgrad B); dgrad
    dX = dY . W and wgrad dW = dY^T . X, both by fp8_gemm_mx.  Inputs as backward-blockwise."""
    import block_scaled_quantize_amd as bsq
    import synth
    bsq.load()
    dev = torch.device("cuda", 0)
    M = args.tokens
    E4 = bsq.E4M3
    layers = []
    for name, k, n in LAYERS_8B:
        layers.append(dict(
            name=name, K=k, N=n,
            x=synth.activations_with_outliers(M, k, 0, f"bench/bwdb/{name}/X").to(dev),
            w=synth.normal((n, k), 0.02, 0, f"bench/bwdb/{name}/W").to(dev),
            dy=synth.normal((M, n), 1e-3, 0, f"bench/bwdb/{name}/dY").to(dev),
            dx=torch.empty((M, k), dtype=torch.bfloat16, device=dev),
            dw=torch.empty((n, k), dtype=torch.bfloat16, device=dev)))
    torch.cuda.synchronize()
    flops = sum(4.0 * M * L["N"] * L["K"] for L in layers)
    timer = EventTimer()

    def step(t=None):
        def run(key, fn):
            return fn() if t is None else t.time((key, L["name"]), fn)
        for L in layers:
            qdy, sdy, dyt, sdyt = run("q_dy", lambda: bsq.quantize_mx_and_columnwise_t(L["dy"], E4))
            qwt, swt = run("q_wT", lambda: bsq.quantize_mx_columnwise_t(L["w"], E4))
            xt, sxt = run("q_xT", lambda: bsq.quantize_mx_columnwise_t(L["x"], E4))
            run("dgrad", lambda: bsq.gemm_mx(qdy, sdy, qwt, swt, c=L["dx"]))
            run("wgrad", lambda: bsq.gemm_mx(dyt, sdyt, xt, sxt, c=L["dw"]))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    for _ in range(max(3, min(args.steps, 10))):
        step(timer)
    torch.cuda.synchronize()
    per, g_ms, g_f = {}, [], []
    q_bytes, q_ms = 0.0, 0.0
    for L in layers:
        f = 2.0 * M * L["N"] * L["K"]
        d = {}
        for key in ("dgrad", "wgrad"):
            ms = timer.mean_ms((key, L["name"]))
            d[f"{key}_us"] = round(ms * 1e3, 2)
            d[f"{key}_tflops"] = round(f / ms / 1e9, 1)
            g_ms.append(ms)
            g_f.append(f)
        # dY: 2 B read, 1 B of row codes, 1 B of transposed codes (and two scale bytes per 32)
        for key, n_el, per_el in (("q_dy", M * L["N"], 4.0 + 2 / 32), ("q_wT", L["N"] * L["K"], 3.0 + 1 / 32),
                                  ("q_xT", M * L["K"], 3.0 + 1 / 32)):
            ms = timer.mean_ms((key, L["name"]))
            byts = per_el * n_el
            d[f"{key}_us"] = round(ms * 1e3, 2)
            d[f"{key}_gbps"] = round(byts / ms / 1e6, 1)
            q_bytes += byts
            q_ms += ms
        per[L["name"]] = d
    achieved = float(np.mean(g_f)) / float(np.mean(g_ms)) / 1e9
    return dict(metric="microscaling FP8 GEMM TFLOP/s, backward (dgrad + wgrad)",
                value=round(flops / dt / 1e12, 2), unit="TFLOP/s", n_gpus=1, steps=args.steps,
                warmup=args.warmup, ms_per_step=round(dt * 1e3, 4), higher_is_better=True,
                scaling="weak", vs_baseline=None, dtype="fp8e4m3 x fp8e4m3 -> fp32 acc -> bf16",
                data="synthetic",
                config=dict(workload="llama3.1-8b-backward-mxfp8", tokens=M,
                            scaling="32-element blocks, E8M0 bytes: dY along out-features "
                            "(dgrad), dY^T, X^T along tokens (wgrad), W^T along out-features"),
                roofline=dict(bound="mfma", achieved=round(achieved, 1), peak=FP8_PEAK_TFLOPS,
                              unit="TFLOP/s", frac=round(achieved / FP8_PEAK_TFLOPS, 4),
                              traffic=None,
                              kernel="gemm_persistent_kernel<Cfg<256,256,2,4>,FPROP,E4M3,E4M3,mx> "
                                     "(dgrad and wgrad launches)",
                              mean_launch_us=round(float(np.mean(g_ms)) * 1e3, 2)),
                quant_gbps=round(q_bytes / q_ms / 1e6, 1),
                quant_hbm_frac=round(q_bytes / q_ms / 1e6 / HBM_PEAK_GBPS, 4),
                layers=per)


def bench_fprop_qout(args):
    """The 8B fprop layers with the output quantized in the GEMM epilogue (the next layer's 1x128
    E4M3 operand), against the same GEMM followed by the separate quantizer.  Per layer and step:
    the fused call writes bf16 + codes + scales; timed per launch with HIP events.  value = GEMM
    flops / time of the fused launches."""
    import block_scaled_quantize_amd as bsq
    import synth
    bsq.load()
    dev = torch.device("cuda", 0)
    M = args.tokens
    E4, B1, B128 = bsq.E4M3, bsq.BLOCK_1x128, bsq.BLOCK_128x128
    layers = []
    for name, k, n in LAYERS_8B:
        x = synth.activations_with_outliers(M, k, 0, f"bench/8b/{name}/X").to(dev)
        w = synth.normal((n, k), 0.02, 0, f"bench/8b/{name}/W").to(dev)
        qx, sx = bsq.quantize_blockwise(x, E4, B1)
        qw, sw = bsq.quantize_blockwise(w, E4, B128)
        layers.append(dict(name=name, K=k, N=n, qx=qx, sx=sx, qw=qw, sw=sw,
                           y=torch.empty((M, n), dtype=torch.bfloat16, device=dev),
                           yq=torch.empty((M, n), dtype=torch.uint8, device=dev),
                           ys=torch.empty((n // 128, M), dtype=torch.float32, device=dev)))
        del x, w
    torch.cuda.synchronize()
    timer = EventTimer()

    def fused(L, bf16=True):
        bsq.gemm_blockscaled_qout(L["qx"], B1, L["sx"], L["qw"], B128, L["sw"], want_bf16=bf16,
                                  c=L["y"] if bf16 else None, cq=L["yq"], cqs=L["ys"])

    def separate(L):
        bsq.gemm_blockscaled(bsq.FPROP, L["qx"], E4, B1, L["sx"], L["qw"], E4, B128, L["sw"], c=L["y"])
        bsq.quantize_blockwise(L["y"], E4, B1, q=L["yq"], scale_inv=L["ys"])

    for _ in range(args.warmup):
        for L in layers:
            fused(L)
            separate(L)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        for L in layers:
            timer.time(("fused", L["name"]), lambda: fused(L))
            timer.time(("codes_only", L["name"]), lambda: fused(L, False))
            timer.time(("separate", L["name"]), lambda: separate(L))
    torch.cuda.synchronize()
    per, tot_f, tot_ms = {}, 0.0, 0.0
    for L in layers:
        f = 2.0 * M * L["N"] * L["K"]
        d = {k + "_us": round(timer.mean_ms((k, L["name"])) * 1e3, 2)
             for k in ("fused", "codes_only", "separate")}
        d["fused_tflops"] = round(f / timer.mean_ms(("fused", L["name"])) / 1e9, 1)
        per[L["name"]] = d
        tot_f += f
        tot_ms += timer.mean_ms(("fused", L["name"]))
    sep_ms = sum(timer.mean_ms(("separate", L["name"])) for L in layers)
    return dict(metric="block-scaled FP8 GEMM TFLOP/s with the output quantized in the epilogue",
                value=round(tot_f / tot_ms / 1e9, 1), unit="TFLOP/s", n_gpus=1, steps=args.steps,
                warmup=args.warmup, ms_per_step=round(tot_ms, 4), higher_is_better=True,
                scaling="weak", vs_baseline=None, dtype="fp8e4m3 x fp8e4m3 -> fp32 acc -> bf16 + e4m3",
                data="synthetic",
                config=dict(workload="llama3.1-8b-fprop-qout", tokens=M,
                            output="bf16 + E4M3 codes + 1x128 scales (fused) vs GEMM then quantizer"),
                roofline=dict(bound="mfma", achieved=round(tot_f / tot_ms / 1e9, 1),
                              peak=FP8_PEAK_TFLOPS, unit="TFLOP/s",
                              frac=round(tot_f / tot_ms / 1e9 / FP8_PEAK_TFLOPS, 4), traffic=None,
                              kernel="gemm_kernel<Cfg<256,256,2,4>,FPROP,E4M3,E4M3,fold,qout>"),
                speedup_vs_separate=round(sep_ms / tot_ms, 4), layers=per)


def bench_kv_decode(args):
    """One decode step over an FP8 KV cache ("NVIDIA NeMo RL ...", section "Ganancias de
    rendimiento en el mundo real": FP8 KV cache and attention), Llama-3.1-8B attention shape
    (32 query heads, 8 KV heads, head dim 128), 64 sequences with a 4096-token cache and seeded
    lengths in [2048, 4096] (--kv-batch: another batch; --kv-split: chunked decode).  Per step: the
    step's new token of every sequence is quantized into
    the cache (1x128 per head vector) and grouped-query attention reads the whole cache.
    value = algorithmic bytes of the step / step time."""
    import block_scaled_quantize_amd as bsq
    bsq.load()
    dev = torch.device("cuda", 0)
    B, T, H, KVH, D = args.kv_batch, 4096, 32, 8, 128
    g = np.random.default_rng(11)
    lens_np = g.integers(T // 2, T + 1, size=B).astype(np.int32)
    lens = torch.from_numpy(lens_np).to(dev)
    pos = (lens - 1).to(torch.int32)
    gen = torch.Generator(device=dev).manual_seed(11)
    kc = torch.empty((B, T, KVH, D), dtype=torch.uint8, device=dev)
    vc = torch.empty_like(kc)
    ks = torch.empty((B, T, KVH), dtype=torch.float32, device=dev)
    vs = torch.empty_like(ks)
    for b in range(B):   # fill the cache: synthetic N(0, 1) keys and values, 1x128 quantized
        for codes, fac in ((kc, ks), (vc, vs)):
            x = torch.randn((T * KVH, D), generator=gen, device=dev).to(torch.bfloat16)
            bsq.quantize_blockwise(x, bsq.E4M3, bsq.BLOCK_1x128, bsq.SCALE_FP32,
                                   q=codes[b].view(T * KVH, D), scale_inv=fac[b].view(1, T * KVH))
    q = torch.randn((B, H, D), generator=gen, device=dev).to(torch.bfloat16)
    kn = torch.randn((B, KVH, D), generator=gen, device=dev).to(torch.bfloat16)
    vn = torch.randn((B, KVH, D), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    sm = 1.0 / float(np.sqrt(D))
    split = (bsq.decode_split_tokens(B, KVH, T) if args.kv_split < 0
             else (args.kv_split if args.kv_split > 0 else None))
    ws = None
    if split:
        ws = torch.empty((bsq.attention_decode_workspace_size(B, H, KVH, T, split),),
                         dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(t=None):
        def run(key, fn):
            return fn() if t is None else t.time(key, fn)
        run("append", lambda: bsq.kv_cache_append(kn, vn, pos, kc, ks, vc, vs))
        run("decode", lambda: bsq.attention_decode(q, kc, ks, vc, vs, lens, sm, out=out,
                                                   split_tokens=split, workspace=ws))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    timer = EventTimer()
    for _ in range(max(3, min(args.steps, 20))):
        step(timer)
    torch.cuda.synchronize()
    tokens = int(lens_np.sum())
    decode_bytes = tokens * KVH * (2 * D + 8) + 2 * (2 * B * H * D) + 4 * B
    append_bytes = B * KVH * 2 * (2 * D + D + 4) + 4 * B
    dec_ms = timer.mean_ms("decode")
    app_ms = timer.mean_ms("append")
    achieved = decode_bytes / dec_ms / 1e6
    res = dict(metric="FP8 KV-cache decode step GB/s (cache write + grouped-query attention)",
               value=round((decode_bytes + append_bytes) / dt / 1e9, 1), unit="GB/s", n_gpus=1,
               steps=args.steps, warmup=args.warmup, ms_per_step=round(dt * 1e3, 4),
               higher_is_better=True, scaling="weak", vs_baseline=None,
               dtype="e4m3 cache; bf16 MFMA products (keys and values decoded exactly, weights as bf16 hi + lo), fp32 accumulate and softmax; bf16 q/out", data="synthetic",
               config=dict(workload="llama3.1-8b-attention-decode-fp8-kv", batch=B, cache_tokens=T,
                           split_tokens=split,
                           q_heads=H, kv_heads=KVH, head_dim=D, mean_len=round(tokens / B, 1)),
               roofline=dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS,
                             unit="GB/s", frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=None,
                             kernel="attn_decode_mma_kernel<E4M3, 4 query heads per KV head%s> (scores and value sums on bf16 MFMA)"
                                    % (", split" if split else ""),
                             mean_launch_us=round(dec_ms * 1e3, 2),
                             bytes_per_launch=decode_bytes),
               decode_us=round(dec_ms * 1e3, 2), append_us=round(app_ms * 1e3, 2),
               bf16_cache_bytes_ratio=round((tokens * KVH * 4 * D) / (tokens * KVH * (2 * D + 8)), 3))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_kv(lens_np, KVH, H, D, sm)
    return res


def cpu_baseline_kv(lens_np, KVH, H, D, sm, min_seconds: float = 10.0):
    """The oracle's decode attention on two sample sequences of the workload's first two
    lengths (synthetic values of the same distribution, quantized by the oracle), repeated to
    >= min_seconds; GB/s of cache read."""
    import oracle
    import synth

    def u16(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    sample = []
    for i in range(2):
        n = int(lens_np[i])
        cache = []
        for kind in ("K", "V"):
            x = synth.normal((n * KVH, D), 1.0, 11, f"bench/kv/{kind}{i}")
            c, f = oracle.quantize_blockwise(u16(x), oracle.E4M3, oracle.BLOCK_1x128,
                                             oracle.SCALE_FP32)
            cache += [c.reshape(1, n, KVH, D), f.reshape(1, n, KVH)]
        q = u16(synth.normal((1, H, D), 1.0, 11, f"bench/kv/q{i}")).reshape(1, H, D)
        sample.append((q, cache, n))
    nbytes, reps = 0, 0
    t0 = time.perf_counter()
    while True:
        for q, (kc, ks, vc, vs), n in sample:
            oracle.attention_decode(q, kc, ks, vc, vs, [n], sm, oracle.E4M3)
            nbytes += n * KVH * (2 * D + 8) + 4 * H * D
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    return dict(value=round(nbytes / dt / 1e9, 4), unit="GB/s", cores=blas_threads(),
                kind="oracle",
                sample=f"2 sequences of {int(lens_np[0])} and {int(lens_np[1])} tokens (32 query / 8 KV "
                       f"heads) x {reps} repetitions, {dt:.1f} s; NumPy fp64, BLAS threads "
                       f"{blas_threads()}")


def bench_copy(args):
    """A plain 1 GiB device copy (torch), the calibration kernel for the HBM byte counters."""
    dev = torch.device("cuda", 0)
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    for _ in range(args.warmup):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(args.steps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / args.steps
    return dict(metric="device copy GB/s (read + write)", value=round(2 * n / ms / 1e6, 1),
                unit="GB/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
                ms_per_step=round(ms, 4), higher_is_better=True, scaling="weak",
                vs_baseline=None, dtype="u8", data="synthetic",
                config=dict(workload="copy-1GiB", bytes_read=n, bytes_written=n), roofline=None)


# ----------------------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path; the kernels "
              "run on one GPU's share of the work", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.workload == "llama8b-fprop":
        res = bench_llama8b(args)
    elif args.workload == "llama8b-fprop-pow2":
        res = bench_llama8b(args, pow2=True)
    elif args.workload == "backward-mx":
        res = bench_backward_mx(args)
    elif args.workload == "llama8b-fprop-mx":
        res = bench_llama8b_mx(args)
    elif args.workload == "quant-sweep":
        res = bench_quant_sweep(args)
    elif args.workload == "moe":
        res = bench_moe(args)
    elif args.workload == "backward":
        res = bench_backward(args)
    elif args.workload == "backward-blockwise":
        res = bench_backward_blockwise(args)
    elif args.workload == "llama8b-fprop-qout":
        res = bench_fprop_qout(args)
    elif args.workload == "kv-decode":
        res = bench_kv_decode(args)
    elif args.workload == "stream":
        res = bench_stream(args)
    elif args.workload == "mfma-ceiling":
        res = bench_mfma_ceiling(args)
    elif args.workload == "copy":
        res = bench_copy(args)
    else:
        raise SystemExit(f"workload {args.workload} is not available yet")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
