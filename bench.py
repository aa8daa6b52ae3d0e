"""Benchmark of the FP8 linear-layer hot path on one MI355X.

Default workload (one "step"): the four Llama-3.1-8B-shaped fprop linear layers at M = 8192
tokens -- QKV 4096->6144, O 4096->4096, gate+up 4096->28672, down 14336->4096.  For each layer
the step quantizes the bf16 activation (1x128 blocks, E4M3), re-quantizes the bf16 weight
(128x128 tiles, E4M3: the per-step scale recalibration), and runs the block-scaled FP8 GEMM
with fp32 accumulation and bf16 output.  Inputs are seeded synthetic bf16 tensors resident in
HBM before timing: activations N(0,1) with 1% of the channels scaled by 50, weights N(0,0.02).

value = sum of the GEMMs' 2*M*N*K over the step / step time (TFLOP/s, quantization included).
roofline: the dominant kernel (the block-scaled GEMM) -- algorithmic flops per launch (mean
over the four shapes) / mean launch duration measured with HIP events on the launch stream,
against the MI355X dense FP8 MFMA peak.
cpu_baseline: the CPU oracle (C quantizer + NumPy fp64 GEMM) on a bounded row sample of the
same step, on the host's cores.

Other workloads (--workload): quant-sweep (HBM-bound quantizer), moe (grouped GEMM),
backward (delayed-scaled dgrad / wgrad), tiny.  Each prints one JSON line.
"""
from __future__ import annotations

import argparse
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

LAYERS_8B = [("qkv", 4096, 6144), ("o", 4096, 4096), ("gate_up", 4096, 28672), ("down", 14336, 4096)]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b-fprop",
                    choices=["llama8b-fprop", "quant-sweep", "moe", "backward", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tokens", type=int, default=8192)
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


def cpu_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# ----------------------------------------------------------------------------- 8B fprop

def bench_llama8b(args):
    import block_scaled_quantize_amd as bsq
    import synth
    bsq.load()
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

    def step(timer=None):
        for L in layers:
            def qx():
                bsq.quantize_blockwise(L["x"], bsq.E4M3, bsq.BLOCK_1x128, q=L["qx"], scale_inv=L["sx"])

            def qw():
                bsq.quantize_blockwise(L["w"], bsq.E4M3, bsq.BLOCK_128x128, q=L["qw"], scale_inv=L["sw"])

            def mm():
                bsq.gemm_blockscaled(bsq.FPROP, L["qx"], bsq.E4M3, bsq.BLOCK_1x128, L["sx"], L["qw"],
                                     bsq.E4M3, bsq.BLOCK_128x128, L["sw"], c=L["y"])
            if timer is None:
                qx(); qw(); mm()
            else:
                timer.time(("qx", L["name"]), qx)
                timer.time(("qw", L["name"]), qw)
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
    q_bytes, q_ms = 0.0, 0.0
    for L in layers:
        g = timer.mean_ms(("gemm", L["name"]))
        f = 2.0 * M * L["N"] * L["K"]
        gemm_ms.append(g)
        gemm_flops.append(f)
        qx_ms = timer.mean_ms(("qx", L["name"]))
        qw_ms = timer.mean_ms(("qw", L["name"]))
        xb = M * L["K"] * (2 + 1) + 4 * M * (L["K"] // 128)
        wb = L["N"] * L["K"] * (2 + 1) + 4 * (L["N"] // 128) * (L["K"] // 128)
        q_bytes += xb + wb
        q_ms += qx_ms + qw_ms
        per_layer[L["name"]] = dict(gemm_us=round(g * 1e3, 2), gemm_tflops=round(f / g / 1e9, 1),
                                    quant_x_us=round(qx_ms * 1e3, 2), quant_x_gbps=round(xb / qx_ms / 1e6, 1),
                                    quant_w_us=round(qw_ms * 1e3, 2), quant_w_gbps=round(wb / qw_ms / 1e6, 1))
    mean_launch_flops = float(np.mean(gemm_flops))
    mean_launch_ms = float(np.mean(gemm_ms))
    achieved = mean_launch_flops / mean_launch_ms / 1e9
    result = dict(
        metric="block-scaled FP8 GEMM TFLOP/s (+quantize GB/s), % of MI355X FP8/HBM peak",
        value=round(flops / dt / 1e12, 2), unit="TFLOP/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=round(dt * 1e3, 4), higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype="fp8e4m3 x fp8e4m3 -> fp32 acc -> bf16",
        data="synthetic",
        config=dict(workload="llama3.1-8b-fprop-linear", tokens=M,
                    layers="qkv 4096->6144, o 4096->4096, gate_up 4096->28672, down 14336->4096",
                    act_scales="1x128 E4M3", weight_scales="128x128 E4M3 (re-quantized every step)",
                    parallelism="single GPU"),
        roofline=dict(bound="mfma", achieved=round(achieved, 1), peak=FP8_PEAK_TFLOPS,
                      unit="TFLOP/s", frac=round(achieved / FP8_PEAK_TFLOPS, 4), traffic=None,
                      kernel="gemm_kernel<FPROP,E4M3,E4M3,fold,BM=256>",
                      per_launch_flops=mean_launch_flops, mean_launch_us=round(mean_launch_ms * 1e3, 2)),
        gemm_only_tflops=round(sum(gemm_flops) / sum(gemm_ms) / 1e9, 1),
        quant_gbps=round(q_bytes / q_ms / 1e6, 1),
        quant_hbm_frac=round(q_bytes / q_ms / 1e6 / HBM_PEAK_GBPS, 4),
        layers=per_layer,
    )
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_8b(layers, M)
    return result


def cpu_baseline_8b(layers, M, rows: int = 64):
    """The oracle on a row sample of the same step: quantize `rows` activation rows (1x128),
    the full weight (128x128), dequantize and multiply in fp64.  Scaled to TFLOP/s of the
    sample's GEMM flops."""
    import oracle
    oracle.build()
    t0 = time.perf_counter()
    flops = 0.0
    for L in layers:
        xs = L["x"][:rows].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        ws = L["w"].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        qx, sx = oracle.quantize_blockwise(xs, oracle.E4M3, oracle.BLOCK_1x128, oracle.SCALE_FP32)
        qw, sw = oracle.quantize_blockwise(ws, oracle.E4M3, oracle.BLOCK_128x128, oracle.SCALE_FP32)
        oracle.gemm(oracle.FPROP, qx, oracle.E4M3, oracle.BLOCK_1x128, sx, qw, oracle.E4M3,
                    oracle.BLOCK_128x128, sw)
        flops += 2.0 * rows * L["N"] * L["K"]
    dt = time.perf_counter() - t0
    return dict(value=round(flops / dt / 1e12, 5), unit="TFLOP/s", cores=cpu_cores(), kind="oracle",
                sample=f"{rows} of {M} token rows per layer (all four layers, full weights "
                       f"re-quantized), {dt:.1f} s")


# ----------------------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(see the sharding notes in the design document)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.workload == "llama8b-fprop":
        res = bench_llama8b(args)
    else:
        raise SystemExit(f"workload {args.workload} is not available yet")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
