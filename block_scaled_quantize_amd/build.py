"""Build libfp8bs.so from the HIP sources in csrc/ (gfx950 only) with hipcc.

Usage: python -m block_scaled_quantize_amd.build [--force] [-j N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libfp8bs.so")
# kernels the benchmark measures the device's streaming rate and sustained matrix-core rate with
# (not the C ABI)
BENCH_LIB = os.path.join(HERE, "libfp8bs_bench.so")
BENCH_SOURCES = ["bench_stream.hip", "bench_mfma.hip"]
# (the GEMM kernels are split over several files so that they compile in parallel)
SOURCES = ["gemm_fprop.hip", "gemm_fprop_pow2.hip", "gemm_mx.hip", "gemm_dgrad.hip", "gemm_wgrad.hip",
           "gemm_grouped.hip", "gemm_qout.hip", "gemm.hip", "quantize.hip", "quantize_t.hip",
           "attention.hip"]
HEADERS = [os.path.join(CSRC, "common.h"), os.path.join(CSRC, "gemm_impl.h"),
           os.path.join(INCLUDE, "fp8bs.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # gfx950 packed-fp32 instructions are kept out of generated code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def _newer(target: str, deps) -> bool:
    if not os.path.exists(target):
        return False
    t = os.path.getmtime(target)
    return all(os.path.getmtime(d) <= t for d in deps)


def _compile(src: str, force: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if not force and _newer(obj, [path] + HEADERS):
        return obj
    cmd = [HIPCC, *FLAGS, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(force: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        raise RuntimeError("hipcc not found")
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES) + len(BENCH_SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, force), SOURCES + BENCH_SOURCES))
    _link(LIB, objs[:len(SOURCES)], force)
    _link(BENCH_LIB, objs[len(SOURCES):], force)
    return LIB


def _link(lib: str, objs, force: bool) -> None:
    if force or not _newer(lib, objs):
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("link failed")
        os.replace(tmp, lib)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--force", action="store_true")
    ap.add_argument("-j", type=int, default=None)
    a = ap.parse_args()
    print(build(a.force, a.j))
