"""CPU oracle for block-scaled FP8 quantization and the block-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline leg of
the benchmark may import this package.  The product library (``block_scaled_quantize_amd``)
never imports it, and the two share no code: this package drives a plain C file
(``fp8_oracle.c``, built with gcc) for the codec and the quantizers, and NumPy fp64 for the
GEMM reference.

Sources, by page title and section (nothing is copied from them):

* "Infraestructura de Entrenamiento FP8: Precisión Numérica de Nueva Generación" (introl.com),
  sections "El panorama de la precisión numérica" (E4M3 / E5M2 bit splits, E4M3 range +-448)
  and "Transformer Engine: la base de software" (delayed scaling recipe: margin 0, history 16,
  "max"; HYBRID = E4M3 forward / E5M2 backward).
* "NVIDIA NeMo RL logra una aceleración del 48% con entrenamiento de precisión FP8 de extremo a
  extremo" (hotbookzone.com), section "El avance técnico" (E4M3 blocks: 128x128 for weights,
  1x128 for activations; FP8 linear layers) and section "Por qué esto es importante para la
  economía de la IA" (power-of-2 scale factors).
* "Infraestructura de Entrenamiento FP8 ...", sections "Estrategias de escalado y estabilidad"
  (block scaling, MXFP8: separate scale factors for blocks within a tensor) and "Blackwell MXFP8
  y NVFP4: mirando hacia adelante" (hardware-accelerated block scaling).  The pages state neither
  the block size nor the scale format; the reading here is the microscaling one: blocks of 32
  consecutive elements along a row, one power-of-two scale per block stored as an E8M0 byte
  (the biased binary exponent, 2^(code - 127); code 255 is NaN), the scale chosen by the same
  power-of-2 rule as the blockwise quantizer.

GEMM reference: dequantize both operands to fp64 (exact), then one fp64 matrix product per
layout.  It is exact up to the rounding of fp64 accumulation, which is far below the
tolerance the GPU result is held to.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

E4M3, E5M2 = 0, 1
BLOCK_1x128, BLOCK_128x128, PER_TENSOR, BLOCK_1x32 = 0, 1, 2, 3
SCALE_FP32, SCALE_POW2 = 0, 1
FPROP, DGRAD, WGRAD = 0, 1, 2

FMAX = {E4M3: 448.0, E5M2: 57344.0}


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def build(force: bool = False) -> str:
    """Compile fp8_oracle.c into liboracle.so with gcc (IEEE arithmetic, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-pthread",
               "-fno-fast-math", "-ffp-contract=off", "-frounding-math", "-fsignaling-nans",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib_handle = None


def _lib():
    global _lib_handle
    if _lib_handle is None:
        lib = ctypes.CDLL(build())
        i64, i32, u32 = ctypes.c_int64, ctypes.c_int, ctypes.c_uint32
        vp = ctypes.c_void_p
        lib.o_decode.argtypes = [i32, i32]
        lib.o_decode.restype = ctypes.c_double
        lib.o_encode.argtypes = [i32, ctypes.c_float]
        lib.o_encode.restype = ctypes.c_uint8
        lib.o_encode_array.argtypes = [i32, vp, i64, vp, i32]
        lib.o_encode_bit_range.argtypes = [i32, u32, i64, vp, i32]
        lib.o_scale_from_amax.argtypes = [i32, i32, ctypes.c_float, i32]
        lib.o_scale_from_amax.restype = ctypes.c_float
        lib.o_quantize_blockwise.argtypes = [vp, i64, i64, i32, i32, i32, vp, vp, i32]
        lib.o_delayed_step.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp, vp, vp, i32]
        lib.o_dequantize.argtypes = [vp, i64, i64, i32, i64, i64, vp, vp, i32]
        for name in ("o_encode_array", "o_encode_bit_range", "o_quantize_blockwise",
                     "o_delayed_step", "o_dequantize"):
            getattr(lib, name).restype = i32
        _lib_handle = lib
    return _lib_handle


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what}: bad argument (rc={rc})")


# ----------------------------------------------------------------------------- codec

def decode_table(fmt: int) -> np.ndarray:
    """Value of each of the 256 codes as fp64 (NaN for NaN codes, +-inf for E5M2 inf)."""
    lib = _lib()
    return np.array([lib.o_decode(fmt, c) for c in range(256)], dtype=np.float64)


def decode(fmt: int, codes: np.ndarray) -> np.ndarray:
    return decode_table(fmt)[np.asarray(codes, dtype=np.uint8)]


def encode(fmt: int, values, nthreads: int | None = None) -> np.ndarray:
    """Saturating round-to-nearest-even encoding of fp32 values."""
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float32))
    out = np.empty(v.shape, dtype=np.uint8)
    _check(_lib().o_encode_array(fmt, _ptr(v), v.size, _ptr(out),
                                 nthreads or default_threads()), "encode")
    return out


def encode_bit_range(fmt: int, first_bits: int, count: int,
                     nthreads: int | None = None) -> np.ndarray:
    """Encode the fp32 values with bit patterns first_bits .. first_bits + count - 1."""
    out = np.empty(count, dtype=np.uint8)
    _check(_lib().o_encode_bit_range(fmt, first_bits, count, _ptr(out),
                                     nthreads or default_threads()), "encode_bit_range")
    return out


def scale_from_amax(fmt: int, mode: int, amax: float, finite: bool = True) -> np.float32:
    return np.float32(_lib().o_scale_from_amax(fmt, mode, float(np.float32(amax)), int(finite)))


# ----------------------------------------------------------------------------- quantizers

def _as_bf16_bits(x) -> np.ndarray:
    """Accept a torch bf16 tensor or a uint16 array of bf16 bit patterns."""
    if hasattr(x, "dtype") and str(x.dtype) == "torch.bfloat16":
        import torch
        return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    a = np.asarray(x)
    if a.dtype != np.uint16:
        raise TypeError("expected bf16 bit patterns (uint16) or a torch.bfloat16 tensor")
    return np.ascontiguousarray(a)


def block_shape(gran: int, rows: int, cols: int) -> tuple[int, int]:
    if gran == BLOCK_1x128:
        return 1, 128
    if gran == BLOCK_1x32:
        return 1, 32
    if gran == BLOCK_128x128:
        return 128, 128
    if gran == PER_TENSOR:
        return max(rows, 1), max(cols, 1)
    raise ValueError("unknown granularity")


def quantize_blockwise(x, fmt: int, gran: int, mode: int, nthreads: int | None = None):
    """Blockwise quantization of a 2-D bf16 matrix.

    Returns (codes uint8 [R, C], scale_inv float32 [ceil(R/bh), ceil(C/bw)]) where the scale
    array is in logical block order (block row, block column).
    """
    xb = _as_bf16_bits(x)
    if xb.ndim != 2:
        raise ValueError("expected a 2-D matrix")
    rows, cols = xb.shape
    bh, bw = block_shape(gran, rows, cols)
    q = np.empty((rows, cols), dtype=np.uint8)
    si = np.empty(((rows + bh - 1) // bh, (cols + bw - 1) // bw), dtype=np.float32)
    _check(_lib().o_quantize_blockwise(_ptr(xb), rows, cols, fmt, gran, mode, _ptr(q), _ptr(si),
                                       nthreads or default_threads()), "quantize_blockwise")
    return q, si


def e8m0_decode(codes) -> np.ndarray:
    """E8M0 scale bytes as fp64 values: 2^(code - 127), NaN for code 255."""
    c = np.asarray(codes, dtype=np.int64)
    out = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, out)


def e8m0_of_pow2(values) -> np.ndarray:
    """The E8M0 byte of each power of two in [2^-127, 2^127] (its binary exponent + 127)."""
    v = np.asarray(values, dtype=np.float64)
    m, e = np.frexp(v)                   # v = m * 2^e, m in [0.5, 1)
    if not np.all(m == 0.5):
        raise ValueError("not a power of two")
    code = e - 1 + 127
    if np.any(code < 0) or np.any(code > 254):
        raise ValueError("outside the E8M0 range")
    return code.astype(np.uint8)


def quantize_mx(x, fmt: int, nthreads: int | None = None):
    """Microscaling quantization of a 2-D bf16 matrix: blocks of 32 consecutive elements along
    each row, the power-of-2 scale rule, dequantization factors stored as E8M0 bytes.

    Returns (codes uint8 [R, C], scale bytes uint8 [R, ceil(C/32)])."""
    q, si = quantize_blockwise(x, fmt, BLOCK_1x32, SCALE_POW2, nthreads)
    return q, e8m0_of_pow2(si)


def gemm_mx(qa, fa: int, sa_e8m0, qb, fb: int, sb_e8m0) -> np.ndarray:
    """fp64 reference of the microscaling GEMM C = A . B^T, A[M, K] and B[N, K] stored row-major
    with one E8M0 scale per 32 consecutive K elements of a row (scale arrays [M, ceil(K/32)] and
    [N, ceil(K/32)])."""
    return gemm(FPROP, qa, fa, BLOCK_1x32, e8m0_decode(sa_e8m0), qb, fb, BLOCK_1x32,
                e8m0_decode(sb_e8m0))


def quantize_mx_columnwise_t(x, fmt: int, nthreads: int | None = None):
    """Microscaling quantization along columns: blocks of 32 consecutive rows of one column of
    x[R, C], codes returned transposed.  Such a block is, by definition, a 32-element row block
    of x^T, so this is quantize_mx of the transpose (the microscaling form of the weight- and
    data-gradient operands, whose contraction runs along the rows of x).

    Returns (codes uint8 [C, R] (of x^T), scale bytes uint8 [C, ceil(R/32)])."""
    xb = _as_bf16_bits(x)
    if xb.ndim != 2:
        raise ValueError("expected a 2-D matrix")
    return quantize_mx(np.ascontiguousarray(xb.T), fmt, nthreads)


def quantize_columnwise_t(x, fmt: int, mode: int, nthreads: int | None = None):
    """Columnwise quantization: blocks of 128 consecutive rows of one column of x[R, C], codes
    returned transposed.  A block of 128 rows of column c of x is, by definition, a 1x128 block
    of row c of x^T, so this is the blockwise 1x128 quantization of the transpose ("NVIDIA NeMo
    RL ...", section "El avance técnico": one scale per 128 elements along the contracted
    dimension, here the token dimension of the weight-gradient product).

    Returns (codes uint8 [C, R] (of x^T), scale_inv float32 [C, ceil(R/128)] in logical block
    order (row of x^T, block along R))."""
    xb = _as_bf16_bits(x)
    if xb.ndim != 2:
        raise ValueError("expected a 2-D matrix")
    return quantize_blockwise(np.ascontiguousarray(xb.T), fmt, BLOCK_1x128, mode, nthreads)


@dataclass
class DelayedState:
    """Per-tensor delayed-scaling state: amax history (newest first) and the current scale."""
    hist_len: int = 16
    history: np.ndarray = field(default=None)
    scale: np.ndarray = field(default=None)

    def __post_init__(self):
        if self.history is None:
            self.history = np.zeros(self.hist_len, dtype=np.float32)
        if self.scale is None:
            self.scale = np.ones(1, dtype=np.float32)

    def copy(self) -> "DelayedState":
        return DelayedState(self.hist_len, self.history.copy(), self.scale.copy())


def delayed_step(x, fmt: int, mode: int, margin: int, state: DelayedState,
                 nthreads: int | None = None):
    """One delayed-scaling step on a bf16 tensor (any shape, flattened).

    Returns (codes uint8 with x's shape, scale_inv_used float32); advances ``state``.
    """
    xb = _as_bf16_bits(x)
    q = np.empty(xb.shape, dtype=np.uint8)
    siu = np.zeros(1, dtype=np.float32)
    _check(_lib().o_delayed_step(_ptr(xb), xb.size, fmt, mode, margin, state.hist_len,
                                 _ptr(state.history), _ptr(state.scale), _ptr(q), _ptr(siu),
                                 nthreads or default_threads()), "delayed_step")
    return q, siu[0]


# ----------------------------------------------------------------------------- GEMM reference

def dequantize(q: np.ndarray, fmt: int, gran: int, scale_inv, nthreads: int | None = None):
    """fp64 values decode(code) * scale_inv[block] of a stored 2-D code matrix.

    ``gran`` names the block shape on the stored matrix (1x128 = one row by 128 consecutive
    columns; 128x128 tiles; PER_TENSOR = one scale).  ``scale_inv`` is in logical block order.
    """
    q = np.ascontiguousarray(q, dtype=np.uint8)
    rows, cols = q.shape
    bh, bw = block_shape(gran, rows, cols)
    si = np.ascontiguousarray(np.asarray(scale_inv, dtype=np.float32).reshape(-1))
    nb = ((rows + bh - 1) // bh) * ((cols + bw - 1) // bw)
    if si.size != nb:
        raise ValueError(f"scale_inv has {si.size} entries, expected {nb}")
    out = np.empty((rows, cols), dtype=np.float64)
    _check(_lib().o_dequantize(_ptr(q), rows, cols, fmt, bh, bw, _ptr(si), _ptr(out),
                               nthreads or default_threads()), "dequantize")
    return out


def gemm(layout: int, qa, fa: int, ga: int, sa, qb, fb: int, gb: int, sb) -> np.ndarray:
    """fp64 reference of the block-scaled GEMM.

    Stored operands (row-major):
      FPROP  A[M,K], B[N,K]:  C = A . B^T
      DGRAD  A[M,K], B[K,N]:  C = A . B
      WGRAD  A[K,M], B[K,N]:  C = A^T . B
    """
    ad = dequantize(qa, fa, ga, sa)
    bd = dequantize(qb, fb, gb, sb)
    if layout == FPROP:
        return ad @ bd.T
    if layout == DGRAD:
        return ad @ bd
    if layout == WGRAD:
        return ad.T @ bd
    raise ValueError("unknown layout")


def grouped_gemm(offsets, qa, sa, fa: int, qbs, sbs, fb: int) -> np.ndarray:
    """fp64 reference of the grouped (MoE) GEMM: for each group g, rows
    [offsets[g], offsets[g+1]) of A[total_M, K] (1x128 scales, logical [total_M, K/128]) times
    B_g[N, K]^T (128x128 scales, logical [N/128, K/128])."""
    offsets = np.asarray(offsets, dtype=np.int64)
    total_m, _ = qa.shape
    n = qbs.shape[1]
    out = np.zeros((total_m, n), dtype=np.float64)
    for g in range(len(offsets) - 1):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 <= r0:
            continue
        out[r0:r1] = gemm(FPROP, qa[r0:r1], fa, BLOCK_1x128, sa[r0:r1], qbs[g], fb,
                          BLOCK_128x128, sbs[g])
    return out


def rel_frobenius(c, ref) -> float:
    c = np.asarray(c, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(c - ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


# ----------------------------------------------------------------------------- FP8 KV cache

def kv_cache_append(cache_codes: np.ndarray, cache_si: np.ndarray, new_bits, positions, fmt: int,
                    mode: int) -> None:
    """Write one new token per sequence into an FP8 KV cache, in place.

    "NVIDIA NeMo RL ..." (hotbookzone.com), section "Ganancias de rendimiento en el mundo real":
    FP8 is extended to the KV cache.  The pages give no cache format; the reading taken here is
    the activation recipe of section "El avance técnico" applied to cached keys and values: each
    128-element head vector of a token is one 1x128 block (E4M3 codes, fp32 scale), quantized
    by the blockwise rule (``quantize_blockwise``).

    cache_codes uint8 [B][T][KVH][128]; cache_si float32 [B][T][KVH] (dequantization factors);
    new_bits: bf16 bit patterns [B][KVH][128]; positions int [B]: token slot of each sequence
    (a slot outside [0, T) leaves that sequence's cache unchanged).
    """
    nb, t_cap, kvh, d = cache_codes.shape
    if d != 128 or cache_si.shape != (nb, t_cap, kvh):
        raise ValueError("cache shapes")
    nbits = _as_bf16_bits(new_bits).reshape(nb, kvh, d)
    for b in range(nb):
        t = int(positions[b])
        if t < 0 or t >= t_cap:
            continue
        q, si = quantize_blockwise(np.ascontiguousarray(nbits[b]), fmt, BLOCK_1x128, mode)
        cache_codes[b, t] = q
        cache_si[b, t] = si[:, 0]


def attention_decode(q_bits, k_codes, k_si, v_codes, v_si, lens, sm_scale: float,
                     fmt: int) -> np.ndarray:
    """fp64 reference of one decode step of grouped-query attention over an FP8 KV cache.

    For sequence b and query head h (KV head kv = h // (H // KVH)), with the cached keys and
    values dequantized exactly (code value times the head vector's factor):
        s_t = sm_scale * sum_d q[b,h,d] K[b,t,kv,d]     for t < L_b
        out[b,h,:] = sum_t softmax(s)_t V[b,t,kv,:]
    L_b = lens[b] clamped to [0, T]; a sequence with no cached token gives zeros (reading: there
    is nothing to attend to).  "Ganancias de rendimiento en el mundo real" (FP8 KV cache and
    attention) fixes no more than that the cache is FP8; the queries stay in bf16 and the
    arithmetic is exact here (fp64).

    q_bits: bf16 bits [B][H][128]; k_codes, v_codes: uint8 [B][T][KVH][128]; k_si, v_si: float32
    [B][T][KVH].  Returns fp64 [B][H][128].
    """
    qb = _as_bf16_bits(q_bits)
    nb, nh, d = qb.shape
    _, t_cap, kvh, _ = k_codes.shape
    if nh % kvh != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    group = nh // kvh
    q = (qb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    table = decode_table(fmt)
    out = np.zeros((nb, nh, d), dtype=np.float64)
    for b in range(nb):
        n = min(max(int(lens[b]), 0), t_cap)
        if n == 0:
            continue
        kd = table[k_codes[b, :n]] * k_si[b, :n, :, None].astype(np.float64)   # [n][KVH][D]
        vd = table[v_codes[b, :n]] * v_si[b, :n, :, None].astype(np.float64)
        for h in range(nh):
            kv = h // group
            s = (kd[:, kv, :] @ q[b, h]) * float(sm_scale)
            s = s - s.max()
            p = np.exp(s)
            p = p / p.sum()
            out[b, h] = p @ vd[:, kv, :]
    return out
