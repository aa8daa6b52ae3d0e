"""Python binding of libfp8bs (block-scaled FP8 quantization and GEMM on AMD MI355X).

Argument marshalling only: every step of the computation runs in the HIP kernels behind the
C ABI declared in ``include/fp8bs.h``.  PyTorch provides device memory and the current HIP
stream.  There is no CPU fallback: if the shared library is missing or a GPU is not present,
calls raise.

Names follow the C ABI: ``quantize_blockwise`` (fp8_quantize_blockwise), ``quantize_delayed``
(fp8_quantize_delayed), ``gemm_blockscaled`` (fp8_gemm_blockscaled), ``grouped_gemm``
(fp8_grouped_gemm), ``cast_fp32`` (fp8_cast_fp32).
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp8bs.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "fp8bs.h")

E4M3, E5M2 = 0, 1
BLOCK_1x128, BLOCK_128x128, PER_TENSOR = 0, 1, 2
SCALE_FP32, SCALE_POW2 = 0, 1
FPROP, DGRAD, WGRAD = 0, 1, 2
# output-tile configurations of the *_tiled entry points (fp8bs_tile)
TILE_AUTO, TILE_256x128_W4, TILE_256x128_W8, TILE_256x256_W8, TILE_128x128_W4 = 0, 1, 2, 3, 4

OK = 0
ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED, ERR_LAUNCH, ERR_WORKSPACE, ERR_ARG = (
    -1, -2, -3, -4, -5, -6, -7)


class Fp8bsError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lib = None


def declared_functions() -> list[str]:
    """Names of the functions include/fp8bs.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libfp8bs.so (after torch, so that one HIP runtime is shared)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m block_scaled_quantize_amd.build`")
    lib = ctypes.CDLL(path)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    lib.fp8bs_status_string.argtypes = [i32]
    lib.fp8bs_status_string.restype = ctypes.c_char_p
    lib.fp8_quantize_blockwise.argtypes = [vp, i64, i64, i64, i32, i32, i32, vp, i64, vp, vp]
    lib.fp8_quantize_columnwise_t.argtypes = [vp, i64, i64, i64, i32, i32, vp, i64, vp, vp]
    lib.fp8_quantize_mx_columnwise_t.argtypes = [vp, i64, i64, i64, i32, vp, i64, vp, vp]
    lib.fp8_quantize_1x128_and_columnwise_t.argtypes = [vp, i64, i64, i64, i32, i32, vp, i64, vp,
                                                        vp, i64, vp, vp]
    lib.fp8_quantize_mx_and_columnwise_t.argtypes = [vp, i64, i64, i64, i32, vp, i64, vp, vp, i64,
                                                     vp, vp]
    lib.fp8_grouped_gemm_mx.argtypes = [i32, vp, i64, i64, i64, vp, i64, i32, vp, vp, i64, i32, vp,
                                        vp, i64, vp]
    lib.fp8_quantize_mx.argtypes = [vp, i64, i64, i64, i32, vp, i64, vp, vp]
    lib.fp8_gemm_mx.argtypes = [i64, i64, i64, vp, i64, i32, vp, vp, i64, i32, vp, vp, i64, vp]
    lib.fp8_quantize_blockwise_batched.argtypes = [i32, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp]
    lib.fp8_quantize_delayed.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.fp8_quantize_delayed_noalloc.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp]
    lib.fp8_quantize_delayed_workspace_size.argtypes = []
    lib.fp8_quantize_delayed_workspace_size.restype = sz
    lib.fp8_cast_fp32.argtypes = [vp, i64, i32, vp, vp]
    lib.fp8_gemm_blockscaled.argtypes = [i32, i64, i64, i64, vp, i64, i32, i32, vp, vp, i64, i32,
                                         i32, vp, vp, i64, vp]
    lib.fp8_grouped_gemm.argtypes = [ctypes.c_int32, vp, i64, i64, i64, vp, i64, i32, vp, vp,
                                     i64, i32, vp, vp, i64, vp]
    lib.fp8_gemm_blockscaled_pow2.argtypes = lib.fp8_gemm_blockscaled.argtypes
    lib.fp8_gemm_blockscaled_qout.argtypes = [i64, i64, i64, vp, i64, i32, vp, vp, i64, i32, vp,
                                              i32, vp, i64, i32, vp, i64, vp, vp]
    lib.fp8_grouped_gemm_pow2.argtypes = lib.fp8_grouped_gemm.argtypes
    lib.fp8_gemm_blockscaled_tiled.argtypes = [i32, i32] + lib.fp8_gemm_blockscaled.argtypes
    lib.fp8_grouped_gemm_tiled.argtypes = [i32, i32] + lib.fp8_grouped_gemm.argtypes
    lib.fp8_gemm_blockscaled_qout_tiled.argtypes = [i32] + lib.fp8_gemm_blockscaled_qout.argtypes
    lib.fp8_kv_cache_append.argtypes = [i64, i64, i64, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp]
    lib.fp8_attention_decode.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp,
                                         ctypes.c_float, i32, vp, vp]
    lib.fp8_attention_decode_split.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp,
                                               ctypes.c_float, i32, i64, vp, sz, vp, vp]
    lib.fp8_attention_decode_workspace_size.argtypes = [i64, i64, i64, i64, i64]
    lib.fp8_attention_decode_workspace_size.restype = sz
    for name in ("fp8_quantize_blockwise", "fp8_quantize_columnwise_t",
                 "fp8_quantize_mx_columnwise_t", "fp8_quantize_1x128_and_columnwise_t",
                 "fp8_quantize_mx_and_columnwise_t", "fp8_grouped_gemm_mx",
                 "fp8_quantize_delayed",
                 "fp8_quantize_blockwise_batched",
                 "fp8_quantize_delayed_noalloc",
                 "fp8_cast_fp32",
                 "fp8_gemm_blockscaled", "fp8_grouped_gemm", "fp8_gemm_blockscaled_pow2",
                 "fp8_gemm_blockscaled_qout",
                 "fp8_grouped_gemm_pow2", "fp8_gemm_blockscaled_tiled", "fp8_grouped_gemm_tiled",
                 "fp8_gemm_blockscaled_qout_tiled", "fp8_quantize_mx", "fp8_gemm_mx"):
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().fp8bs_status_string(status).decode()


def _check(rc: int, what: str) -> None:
    if rc != OK:
        raise Fp8bsError(rc, what)


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _bf16_out(rows: int, cols: int, device) -> torch.Tensor:
    """A bf16 output matrix whose row pitch is even (the GEMM's 4-byte store alignment)."""
    ld = cols + (cols & 1)
    return torch.empty((rows, ld), dtype=torch.bfloat16, device=device)[:, :cols]


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    return t.data_ptr()


def _ceil(a: int, b: int) -> int:
    return -(-a // b)


def _need(t: torch.Tensor, shape, dtype, what: str, contiguous: bool = True) -> None:
    """Raise ValueError unless t is a device tensor of this shape and dtype (and contiguous)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{what}: expected a device tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or (contiguous and not t.is_contiguous()):
        raise ValueError(f"{what}: expected a{' contiguous' if contiguous else ''} {dtype} tensor of "
                         f"shape {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


def _need_matrix(t: torch.Tensor, shape, dtype, what: str) -> None:
    """A row-major 2-D matrix of this shape (any row pitch, unit column stride)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{what}: expected a device tensor")
    if (t.dim() != 2 or tuple(t.shape) != tuple(shape) or t.dtype != dtype or
            (t.shape[1] > 1 and t.stride(1) != 1) or t.stride(0) < max(1, t.shape[1])):
        raise ValueError(f"{what}: expected a row-major {dtype} matrix of shape {tuple(shape)}, got "
                         f"{t.dtype} {tuple(t.shape)} strides {tuple(t.stride())}")


def _operand_scale_shape(gran: int, stored_rows: int, stored_cols: int) -> tuple[int, ...]:
    if gran not in (BLOCK_1x128, BLOCK_128x128, PER_TENSOR):
        raise ValueError("unknown scale granularity")
    return scale_shape(stored_rows, stored_cols, gran)


def scale_shape(rows: int, cols: int, gran: int) -> tuple[int, ...]:
    """Shape of the dequantization-factor array of a [rows, cols] matrix."""
    if gran == BLOCK_1x128:
        return (_ceil(cols, 128), rows)
    if gran == BLOCK_128x128:
        return (_ceil(rows, 128), _ceil(cols, 128))
    return (1,)


# ----------------------------------------------------------------------------- quantization

def quantize_blockwise(x: torch.Tensor, fmt: int, gran: int, mode: int = SCALE_FP32,
                       q: torch.Tensor | None = None, scale_inv: torch.Tensor | None = None,
                       stream=None):
    """Blockwise quantization of a 2-D bf16 matrix (rows may be strided).

    Returns (codes uint8 [rows, cols], scale_inv float32 in the C ABI layout)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 matrix with unit column stride")
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scale_inv is None:
        scale_inv = torch.empty(scale_shape(rows, cols, gran), dtype=torch.float32, device=x.device)
    _check(load().fp8_quantize_blockwise(_ptr(x), rows, cols, x.stride(0), fmt, gran, mode,
                                         _ptr(q), q.stride(0), _ptr(scale_inv), _stream(stream)),
           "fp8_quantize_blockwise")
    return q, scale_inv


def mx_scale_shape(rows: int, cols: int) -> tuple[int, int, int]:
    """Shape of a microscaling scale array: [ceil(cols / 128)][rows][4] E8M0 bytes."""
    return (_ceil(cols, 128), rows, 4)


def quantize_mx(x: torch.Tensor, fmt: int, q: torch.Tensor | None = None,
                scales: torch.Tensor | None = None, stream=None):
    """Microscaling quantization of a 2-D bf16 matrix: 32-element row blocks, E8M0 scale bytes.

    Returns (codes uint8 [rows, cols], scale bytes uint8 mx_scale_shape(rows, cols))."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 matrix with unit column stride")
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(mx_scale_shape(rows, cols), dtype=torch.uint8, device=x.device)
    _need_matrix(q, (rows, cols), torch.uint8, "q")
    _need(scales, mx_scale_shape(rows, cols), torch.uint8, "scales")
    _check(load().fp8_quantize_mx(_ptr(x), rows, cols, x.stride(0), fmt, _ptr(q), q.stride(0),
                                  _ptr(scales), _stream(stream)), "fp8_quantize_mx")
    return q, scales


def gemm_mx(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor,
            fa: int = E4M3, fb: int = E4M3, c: torch.Tensor | None = None,
            stream=None) -> torch.Tensor:
    """Microscaling FP8 GEMM C[M, N] = A[M, K] . B[N, K]^T with E8M0 scale bytes
    sa mx_scale_shape(M, K) and sb mx_scale_shape(N, K) (as quantize_mx writes them), bf16
    output."""
    if a.dtype != torch.uint8 or b.dtype != torch.uint8 or a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D uint8 code matrices")
    (M, K), N = a.shape, b.shape[0]
    if b.shape[1] != K:
        raise ValueError("K mismatch")
    _need_matrix(a, a.shape, torch.uint8, "a")
    _need_matrix(b, b.shape, torch.uint8, "b")
    _need(sa, mx_scale_shape(M, K), torch.uint8, "sa")
    _need(sb, mx_scale_shape(N, K), torch.uint8, "sb")
    if c is None:
        c = _bf16_out(M, N, a.device)
    _need_matrix(c, (M, N), torch.bfloat16, "c")
    _check(load().fp8_gemm_mx(M, N, K, _ptr(a), a.stride(0), fa, _ptr(sa), _ptr(b), b.stride(0),
                              fb, _ptr(sb), _ptr(c), c.stride(0), _stream(stream)), "fp8_gemm_mx")
    return c


def quantize_blockwise_batched(xs, grans, fmt: int, mode: int = SCALE_FP32, qs=None,
                               scale_invs=None, stream=None):
    """Blockwise quantization of several 2-D bf16 matrices in one launch
    (fp8_quantize_blockwise_batched); grans[i] is BLOCK_1x128 or BLOCK_128x128 for xs[i].

    Returns (list of codes, list of scale_inv), as quantize_blockwise returns for each."""
    n = len(xs)
    if len(grans) != n:
        raise ValueError("one granularity per tensor")
    qs = list(qs) if qs is not None else [None] * n
    scale_invs = list(scale_invs) if scale_invs is not None else [None] * n
    for i, x in enumerate(xs):
        if x.dtype != torch.bfloat16 or x.dim() != 2 or (x.shape[1] > 1 and x.stride(1) != 1):
            raise ValueError("each x must be a 2-D bf16 matrix with unit column stride")
        rows, cols = x.shape
        if qs[i] is None:
            qs[i] = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
        _need_matrix(qs[i], (rows, cols), torch.uint8, f"q[{i}]")
        shape = _operand_scale_shape(grans[i], rows, cols)
        if scale_invs[i] is None:
            scale_invs[i] = torch.empty(shape, dtype=torch.float32, device=x.device)
        _need(scale_invs[i], shape, torch.float32, f"scale_inv[{i}]")
    P = ctypes.c_void_p * max(n, 1)
    I64 = ctypes.c_int64 * max(n, 1)
    I32 = ctypes.c_int * max(n, 1)
    _check(load().fp8_quantize_blockwise_batched(
        n, P(*[_ptr(x) for x in xs]), I64(*[x.shape[0] for x in xs]), I64(*[x.shape[1] for x in xs]),
        I64(*[x.stride(0) for x in xs]), I32(*grans), fmt, mode, P(*[_ptr(q) for q in qs]),
        I64(*[q.stride(0) for q in qs]), P(*[_ptr(s) for s in scale_invs]), _stream(stream)),
        "fp8_quantize_blockwise_batched")
    return qs, scale_invs


def quantize_columnwise_t(x: torch.Tensor, fmt: int, mode: int = SCALE_FP32,
                          qt: torch.Tensor | None = None, scale_inv: torch.Tensor | None = None,
                          stream=None):
    """Columnwise (128 rows x 1 column blocks) quantization of a 2-D bf16 matrix x[rows, cols],
    codes written transposed.

    Returns (codes uint8 [cols, rows] = the codes of x^T, scale_inv float32
    [ceil(rows/128), cols] = the 1x128 scale layout of x^T)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 matrix with unit column stride")
    rows, cols = x.shape
    if qt is None:
        qt = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    if scale_inv is None:
        scale_inv = torch.empty(((rows + 127) // 128, cols), dtype=torch.float32, device=x.device)
    _check(load().fp8_quantize_columnwise_t(_ptr(x), rows, cols, x.stride(0), fmt, mode, _ptr(qt),
                                            qt.stride(0), _ptr(scale_inv), _stream(stream)),
           "fp8_quantize_columnwise_t")
    return qt, scale_inv


def quantize_1x128_and_columnwise_t(x: torch.Tensor, fmt: int, mode: int = SCALE_FP32,
                                    q: torch.Tensor | None = None,
                                    scale_inv: torch.Tensor | None = None,
                                    qt: torch.Tensor | None = None,
                                    scale_inv_t: torch.Tensor | None = None, stream=None):
    """quantize_blockwise(x, fmt, BLOCK_1x128, mode) and quantize_columnwise_t(x, fmt, mode) in
    one pass over x.  Returns (q, scale_inv, qt, scale_inv_t) as those two calls would."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 matrix with unit column stride")
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scale_inv is None:
        scale_inv = torch.empty(scale_shape(rows, cols, BLOCK_1x128), dtype=torch.float32,
                                device=x.device)
    if qt is None:
        qt = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    if scale_inv_t is None:
        scale_inv_t = torch.empty(((rows + 127) // 128, cols), dtype=torch.float32, device=x.device)
    _need_matrix(q, (rows, cols), torch.uint8, "q")
    _need_matrix(qt, (cols, rows), torch.uint8, "qt")
    _need(scale_inv, scale_shape(rows, cols, BLOCK_1x128), torch.float32, "scale_inv")
    _need(scale_inv_t, ((rows + 127) // 128, cols), torch.float32, "scale_inv_t")
    _check(load().fp8_quantize_1x128_and_columnwise_t(
        _ptr(x), rows, cols, x.stride(0), fmt, mode, _ptr(q), q.stride(0), _ptr(scale_inv),
        _ptr(qt), qt.stride(0), _ptr(scale_inv_t), _stream(stream)),
        "fp8_quantize_1x128_and_columnwise_t")
    return q, scale_inv, qt, scale_inv_t


def quantize_mx_and_columnwise_t(x: torch.Tensor, fmt: int, q: torch.Tensor | None = None,
                                 scales: torch.Tensor | None = None,
                                 qt: torch.Tensor | None = None,
                                 scales_t: torch.Tensor | None = None, stream=None):
    """quantize_mx(x, fmt) and quantize_mx_columnwise_t(x, fmt) in one pass over x.
    Returns (q, scales, qt, scales_t) as those two calls would."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 matrix with unit column stride")
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(mx_scale_shape(rows, cols), dtype=torch.uint8, device=x.device)
    if qt is None:
        qt = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    if scales_t is None:
        scales_t = torch.empty(mx_scale_shape(cols, rows), dtype=torch.uint8, device=x.device)
    _need_matrix(q, (rows, cols), torch.uint8, "q")
    _need_matrix(qt, (cols, rows), torch.uint8, "qt")
    _need(scales, mx_scale_shape(rows, cols), torch.uint8, "scales")
    _need(scales_t, mx_scale_shape(cols, rows), torch.uint8, "scales_t")
    _check(load().fp8_quantize_mx_and_columnwise_t(
        _ptr(x), rows, cols, x.stride(0), fmt, _ptr(q), q.stride(0), _ptr(scales), _ptr(qt),
        qt.stride(0), _ptr(scales_t), _stream(stream)), "fp8_quantize_mx_and_columnwise_t")
    return q, scales, qt, scales_t


def quantize_mx_columnwise_t(x: torch.Tensor, fmt: int, qt: torch.Tensor | None = None,
                             scales: torch.Tensor | None = None, stream=None):
    """Microscaling quantization along columns (blocks of 32 rows of one column) of a 2-D bf16
    matrix x[rows, cols], codes written transposed.

    Returns (codes uint8 [cols, rows] = the codes of x^T, scale bytes uint8
    mx_scale_shape(cols, rows) = the microscaling scale layout of x^T)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 matrix with unit column stride")
    rows, cols = x.shape
    if qt is None:
        qt = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(mx_scale_shape(cols, rows), dtype=torch.uint8, device=x.device)
    _need_matrix(qt, (cols, rows), torch.uint8, "qt")
    _need(scales, mx_scale_shape(cols, rows), torch.uint8, "scales")
    _check(load().fp8_quantize_mx_columnwise_t(_ptr(x), rows, cols, x.stride(0), fmt, _ptr(qt),
                                               qt.stride(0), _ptr(scales), _stream(stream)),
           "fp8_quantize_mx_columnwise_t")
    return qt, scales


def delayed_workspace_size() -> int:
    return int(load().fp8_quantize_delayed_workspace_size())


class DelayedState:
    """Device-resident delayed-scaling state: amax history (newest first) and scale."""

    def __init__(self, hist_len: int = 16, device="cuda"):
        self.hist_len = hist_len
        self.history = torch.zeros(hist_len, dtype=torch.float32, device=device)
        self.scale = torch.ones(1, dtype=torch.float32, device=device)
        self.workspace = torch.empty(delayed_workspace_size(), dtype=torch.uint8, device=device)


def quantize_delayed(x: torch.Tensor, fmt: int, state: DelayedState, mode: int = SCALE_FP32,
                     margin: int = 0, q: torch.Tensor | None = None,
                     scale_inv_used: torch.Tensor | None = None, stream=None,
                     noalloc: bool = False):
    """One delayed-scaling step on a contiguous bf16 tensor; advances ``state`` on the device.
    noalloc=True calls fp8_quantize_delayed_noalloc (the library's own scratch array instead of
    state.workspace; q and scale_inv_used must then be given, since creating them allocates).

    Returns (codes uint8 with x's shape, scale_inv_used float32[1])."""
    if x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 tensor")
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scale_inv_used is None:
        scale_inv_used = torch.empty(1, dtype=torch.float32, device=x.device)
    _need(q, x.shape, torch.uint8, "q")
    _need(scale_inv_used, (1,), torch.float32, "scale_inv_used")
    if noalloc:
        _check(load().fp8_quantize_delayed_noalloc(_ptr(x), x.numel(), fmt, mode, margin,
                                                   state.hist_len, _ptr(state.history),
                                                   _ptr(state.scale), _ptr(q),
                                                   _ptr(scale_inv_used), _stream(stream)),
               "fp8_quantize_delayed_noalloc")
        return q, scale_inv_used
    _check(load().fp8_quantize_delayed(_ptr(x), x.numel(), fmt, mode, margin, state.hist_len,
                                       _ptr(state.history), _ptr(state.scale), _ptr(q),
                                       _ptr(scale_inv_used), _ptr(state.workspace),
                                       state.workspace.numel(), _stream(stream)),
           "fp8_quantize_delayed")
    return q, scale_inv_used


def cast_fp32(x: torch.Tensor, fmt: int, q: torch.Tensor | None = None, stream=None):
    """Saturating RNE cast of fp32 values to FP8 codes."""
    if x.dtype != torch.float32 or not x.is_contiguous():
        raise ValueError("x must be a contiguous fp32 tensor")
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(load().fp8_cast_fp32(_ptr(x), x.numel(), fmt, _ptr(q), _stream(stream)), "fp8_cast_fp32")
    return q


# ----------------------------------------------------------------------------- GEMM

def gemm_blockscaled(layout: int, a: torch.Tensor, fa: int, ga: int, sa: torch.Tensor,
                     b: torch.Tensor, fb: int, gb: int, sb: torch.Tensor,
                     c: torch.Tensor | None = None, stream=None, pow2: bool = False,
                     tile: int = TILE_AUTO) -> torch.Tensor:
    """Block-scaled FP8 GEMM, bf16 output.  a, b are uint8 code matrices as stored:
    FPROP a[M,K], b[N,K]; DGRAD a[M,K], b[K,N]; WGRAD a[K,M], b[K,N].  pow2=True calls
    fp8_gemm_blockscaled_pow2 (scales must be powers of two; applied by the MFMA).  tile other
    than TILE_AUTO calls fp8_gemm_blockscaled_tiled with that tile configuration."""
    if a.dtype != torch.uint8 or b.dtype != torch.uint8 or a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D uint8 code matrices")
    if layout == FPROP:
        (M, K), N = a.shape, b.shape[0]
        if b.shape[1] != K:
            raise ValueError("K mismatch")
    elif layout == DGRAD:
        (M, K), N = a.shape, b.shape[1]
        if b.shape[0] != K:
            raise ValueError("K mismatch")
    elif layout == WGRAD:
        (K, M), N = a.shape, b.shape[1]
        if b.shape[0] != K:
            raise ValueError("K mismatch")
    else:
        raise ValueError("unknown layout")
    _need_matrix(a, a.shape, torch.uint8, "a")
    _need_matrix(b, b.shape, torch.uint8, "b")
    _need(sa, _operand_scale_shape(ga, *a.shape), torch.float32, "sa")
    _need(sb, _operand_scale_shape(gb, *b.shape), torch.float32, "sb")
    if c is None:
        c = _bf16_out(M, N, a.device)
    _need_matrix(c, (M, N), torch.bfloat16, "c")
    args = (layout, M, N, K, _ptr(a), a.stride(0), fa, ga, _ptr(sa), _ptr(b), b.stride(0), fb, gb,
            _ptr(sb), _ptr(c), c.stride(0), _stream(stream))
    if tile != TILE_AUTO:
        _check(load().fp8_gemm_blockscaled_tiled(tile, int(pow2), *args), "fp8_gemm_blockscaled_tiled")
        return c
    name = "fp8_gemm_blockscaled_pow2" if pow2 else "fp8_gemm_blockscaled"
    _check(getattr(load(), name)(*args), name)
    return c


def gemm_blockscaled_qout(a: torch.Tensor, ga: int, sa: torch.Tensor, b: torch.Tensor, gb: int,
                          sb: torch.Tensor, mode_out: int = SCALE_FP32, pow2_inputs: bool = False,
                          want_bf16: bool = True, c: torch.Tensor | None = None,
                          cq: torch.Tensor | None = None, cqs: torch.Tensor | None = None,
                          stream=None, tile: int = TILE_AUTO):
    """fprop GEMM (a[M,K] . b[N,K]^T, E4M3 codes) whose epilogue also quantizes the bf16 output
    in 1x128 blocks (E4M3).  Returns (c bf16 [M,N] or None, cq uint8 [M,N],
    cqs float32 [ceil(N/128), M]).  tile other than TILE_AUTO calls
    fp8_gemm_blockscaled_qout_tiled."""
    if a.dtype != torch.uint8 or b.dtype != torch.uint8 or a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D uint8 code matrices")
    (M, K), N = a.shape, b.shape[0]
    if b.shape[1] != K:
        raise ValueError("K mismatch")
    _need_matrix(a, a.shape, torch.uint8, "a")
    _need_matrix(b, b.shape, torch.uint8, "b")
    _need(sa, _operand_scale_shape(ga, M, K), torch.float32, "sa")
    _need(sb, _operand_scale_shape(gb, N, K), torch.float32, "sb")
    if c is None and want_bf16:
        c = _bf16_out(M, N, a.device)
    if c is not None:
        _need_matrix(c, (M, N), torch.bfloat16, "c")
    if cq is None:
        cq = torch.empty((M, N), dtype=torch.uint8, device=a.device)
    _need_matrix(cq, (M, N), torch.uint8, "cq")
    if cqs is None:
        cqs = torch.empty(((N + 127) // 128, M), dtype=torch.float32, device=a.device)
    _need(cqs, ((N + 127) // 128, M), torch.float32, "cqs")
    args = (M, N, K, _ptr(a), a.stride(0), ga, _ptr(sa), _ptr(b), b.stride(0), gb, _ptr(sb),
            int(pow2_inputs), _ptr(c) if c is not None else None,
            c.stride(0) if c is not None else 0, mode_out, _ptr(cq), cq.stride(0), _ptr(cqs),
            _stream(stream))
    if tile != TILE_AUTO:
        _check(load().fp8_gemm_blockscaled_qout_tiled(tile, *args), "fp8_gemm_blockscaled_qout_tiled")
    else:
        _check(load().fp8_gemm_blockscaled_qout(*args), "fp8_gemm_blockscaled_qout")
    return c, cq, cqs


def grouped_gemm(offsets: torch.Tensor, a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor,
                 sb: torch.Tensor, fa: int = E4M3, fb: int = E4M3,
                 c: torch.Tensor | None = None, stream=None, pow2: bool = False,
                 tile: int = TILE_AUTO) -> torch.Tensor:
    """Grouped FP8 GEMM: rows [offsets[g], offsets[g+1]) of a[total_M, K] times b[g][N, K]^T.
    offsets is a device int64 tensor of num_groups + 1 entries.  pow2=True calls
    fp8_grouped_gemm_pow2 (power-of-two scales applied by the MFMA); tile other than TILE_AUTO
    calls fp8_grouped_gemm_tiled."""
    if b.dim() != 3 or b.dtype != torch.uint8 or not b.is_cuda:
        raise ValueError("b must be a uint8 device tensor [G, N, K]")
    G, N, K = b.shape
    if (b.stride(2) != 1 and K > 1) or b.stride(1) < K or (G > 1 and b.stride(0) != N * b.stride(1)):
        raise ValueError("b must hold [G, N, K] with unit column stride and experts N rows apart")
    _need(offsets, (G + 1,), torch.int64, "offsets")
    if a.dim() != 2 or a.shape[1] != K:
        raise ValueError("a must be [total_M, K]")
    _need_matrix(a, a.shape, torch.uint8, "a")
    total_m = a.shape[0]
    _need(sa, scale_shape(total_m, K, BLOCK_1x128), torch.float32, "sa")
    _need(sb, (G, _ceil(N, 128), _ceil(K, 128)), torch.float32, "sb")
    if c is None:
        c = _bf16_out(total_m, N, a.device)
    _need_matrix(c, (total_m, N), torch.bfloat16, "c")
    args = (G, _ptr(offsets), total_m, N, K, _ptr(a), a.stride(0), fa, _ptr(sa), _ptr(b),
            b.stride(1), fb, _ptr(sb), _ptr(c), c.stride(0), _stream(stream))
    if tile != TILE_AUTO:
        _check(load().fp8_grouped_gemm_tiled(tile, int(pow2), *args), "fp8_grouped_gemm_tiled")
        return c
    name = "fp8_grouped_gemm_pow2" if pow2 else "fp8_grouped_gemm"
    _check(getattr(load(), name)(*args), name)
    return c


def grouped_gemm_mx(offsets: torch.Tensor, a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor,
                    sb: torch.Tensor, fa: int = E4M3, fb: int = E4M3,
                    c: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Grouped microscaling GEMM: rows [offsets[g], offsets[g+1]) of a[total_M, K] times
    b[g][N, K]^T, with E8M0 scale bytes sa mx_scale_shape(total_M, K) and sb
    [G, *mx_scale_shape(N, K)] (quantize_mx of a and of each expert)."""
    if b.dim() != 3 or b.dtype != torch.uint8 or not b.is_cuda:
        raise ValueError("b must be a uint8 device tensor [G, N, K]")
    G, N, K = b.shape
    if (b.stride(2) != 1 and K > 1) or b.stride(1) < K or (G > 1 and b.stride(0) != N * b.stride(1)):
        raise ValueError("b must hold [G, N, K] with unit column stride and experts N rows apart")
    _need(offsets, (G + 1,), torch.int64, "offsets")
    if a.dim() != 2 or a.shape[1] != K:
        raise ValueError("a must be [total_M, K]")
    _need_matrix(a, a.shape, torch.uint8, "a")
    total_m = a.shape[0]
    _need(sa, mx_scale_shape(total_m, K), torch.uint8, "sa")
    _need(sb, (G,) + mx_scale_shape(N, K), torch.uint8, "sb")
    if c is None:
        c = _bf16_out(total_m, N, a.device)
    _need_matrix(c, (total_m, N), torch.bfloat16, "c")
    _check(load().fp8_grouped_gemm_mx(G, _ptr(offsets), total_m, N, K, _ptr(a), a.stride(0), fa,
                                      _ptr(sa), _ptr(b), b.stride(1), fb, _ptr(sb), _ptr(c),
                                      c.stride(0), _stream(stream)), "fp8_grouped_gemm_mx")
    return c


def kv_cache_append(k_new: torch.Tensor, v_new: torch.Tensor, positions: torch.Tensor,
                    k_codes: torch.Tensor, k_scale_inv: torch.Tensor, v_codes: torch.Tensor,
                    v_scale_inv: torch.Tensor, fmt: int = E4M3, mode: int = SCALE_FP32,
                    stream=None) -> None:
    """Quantize one new token per sequence (k_new, v_new: bf16 [B, KVH, 128]) into the FP8 cache
    (codes uint8 [B, T, KVH, 128], factors float32 [B, T, KVH]) at slot positions[b] (device
    int32 [B])."""
    if k_codes.dim() != 4 or k_codes.shape[3] != 128:
        raise ValueError("k_codes must be [B, T, KVH, 128]")
    B, T, KVH, _ = k_codes.shape
    for t, shape, dt in ((k_new, (B, KVH, 128), torch.bfloat16), (v_new, (B, KVH, 128), torch.bfloat16),
                         (v_codes, (B, T, KVH, 128), torch.uint8),
                         (k_scale_inv, (B, T, KVH), torch.float32),
                         (v_scale_inv, (B, T, KVH), torch.float32), (positions, (B,), torch.int32)):
        if tuple(t.shape) != shape or t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"expected a contiguous {dt} tensor of shape {shape}")
    _check(load().fp8_kv_cache_append(B, KVH, T, _ptr(k_new), _ptr(v_new), _ptr(positions), fmt,
                                      mode, _ptr(k_codes), _ptr(k_scale_inv), _ptr(v_codes),
                                      _ptr(v_scale_inv), _stream(stream)), "fp8_kv_cache_append")


def attention_decode(q: torch.Tensor, k_codes: torch.Tensor, k_scale_inv: torch.Tensor,
                     v_codes: torch.Tensor, v_scale_inv: torch.Tensor, seq_lens: torch.Tensor,
                     sm_scale: float, fmt: int = E4M3, out: torch.Tensor | None = None,
                     stream=None, split_tokens: int | None = None,
                     workspace: torch.Tensor | None = None) -> torch.Tensor:
    """One decode step of grouped-query attention (q: bf16 [B, H, 128]) over the FP8 cache;
    returns bf16 [B, H, 128].  split_tokens: call fp8_attention_decode_split with chunks of that
    many tokens (workspace: a device tensor of at least attention_decode_workspace_size bytes,
    allocated here when not given)."""
    if q.dim() != 3 or q.shape[2] != 128 or q.dtype != torch.bfloat16 or not q.is_contiguous():
        raise ValueError("q must be a contiguous bf16 [B, H, 128] tensor")
    if k_codes.dim() != 4 or k_codes.shape[3] != 128:
        raise ValueError("k_codes must be [B, T, KVH, 128]")
    B, H, _ = q.shape
    _, T, KVH, _ = k_codes.shape
    for t, shape, dt in ((v_codes, (B, T, KVH, 128), torch.uint8), (k_codes, (B, T, KVH, 128), torch.uint8),
                         (k_scale_inv, (B, T, KVH), torch.float32),
                         (v_scale_inv, (B, T, KVH), torch.float32), (seq_lens, (B,), torch.int32)):
        if tuple(t.shape) != shape or t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"expected a contiguous {dt} tensor of shape {shape}")
    if out is None:
        out = torch.empty((B, H, 128), dtype=torch.bfloat16, device=q.device)
    if split_tokens is not None:
        need = attention_decode_workspace_size(B, H, KVH, T, split_tokens)
        if workspace is None:
            workspace = torch.empty((max(need, 4),), dtype=torch.uint8, device=q.device)
        nbytes = workspace.numel() * workspace.element_size()
        _check(load().fp8_attention_decode_split(
            B, H, KVH, T, _ptr(q), _ptr(k_codes), _ptr(k_scale_inv), _ptr(v_codes),
            _ptr(v_scale_inv), _ptr(seq_lens), float(sm_scale), fmt, int(split_tokens),
            _ptr(workspace), nbytes, _ptr(out), _stream(stream)), "fp8_attention_decode_split")
        return out
    _check(load().fp8_attention_decode(B, H, KVH, T, _ptr(q), _ptr(k_codes), _ptr(k_scale_inv),
                                       _ptr(v_codes), _ptr(v_scale_inv), _ptr(seq_lens),
                                       float(sm_scale), fmt, _ptr(out), _stream(stream)),
           "fp8_attention_decode")
    return out


def decode_split_tokens(B: int, KVH: int, T: int, target_workgroups: int = 512) -> int | None:
    """Chunk size for fp8_attention_decode_split, or None (unsplit) when the B * KVH
    (sequence, KV head) workgroups already give every CU two: otherwise enough chunks of a
    multiple of 256 tokens to reach about target_workgroups.  (Measured on the Llama-3.1-8B
    attention shape with a 4096-token cache: 64 sequences unsplit 128 us against 138 us in
    2048-token chunks; 16 sequences 82 us unsplit, 38 us in 1024-token chunks; 4 sequences
    72 us unsplit, 29 us in 512- or 256-token chunks.)"""
    groups = B * KVH
    if groups <= 0 or T <= 0 or groups >= target_workgroups:
        return None
    splits = -(-target_workgroups // groups)
    chunk = -(-T // splits)
    return max(256, -(-chunk // 256) * 256)


def attention_decode_workspace_size(B: int, H: int, KVH: int, T: int, chunk: int) -> int:
    """Bytes of workspace fp8_attention_decode_split needs (0 for invalid sizes)."""
    return int(load().fp8_attention_decode_workspace_size(B, H, KVH, T, chunk))
