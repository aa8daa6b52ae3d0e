"""Shared helpers for the GPU parity tests (comparison utilities; no method arithmetic)."""
import numpy as np
import torch

import oracle


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 numpy array of its bit patterns (CPU copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f32_bits(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32)


def gpu_scales_to_logical(s: torch.Tensor, gran: int) -> np.ndarray:
    """C ABI scale layout -> the oracle's logical [block row][block column] layout."""
    a = s.detach().cpu().numpy()
    if gran == oracle.BLOCK_1x128:
        return np.ascontiguousarray(a.T)      # [C/128][R] -> [R][C/128]
    return a


def logical_to_gpu_scales(s: np.ndarray, gran: int, device="cuda") -> torch.Tensor:
    if gran == oracle.BLOCK_1x128:
        s = np.ascontiguousarray(np.asarray(s, dtype=np.float32).T)
    return torch.from_numpy(np.ascontiguousarray(s, dtype=np.float32)).to(device)


def assert_bytes_equal(got: np.ndarray, want: np.ndarray, what: str):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    bad = np.nonzero(got.reshape(-1) != want.reshape(-1))[0]
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} mismatches, first at flat index {i}: "
                             f"got {got.reshape(-1)[i]!r} want {want.reshape(-1)[i]!r}")


def nan_aware_equal_f32(got, want) -> bool:
    g, w = np.asarray(got, np.float32), np.asarray(want, np.float32)
    both_nan = np.isnan(g) & np.isnan(w)
    return bool(np.all(both_nan | (f32_bits(g) == f32_bits(w))))


def gemm_check(c_gpu: torch.Tensor, ref: np.ndarray, absmag: np.ndarray, what: str,
               gate: float = 1e-2, alarm: float = 4e-3):
    """Tolerance of a bf16-output block-scaled GEMM against the fp64 reference.

    * relative Frobenius error <= gate (1e-2) and <= alarm (4e-3; bf16 output rounding alone
      gives about 1e-3);
    * every element within one bf16 rounding (2^-8 relative) of the reference plus 2^-12 of the
      sum of |products|.  The second term covers the accumulation inside one FP8 MFMA: the
      hardware sums a 128-product K block with less than fp32 precision (measured at about
      5e-5 of the sum of |products| on gfx950, against about 1e-7 for exact fp32 rounding)."""
    c = c_gpu.detach().float().cpu().numpy().astype(np.float64)
    assert c.shape == ref.shape, f"{what}: shape {c.shape} vs {ref.shape}"
    assert np.all(np.isfinite(c)), f"{what}: non-finite output"
    err = oracle.rel_frobenius(c, ref)
    assert err <= gate, f"{what}: rel Frobenius {err:.3e} > {gate}"
    assert err <= alarm, f"{what}: rel Frobenius {err:.3e} above the {alarm} alarm"
    tol = np.abs(ref) * 2.0 ** -8 + absmag * 2.0 ** -12 + 1e-30
    bad = np.abs(c - ref) > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance, first {tuple(i)}: "
                             f"got {c[tuple(i)]} want {ref[tuple(i)]} tol {tol[tuple(i)]}")
    return err


def abs_product(layout, ad: np.ndarray, bd: np.ndarray) -> np.ndarray:
    """sum_k |a||b| per output element (scale of the accumulation error)."""
    a, b = np.abs(ad), np.abs(bd)
    if layout == oracle.FPROP:
        return a @ b.T
    if layout == oracle.DGRAD:
        return a @ b
    return a.T @ b
