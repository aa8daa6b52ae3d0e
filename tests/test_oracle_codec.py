"""Pins of the oracle's FP8 codec against facts fixed outside the oracle.

* E4M3 reaches +-448 ("Infraestructura de Entrenamiento FP8: Precisión Numérica de Nueva
  Generación", section "El panorama de la precisión numérica"); 4/3 and 5/2 exponent/mantissa
  splits (same section).
* The decode of all 256 codes agrees with PyTorch's own float8_e4m3fn / float8_e5m2 dtypes
  (an independent library implementation of the same OCP formats).
* The encoder agrees, on every fp32 input inside the finite range, with PyTorch's
  round-to-nearest-even cast; outside it, it saturates (a reading) and NaN keeps its sign.
* A brute-force nearest search over the decoded table (a different algorithm from the
  oracle's exponent/quantum arithmetic) agrees on every code midpoint and its neighbours and on
  a random sample.
"""
import math

import numpy as np
import pytest
import torch

import oracle

E4M3, E5M2 = oracle.E4M3, oracle.E5M2
TORCH_DT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}
MAXCODE = {E4M3: 0x7E, E5M2: 0x7B}


def torch_decode(fmt):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(TORCH_DT[fmt]).to(torch.float64).numpy()


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_decode_matches_torch_float8(oracle_lib, fmt):
    ours = oracle.decode_table(fmt)
    ref = torch_decode(fmt)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # signed zero
    assert math.copysign(1.0, ours[0x80]) == -1.0 and math.copysign(1.0, ours[0x00]) == 1.0


def test_e4m3_range_is_448_from_page(oracle_lib):
    t = oracle.decode_table(E4M3)
    fin = t[np.isfinite(t)]
    assert fin.max() == 448.0 and fin.min() == -448.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isfinite(t).sum() == 254                   # only S.1111.111 is NaN, no inf
    assert t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9  # min normal / min subnormal


def test_e5m2_table(oracle_lib):
    t = oracle.decode_table(E5M2)
    assert np.isfinite(t).sum() == 248
    assert t[0x7B] == 57344.0 and t[0x7C] == np.inf and t[0xFC] == -np.inf
    assert all(np.isnan(t[c]) for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))
    assert t[0x04] == 2.0 ** -14 and t[0x01] == 2.0 ** -16


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_table_monotone_symmetric_roundtrip(oracle_lib, fmt):
    t = oracle.decode_table(fmt)
    pos = t[: MAXCODE[fmt] + 1]
    assert np.all(np.diff(pos) > 0)                 # codes 0..max are increasing
    for c in range(128):
        if np.isnan(t[c]):
            continue
        assert t[c | 0x80] == -t[c]
    finite_codes = [c for c in range(256) if np.isfinite(t[c])]
    enc = oracle.encode(fmt, np.array([t[c] for c in finite_codes], dtype=np.float32))
    assert enc.tolist() == finite_codes             # enc(dec(c)) == c, -0 included


def test_tie_and_saturation_examples(oracle_lib):
    e = lambda v: int(oracle.encode(E4M3, np.array([v], dtype=np.float32))[0])
    assert e(17.0) == 0x58          # between 16 and 18: tie to the even code (16)
    assert e(19.0) == 0x5A          # between 18 and 20: tie to the even code (20)
    assert e(2.0 ** -10) == 0x00    # half of the smallest subnormal: ties to zero
    assert e(3 * 2.0 ** -10) == 0x02
    assert e(-(2.0 ** -12)) == 0x80  # negative underflow keeps the sign
    for v in (448.0, 460.0, 464.0, 470.0, 1e30, np.inf):
        assert e(v) == 0x7E and e(-v) == 0xFE
    assert e(np.nan) == 0x7F and e(-np.float32(np.nan)) == 0xFF
    e5 = lambda v: int(oracle.encode(E5M2, np.array([v], dtype=np.float32))[0])
    for v in (57344.0, 61440.0, 1e10, np.inf):
        assert e5(v) == 0x7B and e5(-v) == 0xFB


def _brute_nearest(fmt, x: np.ndarray) -> np.ndarray:
    """Nearest finite table value by search, ties to the even code; saturating; NaN -> 0x7F|s."""
    t = oracle.decode_table(fmt)
    maxc = MAXCODE[fmt]
    vals = t[: maxc + 1]                              # 0 .. +FMAX increasing
    with np.errstate(invalid="ignore"):
        a = np.abs(x.astype(np.float64))
    sign = np.signbit(x).astype(np.int64) << 7
    lo = np.searchsorted(vals, a, side="right") - 1   # vals[lo] <= a
    lo = np.clip(lo, 0, maxc)
    hi = np.minimum(lo + 1, maxc)
    mid = (vals[lo] + vals[hi]) / 2                   # exact in fp64
    code = np.where(a < mid, lo, np.where(a > mid, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(vals[lo] == a, lo, code)
    code = np.where(a > vals[maxc], maxc, code)
    out = (code | sign).astype(np.uint8)
    out = np.where(np.isnan(x), (0x7F | sign).astype(np.uint8), out)
    return out


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encoder_vs_brute_force_midpoints_and_sample(oracle_lib, fmt):
    t = oracle.decode_table(fmt)
    maxc = MAXCODE[fmt]
    pts = []
    for c in range(maxc + 1):
        v = t[c]
        nxt = t[c + 1] if c < maxc else 2 * t[maxc]
        for p in (v, (v + nxt) / 2):
            f = np.float32(p)
            b = f.view(np.uint32)
            for d in range(-3, 4):
                if 0 <= int(b) + d < 0x80000000:
                    pts.append(np.uint32(int(b) + d))
    pts = np.array(pts, dtype=np.uint32)
    rng = np.random.Generator(np.random.PCG64(12345))
    sample = rng.integers(0, 2 ** 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    bits = np.concatenate([pts, pts | np.uint32(0x80000000), sample])
    x = bits.view(np.float32)
    assert np.array_equal(oracle.encode(fmt, x), _brute_nearest(fmt, x))


@pytest.mark.slow
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encoder_exhaustive_vs_torch_cast(oracle_lib, fmt):
    """All 2^31 non-negative fp32 inputs: in-range values equal torch's RNE cast; the rest
    follow the saturation / NaN readings.  The negative half is covered by the sign-symmetry
    check below on a sample (the midpoint test above covers both signs exactly)."""
    fmax = oracle.FMAX[fmt]
    chunk = 1 << 26
    for base in range(0, 1 << 31, chunk):
        bits = np.arange(base, base + chunk, dtype=np.uint64).astype(np.uint32)
        x = bits.view(np.float32)
        ours = oracle.encode_bit_range(fmt, base, chunk)
        ref = torch.from_numpy(x).to(TORCH_DT[fmt]).view(torch.uint8).numpy()
        a = np.abs(x)
        inr = a <= fmax
        bad = np.nonzero(ours[inr] != ref[inr])[0]
        assert bad.size == 0, f"mismatch at bits {bits[inr][bad[:4]]}"
        sign = (bits >> 31).astype(np.uint8) << 7
        over = (a > fmax) & ~np.isnan(x)
        assert np.all(ours[over] == (MAXCODE[fmt] | sign[over]))
        nan = np.isnan(x)
        assert np.all(ours[nan] == (0x7F | sign[nan]))
    rng = np.random.Generator(np.random.PCG64(7))
    pos = rng.integers(0, 2 ** 31, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    neg = pos | np.uint32(0x80000000)
    assert np.array_equal(oracle.encode(fmt, neg.view(np.float32)),
                          oracle.encode(fmt, pos.view(np.float32)) | np.uint8(0x80))
