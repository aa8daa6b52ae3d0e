"""Pins of the oracle's blockwise quantizer.

What fixes the expected values (none of them re-types the oracle's scale formula):
* the hand-derived worked example in tests/golden/worked_example_1x128.txt;
* closed forms: the block maximum lands on the +-FMAX code (fp32 scales) or in
  [FMAX/2, FMAX] (power-of-2 scales, "Por qué esto es importante para la economía de la IA"
  section of the NeMo RL FP8 article); exact 2^j equivariance; sign symmetry; lossless
  round-trip of grid values; the half-spacing error bound of round-to-nearest;
* block independence (a block's codes and scale depend only on its own elements), which pins
  the 1x128 / 128x128 block geometry of the article's section "El avance técnico";
* special cases with closed-form results (zero, NaN/Inf, bf16-subnormal blocks).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
E4M3, E5M2 = oracle.E4M3, oracle.E5M2
B1, B128 = oracle.BLOCK_1x128, oracle.BLOCK_128x128
FP32, POW2 = oracle.SCALE_FP32, oracle.SCALE_POW2
MAXCODE = {E4M3: 0x7E, E5M2: 0x7B}


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def f32_bits(x) -> int:
    return int(np.float32(x).view(np.uint32))


def read_golden(name):
    d = {}
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            d[k] = [int(t, 16) for t in v]
    return d


@pytest.mark.parametrize("mode", [FP32, POW2])
def test_worked_example(oracle_lib, mode):
    g = read_golden("worked_example_1x128.txt")
    x = np.zeros((1, 128), dtype=np.uint16)
    x[0, :8] = g["input_bf16_hex"]
    q, si = oracle.quantize_blockwise(x, E4M3, B1, mode)
    if mode == FP32:
        assert q[0, :8].tolist() == g["fp32_codes_hex"]
        assert f32_bits(si[0, 0]) == g["fp32_scale_inv_hex"][0]
        assert f32_bits(oracle.scale_from_amax(E4M3, FP32, 3.0)) == g["fp32_scale_hex"][0]
    else:
        assert q[0, :8].tolist() == g["pow2_codes_hex"]
        assert f32_bits(si[0, 0]) == g["pow2_scale_inv_hex"][0]
    assert np.all(q[0, 8:] == 0)


def _blocks(rows, cols, gran):
    bh = 1 if gran == B1 else 128
    for bi in range(0, rows, bh):
        for bj in range(0, cols, 128):
            yield bi // bh, bj // 128, slice(bi, min(bi + bh, rows)), slice(bj, min(bj + 128, cols))


CASES = [(fmt, gran, mode) for fmt in (E4M3, E5M2) for gran in (B1, B128) for mode in (FP32, POW2)]


@pytest.mark.parametrize("fmt,gran,mode", CASES)
def test_block_max_lands_on_top_codes(oracle_lib, fmt, gran, mode):
    x = synth.student_t((256, 384), 3.0, 1, "pin/blockmax")
    xb = bits_of(x)
    q, si = oracle.quantize_blockwise(xb, fmt, gran, mode)
    table = oracle.decode_table(fmt)
    fmax = oracle.FMAX[fmt]
    xf = x.float().numpy()
    for bi, bj, rs, cs in _blocks(256, 384, gran):
        blk = np.abs(xf[rs, cs])
        at_max = blk == blk.max()
        mags = np.abs(table[q[rs, cs]])
        if mode == FP32:
            assert np.all((q[rs, cs][at_max] & 0x7F) == MAXCODE[fmt])
        else:
            assert np.all((mags[at_max] >= fmax / 2) & (mags[at_max] <= fmax))
            m, e = np.frexp(np.float64(si[bi, bj]))
            assert m == 0.5                        # power of two
        assert mags.max() <= fmax


@pytest.mark.parametrize("fmt,gran,mode", CASES)
def test_sign_symmetry_and_pow2_equivariance(oracle_lib, fmt, gran, mode):
    x = synth.normal((200, 300), 1.0, 2, "pin/equiv")
    q, si = oracle.quantize_blockwise(bits_of(x), fmt, gran, mode)
    qn, sin_ = oracle.quantize_blockwise(bits_of(-x), fmt, gran, mode)
    assert np.array_equal(qn, q ^ np.uint8(0x80))
    assert np.array_equal(sin_, si)
    for j in (-20, -3, 1, 7, 30):
        xs = x * (2.0 ** j)                   # exact in bf16 (no over/underflow here)
        assert torch.equal(xs.float() / (2.0 ** j), x.float())
        qs, ss = oracle.quantize_blockwise(bits_of(xs), fmt, gran, mode)
        assert np.array_equal(qs, q)
        assert np.array_equal(ss, (si * np.float32(2.0 ** j)).astype(np.float32))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_lossless_grid_values(oracle_lib, fmt):
    table = oracle.decode_table(fmt)
    fin = np.array([c for c in range(256) if np.isfinite(table[c])])
    g = np.random.Generator(np.random.PCG64(3))
    codes = g.choice(fin, size=(4, 256))
    codes[:, 0] = MAXCODE[fmt]                 # every block holds +FMAX
    codes[:, 128] = MAXCODE[fmt] | 0x80        # ... or -FMAX
    vals = table[codes]
    x = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(x.double().numpy(), vals)          # grid values are bf16-exact
    for mode in (FP32, POW2):
        q, si = oracle.quantize_blockwise(bits_of(x), fmt, B1, mode)
        assert np.all(si == 1.0)
        dq = table[q]
        assert np.array_equal(dq, vals)                       # -0 vs +0 aside, values equal
        assert np.array_equal(np.signbit(dq), np.signbit(vals))


@pytest.mark.parametrize("fmt,gran,mode", CASES)
def test_half_spacing_error_bound(oracle_lib, fmt, gran, mode):
    x = synth.activations_with_outliers(130, 4 * 128 + 40, 4, "pin/err")
    q, si = oracle.quantize_blockwise(bits_of(x), fmt, gran, mode)
    table = oracle.decode_table(fmt)
    mbits = 3 if fmt == E4M3 else 2
    emin = -6 if fmt == E4M3 else -14
    xf = x.float().numpy()
    for bi, bj, rs, cs in _blocks(*xf.shape, gran):
        s = np.float32(1.0) / si[bi, bj]       # the scale is 1/s_inv up to fp32 rounding
        y = (xf[rs, cs] * s).astype(np.float64)
        e = np.maximum(np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** emin))), emin)
        half = 2.0 ** (e - mbits) / 2
        err = np.abs(table[q[rs, cs]] - y)
        # 1/s_inv differs from s by at most 1 ulp: allow that slack on top of half a spacing
        assert np.all(err <= half * (1 + 1e-6) + np.abs(y) * 2.0 ** -22)


@pytest.mark.parametrize("fmt,gran,mode", CASES)
def test_blocks_are_independent_and_clipped(oracle_lib, fmt, gran, mode):
    rows, cols = 131, 300                        # ragged in both dims
    xb = synth.random_bf16_bits((rows, cols), 5, "pin/ragged")
    xb &= np.uint16(0x7FFF)
    xb[xb >= 0x7F80] = 0x3F80                    # finite only here
    neg = synth.random_bf16_bits((rows, cols), 6, "pin/ragged-sign") & np.uint16(0x8000)
    xb |= neg
    q, si = oracle.quantize_blockwise(xb, fmt, gran, mode)
    for bi, bj, rs, cs in _blocks(rows, cols, gran):
        qb, sb = oracle.quantize_blockwise(np.ascontiguousarray(xb[rs, cs]), fmt, gran, mode)
        assert np.array_equal(qb, q[rs, cs])
        assert sb.shape == (1, 1) and sb[0, 0] == si[bi, bj]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_special_blocks(oracle_lib, fmt):
    fmax_code = MAXCODE[fmt]
    x = np.zeros((6, 128), dtype=np.uint16)
    # row 0: all zeros (with a -0): s = 1, codes +-0
    x[0, 5] = 0x8000
    # row 1: a NaN: s = 1; NaN -> 0x7F|sign; 3.0 encodes at s = 1
    x[1, 0] = 0xFFC1
    x[1, 1] = 0x4040
    # row 2: +Inf and -Inf: s = 1, saturate
    x[2, 0] = 0x7F80
    x[2, 1] = 0xFF80
    x[2, 2] = 0xC040
    # row 3: only bf16 subnormals: FMAX/amax overflows -> s = FLT_MAX, s_inv = 1/FLT_MAX
    x[3, 0] = 0x0001
    x[3, 1] = 0x8003
    # row 4: amax = 1.75 * 2^-119 -> s = 2^127 / 1 ... (E4M3: 448/amax = 2^127 exactly)
    x[4, 0] = 0x0460                              # 1.75 * 2^-119
    # row 5: amax = 2^-119: E4M3 scale 1.75 * 2^127 still fits fp32; E5M2's overflows
    x[5, 0] = 0x0400
    x[5, 1] = 0x0001
    q, si = oracle.quantize_blockwise(x, fmt, B1, FP32)
    assert np.all(q[0] == np.where(x[0] == 0x8000, 0x80, 0)) and si[0, 0] == 1.0
    assert q[1, 0] == 0xFF and q[1, 1] == oracle.encode(fmt, np.float32([3.0]))[0]
    assert si[1, 0] == 1.0
    assert q[2, 0] == fmax_code and q[2, 1] == fmax_code | 0x80 and si[2, 0] == 1.0
    assert q[2, 2] == oracle.encode(fmt, np.float32([-3.0]))[0]
    # s = FLT_MAX (3.4028235e38), s_inv = 1/FLT_MAX -> fp32 subnormal 2^-128 = 0x00200000
    assert f32_bits(si[3, 0]) == 0x00200000
    if fmt == E4M3:
        assert f32_bits(si[4, 0]) == 0x00400000     # 2^-127, a subnormal kept as such
        assert q[4, 0] == 0x7E
    if fmt == E4M3:
        assert q[5, 0] == 0x7E                      # s not clamped: block max -> top code
    else:
        assert f32_bits(si[5, 0]) == 0x00200000     # s clamped to FLT_MAX
        assert q[5, 0] == oracle.encode(fmt, np.float32([2.0 ** -119 * np.finfo(np.float32).max]))[0]


def test_pow2_scale_rounds_down(oracle_lib):
    for amax in (1.0, 3.0, 448.0, 449.0, 0.001, 1e-30, 1e30):
        s = oracle.scale_from_amax(E4M3, POW2, amax)
        m, e = np.frexp(np.float64(s))
        assert m == 0.5
        assert s <= np.float32(448.0) / np.float32(amax)
        assert 2 * np.float64(s) > np.float64(np.float32(448.0) / np.float32(amax))


# ----------------------------------------------------------------------------- columnwise (128x1)
# oracle.quantize_columnwise_t: blocks of 128 consecutive rows of one column, codes transposed.
# Pinned by closed forms on the column blocks themselves (the block maximum of every 128x1 block
# lands on the +-FMAX code; each block's codes and scale depend only on that block) -- a wrong
# block axis, a wrong transpose or a wrong ragged tail fails these.

@pytest.mark.parametrize("fmt,mode", [(E4M3, FP32), (E5M2, FP32), (E4M3, POW2)])
def test_columnwise_block_max_on_top_codes(oracle_lib, fmt, mode):
    rows, cols = 300, 70                       # 3 row blocks, the last one ragged (44 rows)
    x = synth.student_t((rows, cols), 3.0, 7, "pin/colwise")
    # give each column its own magnitude so that row-wise blocks would differ from column blocks
    x = (x.float() * torch.logspace(-3, 3, cols, base=2.0)).to(torch.bfloat16)
    qt, si = oracle.quantize_columnwise_t(bits_of(x), fmt, mode)
    assert qt.shape == (cols, rows) and si.shape == (cols, 3)
    table = oracle.decode_table(fmt)
    fmax = oracle.FMAX[fmt]
    xf = x.float().numpy()
    for c in range(cols):
        for rb in range(3):
            rs = slice(128 * rb, min(128 * rb + 128, rows))
            blk = np.abs(xf[rs, c])
            codes = qt[c, rs]                  # transposed: row c of qt holds column c of x
            at_max = blk == blk.max()
            mags = np.abs(table[codes])
            if mode == FP32:
                assert np.all((codes[at_max] & 0x7F) == MAXCODE[fmt])
            else:
                assert np.all((mags[at_max] >= fmax / 2) & (mags[at_max] <= fmax))
            assert mags.max() <= fmax
            # the sign of every nonzero code follows its element
            nz = mags > 0
            assert np.array_equal(np.signbit(table[codes][nz]), np.signbit(xf[rs, c][nz]))


def test_columnwise_blocks_are_independent(oracle_lib):
    rows, cols = 260, 9
    xb = synth.random_bf16_bits((rows, cols), 8, "pin/colwise-ind") & np.uint16(0x7FFF)
    xb[xb >= 0x7F80] = 0x4000
    qt, si = oracle.quantize_columnwise_t(xb, E4M3, FP32)
    # every 128x1 block quantized on its own (as a 1-column matrix) gives the same codes/scale
    for c in range(cols):
        for rb in range(3):
            r0, r1 = 128 * rb, min(128 * rb + 128, rows)
            qb, sb = oracle.quantize_columnwise_t(np.ascontiguousarray(xb[r0:r1, c:c + 1]), E4M3, FP32)
            assert np.array_equal(qb[0], qt[c, r0:r1])
            assert sb.shape == (1, 1) and sb[0, 0] == si[c, rb]
    # changing one column leaves the others untouched
    xb2 = xb.copy()
    xb2[:, 4] = 0x3F80
    qt2, si2 = oracle.quantize_columnwise_t(xb2, E4M3, FP32)
    keep = [c for c in range(cols) if c != 4]
    assert np.array_equal(qt2[keep], qt[keep]) and np.array_equal(si2[keep], si[keep])
