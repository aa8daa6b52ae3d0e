"""Pins of the oracle's microscaling (MX) quantizer and GEMM reference.

The pages name MXFP8 block scaling without its block size or scale format ("Infraestructura de
Entrenamiento FP8 ...", sections "Estrategias de escalado y estabilidad" and "Blackwell MXFP8 y
NVFP4: mirando hacia adelante"); the reading is 32-element row blocks with E8M0 scale bytes.
What fixes the expected values (none re-types the oracle's formulas):
* E8M0 bytes against binary32 values built from their exponent fields bit by bit;
* the power-of-2 closed form: each block's maximum lands in [FMAX/2, FMAX];
* the 1x128 power-of-2 quantizer (pinned in test_oracle_quant.py): a row whose four 32-element
  sub-blocks share their maximum quantizes to the same codes and scales under both geometries;
* block independence and clipping of the 32-column geometry;
* special blocks (zero, NaN / Inf) with closed-form results;
* the GEMM reference against a brute-force triple loop over decoded codes and scale bytes.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

E4M3, E5M2 = oracle.E4M3, oracle.E5M2
FMAX = oracle.FMAX


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def test_e8m0_decode_matches_exponent_fields():
    codes = np.arange(256)
    got = oracle.e8m0_decode(codes)
    for c in range(1, 255):
        want = np.array([c << 23], dtype=np.uint32).view(np.float32)[0]   # exponent field c
        assert got[c] == float(want), c
    assert got[0] == float(np.array([0x00400000], dtype=np.uint32).view(np.float32)[0])  # 2^-127
    assert np.isnan(got[255])
    assert np.array_equal(oracle.e8m0_of_pow2(got[:255]), codes[:255].astype(np.uint8))
    with pytest.raises(ValueError):
        oracle.e8m0_of_pow2([3.0])


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_block_max_in_top_octave(oracle_lib, fmt):
    x = synth.activations_with_outliers(37, 300, 0, "oracle/mx/top")   # 300 = 9 blocks + 12
    q, s = oracle.quantize_mx(x, fmt)
    assert q.shape == (37, 300) and s.shape == (37, 10)
    xv = x.float().numpy().astype(np.float64)
    scale = 1.0 / oracle.e8m0_decode(s)                                 # the multiplier s
    for r in range(37):
        for b in range(10):
            blk = np.abs(xv[r, 32 * b:32 * b + 32])
            amax = blk.max()
            assert amax > 0
            assert FMAX[fmt] / 2 < amax * scale[r, b] <= FMAX[fmt], (r, b)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_equal_subblocks_match_1x128(oracle_lib, fmt):
    g = torch.Generator().manual_seed(3)
    x = torch.randn(16, 256, generator=g)
    # give every 32-element sub-block of a 128 block the same maximum magnitude
    for r in range(16):
        for b in range(2):
            m = float(x[r, 128 * b:128 * b + 128].abs().max())
            for sb in range(4):
                c0 = 128 * b + 32 * sb
                k = int(x[r, c0:c0 + 32].abs().argmax())
                x[r, c0 + k] = m if x[r, c0 + k] >= 0 else -m
    xb = x.bfloat16()
    q1, s1 = oracle.quantize_blockwise(xb, fmt, oracle.BLOCK_1x128, oracle.SCALE_POW2)
    qm, sm = oracle.quantize_mx(xb, fmt)
    assert np.array_equal(q1, qm)
    assert np.array_equal(np.repeat(s1.astype(np.float64), 4, axis=1), oracle.e8m0_decode(sm))


def test_blocks_are_independent_and_clipped(oracle_lib):
    x = torch.randn(3, 100).bfloat16()                                   # blocks 32, 32, 32, 4
    q0, s0 = oracle.quantize_mx(x, E4M3)
    y = x.clone()
    y[1, 40] = 1000.0                                                    # block (1, 1) only
    q1, s1 = oracle.quantize_mx(y, E4M3)
    changed = s0 != s1
    assert changed[1, 1] and changed.sum() == 1
    diff = np.argwhere(q0 != q1)
    assert all(r == 1 and 32 <= c < 64 for r, c in diff)
    y = x.clone()
    y[2, 99] = -5000.0                                                   # the 4-element block
    q2, s2 = oracle.quantize_mx(y, E4M3)
    assert (s0 != s2).sum() == 1 and s2[2, 3] != s0[2, 3]


def test_special_blocks(oracle_lib):
    x = torch.zeros(2, 64)
    x[1, 0] = float("nan")
    x[1, 1] = 3.0
    x[1, 40] = float("inf")
    q, s = oracle.quantize_mx(x.bfloat16(), E4M3)
    assert np.all(s == 127)              # zero and non-finite blocks: scale 1
    assert np.all(q[0] == 0)
    assert (q[1, 0] & 0x7F) == 0x7F and q[1, 40] == 0x7E    # NaN code; +Inf saturates to +448
    assert oracle.decode(E4M3, q[1, 1:2])[0] == 3.0


def test_gemm_mx_brute_force(oracle_lib):
    rng = np.random.default_rng(7)
    M, N, K = 3, 4, 70                                   # K: 2 full blocks and one of 6
    qa = rng.integers(0, 0x78, (M, K)).astype(np.uint8) | (rng.integers(0, 2, (M, K)) << 7).astype(np.uint8)
    qb = rng.integers(0, 0x78, (N, K)).astype(np.uint8) | (rng.integers(0, 2, (N, K)) << 7).astype(np.uint8)
    sa = rng.integers(110, 140, (M, 3)).astype(np.uint8)
    sb = rng.integers(110, 140, (N, 3)).astype(np.uint8)
    got = oracle.gemm_mx(qa, E4M3, sa, qb, E4M3, sb)
    da, db = oracle.decode(E4M3, qa), oracle.decode(E4M3, qb)
    want = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += da[m, k] * 2.0 ** (int(sa[m, k // 32]) - 127) * db[n, k] * 2.0 ** (int(sb[n, k // 32]) - 127)
            want[m, n] = acc
    assert np.allclose(got, want, rtol=1e-12, atol=0)


def test_columnwise_mx_is_per_column_row_quantization():
    """Columnwise microscaling on a non-square matrix: column c of x, quantized as one row of
    32-element blocks, gives row c of the transposed codes and scale bytes (a swapped
    orientation would mix columns or fail the shape); the ragged last block of 70 rows is a
    6-element block."""
    x = synth.activations_with_outliers(70, 5, 3, "oracle/mx/colwise")
    xb = bits_of(x)
    q, s = oracle.quantize_mx_columnwise_t(xb, E4M3)
    assert q.shape == (5, 70) and s.shape == (5, 3)
    for c in range(5):
        qc, sc = oracle.quantize_mx(np.ascontiguousarray(xb[:, c][None, :]), E4M3)
        assert np.array_equal(q[c], qc[0]), c
        assert np.array_equal(s[c], sc[0]), c
