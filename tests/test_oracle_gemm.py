"""Pins of the oracle's GEMM reference (dequantize to fp64, then one matrix product).

* Brute force: an exact rational triple loop (Python ``fractions``) over explicit index
  formulas for each layout and each block geometry, on tiny shapes; the fp64 result must agree
  to 1e-12 relative.
* Lossless special case: grid values with unit scales reduce to a plain matrix product of the
  original values.
* Scale equivariance: multiplying a scale array by 2^j multiplies C by 2^j exactly.
The FP8 linear layer (GEMM in FP8 with the 1x128 / 128x128 scales applied, fp32 accumulation,
bf16 output) is the one of "NVIDIA NeMo RL logra una aceleración del 48% ...", section
"El avance técnico".
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

E4M3, E5M2 = oracle.E4M3, oracle.E5M2
B1, B128, PT = oracle.BLOCK_1x128, oracle.BLOCK_128x128, oracle.PER_TENSOR
FPROP, DGRAD, WGRAD = oracle.FPROP, oracle.DGRAD, oracle.WGRAD


def rand_codes(g, shape, fmt):
    t = oracle.decode_table(fmt)
    fin = np.array([c for c in range(256) if np.isfinite(t[c])], dtype=np.uint8)
    return g.choice(fin, size=shape)


def rand_scales(g, rows, cols, gran):
    if gran == B1:
        shp = (rows, -(-cols // 128))
    elif gran == B128:
        shp = (-(-rows // 128), -(-cols // 128))
    else:
        shp = (1, 1)
    e = g.integers(-12, 4, size=shp)
    m = g.uniform(1.0, 2.0, size=shp)
    return (m * 2.0 ** e).astype(np.float32)


def scale_at(s, gran, r, c):
    if gran == B1:
        return s[r, c // 128]
    if gran == B128:
        return s[r // 128, c // 128]
    return s[0, 0]


def brute(layout, qa, fa, ga, sa, qb, fb, gb, sb):
    ta, tb = oracle.decode_table(fa), oracle.decode_table(fb)
    A = [[Fraction(float(ta[qa[i, j]])) * Fraction(float(scale_at(sa, ga, i, j)))
          for j in range(qa.shape[1])] for i in range(qa.shape[0])]
    B = [[Fraction(float(tb[qb[i, j]])) * Fraction(float(scale_at(sb, gb, i, j)))
          for j in range(qb.shape[1])] for i in range(qb.shape[0])]
    if layout == FPROP:     # A[M,K] B[N,K]
        M, K = qa.shape
        N = qb.shape[0]
        C = [[sum(A[m][k] * B[n][k] for k in range(K)) for n in range(N)] for m in range(M)]
        mag = [[sum(abs(A[m][k] * B[n][k]) for k in range(K)) for n in range(N)] for m in range(M)]
    elif layout == DGRAD:   # A[M,K] B[K,N]
        M, K = qa.shape
        N = qb.shape[1]
        C = [[sum(A[m][k] * B[k][n] for k in range(K)) for n in range(N)] for m in range(M)]
        mag = [[sum(abs(A[m][k] * B[k][n]) for k in range(K)) for n in range(N)] for m in range(M)]
    else:                   # A[K,M] B[K,N]
        K, M = qa.shape
        N = qb.shape[1]
        C = [[sum(A[k][m] * B[k][n] for k in range(K)) for n in range(N)] for m in range(M)]
        mag = [[sum(abs(A[k][m] * B[k][n]) for k in range(K)) for n in range(N)] for m in range(M)]
    return np.array(C, dtype=object), np.array(mag, dtype=object)


CASES = [
    (FPROP, (3, 260), (4, 260), B1, B128, E4M3, E4M3),
    (FPROP, (2, 256), (5, 256), B1, B1, E4M3, E5M2),
    (FPROP, (3, 130), (2, 130), PT, PT, E5M2, E4M3),
    (DGRAD, (3, 200), (200, 4), B1, B128, E5M2, E4M3),
    (DGRAD, (2, 140), (140, 3), PT, PT, E5M2, E4M3),
    (WGRAD, (150, 3), (150, 4), PT, PT, E5M2, E4M3),
    (WGRAD, (140, 2), (140, 3), B128, B128, E4M3, E4M3),
]


@pytest.mark.parametrize("layout,sha,shb,ga,gb,fa,fb", CASES)
def test_fp64_reference_vs_exact_brute_force(oracle_lib, layout, sha, shb, ga, gb, fa, fb):
    g = np.random.Generator(np.random.PCG64(11))
    qa, qb = rand_codes(g, sha, fa), rand_codes(g, shb, fb)
    sa, sb = rand_scales(g, *sha, ga), rand_scales(g, *shb, gb)
    got = oracle.gemm(layout, qa, fa, ga, sa, qb, fb, gb, sb)
    C, mag = brute(layout, qa, fa, ga, sa, qb, fb, gb, sb)
    assert got.shape == C.shape
    for idx in np.ndindex(C.shape):
        assert abs(Fraction(float(got[idx])) - C[idx]) <= Fraction(1, 10 ** 12) * (mag[idx] + Fraction(1, 10 ** 300))


def test_lossless_reduces_to_plain_matmul(oracle_lib):
    g = np.random.Generator(np.random.PCG64(12))
    qa, qb = rand_codes(g, (16, 384), E4M3), rand_codes(g, (24, 384), E4M3)
    ta = oracle.decode_table(E4M3)
    ones_a = np.ones((16, 3), np.float32)
    ones_b = np.ones((1, 3), np.float32)
    got = oracle.gemm(FPROP, qa, E4M3, B1, ones_a, qb, E4M3, B128, ones_b)
    assert np.array_equal(got, ta[qa] @ ta[qb].T)


@pytest.mark.parametrize("j", [-5, 3])
def test_scale_equivariance(oracle_lib, j):
    g = np.random.Generator(np.random.PCG64(13))
    qa, qb = rand_codes(g, (8, 256), E4M3), rand_codes(g, (256, 16), E4M3)
    sa, sb = rand_scales(g, 8, 256, B1), rand_scales(g, 256, 16, B128)
    c0 = oracle.gemm(DGRAD, qa, E4M3, B1, sa, qb, E4M3, B128, sb)
    c1 = oracle.gemm(DGRAD, qa, E4M3, B1, sa * np.float32(2.0 ** j), qb, E4M3, B128, sb)
    assert np.array_equal(c1, c0 * 2.0 ** j)


def test_grouped_matches_per_group_brute_force(oracle_lib):
    g = np.random.Generator(np.random.PCG64(14))
    counts = [2, 0, 3, 1]
    off = np.concatenate([[0], np.cumsum(counts)])
    K, N = 256, 3
    qa = rand_codes(g, (off[-1], K), E4M3)
    sa = rand_scales(g, off[-1], K, B1)
    qbs = np.stack([rand_codes(g, (N, K), E4M3) for _ in counts])
    sbs = np.stack([rand_scales(g, N, K, B128) for _ in counts])
    got = oracle.grouped_gemm(off, qa, sa, E4M3, qbs, sbs, E4M3)
    for e in range(len(counts)):
        r0, r1 = off[e], off[e + 1]
        if r1 == r0:
            continue
        C, mag = brute(FPROP, qa[r0:r1], E4M3, B1, sa[r0:r1], qbs[e], E4M3, B128, sbs[e])
        for idx in np.ndindex(C.shape):
            assert abs(Fraction(float(got[r0 + idx[0], idx[1]])) - C[idx]) <= Fraction(1, 10 ** 12) * (mag[idx] + Fraction(1, 10 ** 300))
