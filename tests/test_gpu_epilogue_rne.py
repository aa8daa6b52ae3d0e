"""The GEMM epilogue rounds the fp32 accumulator to bf16 to nearest, ties to even -- checked bit
for bit ("NVIDIA NeMo RL logra una aceleración del 48% ...", section "El avance técnico": the
linear layers' output stays BF16; round-to-nearest-even is the reading taken for that step).

Every operand value is a small integer (A in {-1, 0, 1}, B in 0..15, exact E4M3 codes) and every
scale a power of two, so each product, each K-block sum on the matrix core (groups of at most
8 integer products of magnitude <= 15 lose nothing), each fold and the accumulator are exact in
fp32: the only rounding left is the bf16 store, and the expected output is the round-to-nearest-
even of the exact fp64 result.  A good share of the exact results fall exactly halfway between
two bf16 values; row 0 (and row 1, negated) holds the sums 257, 259, ..., 383 times a power of two
in block 0, which truncation, rounding half up and ties-to-even all round differently.
Covered: the fold (fp32 block scales), per-tensor scales, E8M0 (power-of-2) scales in the MFMA,
1x128 scales on both operands, the fused output-quantization entry point, the grouped GEMM,
every layout and every tile configuration.
"""
import math
import struct

import numpy as np
import pytest
import torch

import block_scaled_quantize_amd as bsq
import oracle
from helpers import assert_bytes_equal, bits, f32_bits, gpu_scales_to_logical, logical_to_gpu_scales

FP, DG, WG = bsq.FPROP, bsq.DGRAD, bsq.WGRAD
B1, B128, PT = bsq.BLOCK_1x128, bsq.BLOCK_128x128, bsq.PER_TENSOR
E4 = bsq.E4M3


def rne_bf16_bits(values) -> np.ndarray:
    """bf16 bit patterns of exact (fp64) values: the nearest value with an 8-bit significand,
    ties to the even significand (normal range only; zero keeps its sign)."""
    out = []
    for x in np.asarray(values, dtype=np.float64).reshape(-1):
        if x == 0.0:
            out.append(0x8000 if math.copysign(1.0, x) < 0 else 0)
            continue
        m, e = math.frexp(abs(x))            # |x| = m 2^e, 0.5 <= m < 1
        q = math.ldexp(m, 8)                 # significand scaled to [128, 256)
        lo = math.floor(q)
        rest = q - lo
        if rest > 0.5 or (rest == 0.5 and lo % 2 == 1):
            lo += 1
        v = math.ldexp(lo, e - 8)            # exactly representable in bf16 (and fp32)
        b = struct.unpack("<I", struct.pack("<f", v))[0] >> 16
        out.append(b | (0x8000 if x < 0 else 0))
    return np.array(out, dtype=np.uint16).reshape(np.shape(values))


def is_tie(values) -> np.ndarray:
    v = np.abs(np.asarray(values, dtype=np.float64))
    m, e = np.frexp(v)
    q = np.ldexp(m, 8)
    return (v != 0) & (q - np.floor(q) == 0.5)


def test_rne_reference_matches_library_cast():
    """CPU pin of the reference rounding: torch's fp32 -> bf16 cast (round to nearest even) on
    random fp32 values, values halfway between bf16 neighbours and their fp32 neighbours."""
    rng = np.random.default_rng(1)
    mant = rng.integers(0, 1 << 7, size=4000).astype(np.uint32)
    exps = rng.integers(100, 150, size=4000).astype(np.uint32)
    sign = rng.integers(0, 2, size=4000).astype(np.uint32)
    halves = (sign << 31) | (exps << 23) | (mant << 16) | 0x8000     # exactly halfway
    near = np.concatenate([halves, halves + 1, halves - 1,
                           rng.integers(0x00800000, 0x7F000000, size=4000).astype(np.uint32)])
    x = near.view(np.float32)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(rne_bf16_bits(x.astype(np.float64)), want)
    assert is_tie(x[:4000].astype(np.float64)).all()


# ----------------------------------------------------------------------------- operands

M, N, K = 320, 272, 256


def logical_operands(seed: int):
    """Logical A[M,K] in {-1,0,1} and B[N,K] in 0..15 with the tie rows described above."""
    rng = np.random.default_rng(seed)
    # mostly +1, so that most sums exceed 256 in magnitude (where bf16 steps exceed 1)
    a = rng.choice(np.array([-1.0, 0.0, 1.0]), size=(M, K), p=[0.15, 0.25, 0.6])
    b = rng.integers(0, 16, size=(N, K)).astype(np.float64)
    a[0, :128], a[0, 128:] = 1.0, 0.0
    a[1, :128], a[1, 128:] = -1.0, 0.0
    for n in range(64):
        b[n, :128] = 2.0
        b[n, :2 * n + 1] = 3.0                 # block-0 sum of rows 0 / 1: +-(257 + 2n)
    return a, b


def scales(gran, rows, cols, rng, lo, hi):
    """Power-of-two scales in the oracle's logical layout of a stored [rows, cols] matrix."""
    shape = {B1: (rows, -(-cols // 128)), B128: (-(-rows // 128), -(-cols // 128)), PT: (1, 1)}[gran]
    return np.exp2(rng.integers(lo, hi + 1, size=shape)).astype(np.float32)


def stored(layout, a, b):
    """The stored matrices of a layout for C = a . b^T."""
    if layout == FP:
        return a, b
    if layout == DG:
        return a, np.ascontiguousarray(b.T)
    return np.ascontiguousarray(a.T), np.ascontiguousarray(b.T)


def codes(v):
    c = oracle.encode(oracle.E4M3, v.astype(np.float32))
    assert np.array_equal(oracle.decode(oracle.E4M3, c), v)
    return c


def device_codes(q):
    rows, cols = q.shape
    store = torch.zeros((rows, -(-cols // 16) * 16), dtype=torch.uint8)
    store[:, :cols] = torch.from_numpy(q)
    return store.cuda()[:, :cols]


def device_scales(s, gran):
    if gran == PT:
        return torch.from_numpy(s.reshape(1)).cuda()
    return logical_to_gpu_scales(s, gran)


def problem(layout, ga, gb, seed=0):
    a, b = logical_operands(seed)
    sa_, sb_ = stored(layout, a, b)
    qa, qb = codes(sa_), codes(sb_)
    rng = np.random.default_rng(seed + 100)
    sa = scales(ga, *qa.shape, rng, -2, 2)
    sb = scales(gb, *qb.shape, rng, -1, 1)
    exact = oracle.gemm(layout, qa, oracle.E4M3, ga, sa, qb, oracle.E4M3, gb, sb)
    assert np.all(np.abs(exact) < 2.0 ** 16)
    assert int(is_tie(exact).sum()) >= 1000, "too few ties to test the rounding"
    return qa, sa, qb, sb, exact


def check_bits(c, exact, what):
    got = c.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    want = rne_bf16_bits(exact)
    bad = np.argwhere(got != want)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} outputs differ from RNE, first {i}: exact "
                             f"{exact[i]!r} got 0x{got[i]:04x} want 0x{want[i]:04x}")


# ----------------------------------------------------------------------------- GPU

@pytest.mark.gpu
@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("layout,ga,gb", [(FP, B1, B128), (DG, B1, B128), (WG, B128, B128),
                                          (FP, PT, PT), (DG, PT, PT), (WG, PT, PT),
                                          (FP, B1, B1), (FP, B128, PT), (WG, PT, B128)])
def test_gemm_output_is_rne(gpu, layout, ga, gb, pow2):
    qa, sa, qb, sb, exact = problem(layout, ga, gb)
    c = gpu.gemm_blockscaled(layout, device_codes(qa), E4, ga, device_scales(sa, ga),
                             device_codes(qb), E4, gb, device_scales(sb, gb), pow2=pow2)
    torch.cuda.synchronize()
    check_bits(c, exact, f"layout {layout} scales {ga}/{gb} pow2 {pow2}")


@pytest.mark.gpu
@pytest.mark.parametrize("tile", [bsq.TILE_256x128_W4, bsq.TILE_256x128_W8, bsq.TILE_256x256_W8,
                                  bsq.TILE_128x128_W4])
def test_every_tile_output_is_rne(gpu, tile):
    for layout, ga, gb in [(FP, B1, B128), (DG, B1, B128), (WG, PT, PT)]:
        qa, sa, qb, sb, exact = problem(layout, ga, gb, seed=tile)
        for pow2 in (False, True):
            c = gpu.gemm_blockscaled(layout, device_codes(qa), E4, ga, device_scales(sa, ga),
                                     device_codes(qb), E4, gb, device_scales(sb, gb), pow2=pow2,
                                     tile=tile)
            torch.cuda.synchronize()
            check_bits(c, exact, f"tile {tile} layout {layout} pow2 {pow2}")


@pytest.mark.gpu
@pytest.mark.parametrize("ga,gb,pow2_in", [(B1, B128, False), (B1, B128, True), (PT, PT, False)])
def test_fused_quantized_output_rne(gpu, ga, gb, pow2_in):
    """fp8_gemm_blockscaled_qout: the bf16 output is the RNE of the exact result, and the fused
    codes and scales are the oracle's 1x128 quantization of exactly that bf16 matrix."""
    qa, sa, qb, sb, exact = problem(FP, ga, gb, seed=3)
    c, cq, cqs = gpu.gemm_blockscaled_qout(device_codes(qa), ga, device_scales(sa, ga),
                                           device_codes(qb), gb, device_scales(sb, gb),
                                           bsq.SCALE_FP32, pow2_in)
    torch.cuda.synchronize()
    check_bits(c, exact, f"qout {ga}/{gb} pow2 {pow2_in}")
    want_bf16 = rne_bf16_bits(exact)
    qo, so = oracle.quantize_blockwise(want_bf16, oracle.E4M3, oracle.BLOCK_1x128, oracle.SCALE_FP32)
    assert_bytes_equal(cq.cpu().numpy(), qo, "fused codes")
    assert_bytes_equal(f32_bits(gpu_scales_to_logical(cqs, B1)), f32_bits(so), "fused scales")


@pytest.mark.gpu
@pytest.mark.parametrize("pow2", [False, True])
def test_grouped_output_is_rne(gpu, pow2):
    """Grouped GEMM over 3 experts (rows 0..99, none, 100..319): each expert's weight is B with
    its own power-of-two scales."""
    a, b = logical_operands(5)
    qa = codes(a)
    rng = np.random.default_rng(7)
    sa = scales(B1, M, K, rng, -2, 2)
    off = np.array([0, 100, 100, M], dtype=np.int64)
    qbs = np.stack([codes(np.roll(b, g, axis=0)) for g in range(3)])
    sbs = np.stack([scales(B128, N, K, rng, -1, 1) for _ in range(3)])
    exact = oracle.grouped_gemm(off, qa, sa, oracle.E4M3, qbs, sbs, oracle.E4M3)
    assert int(is_tie(exact).sum()) >= 1000
    c = gpu.grouped_gemm(torch.from_numpy(off).cuda(), device_codes(qa), logical_to_gpu_scales(sa, B1),
                         torch.from_numpy(qbs).cuda(), torch.from_numpy(sbs).cuda(), pow2=pow2)
    torch.cuda.synchronize()
    check_bits(c, exact, f"grouped pow2 {pow2}")
