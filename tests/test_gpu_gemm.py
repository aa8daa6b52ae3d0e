"""GPU parity of the block-scaled FP8 GEMM (dense and grouped) against the oracle's fp64
reference: rel. Frobenius <= 1e-2 (gate) and <= 4e-3 (alarm), and every element within one bf16
rounding plus the fp32-accumulation bound (see helpers.gemm_check).

The operand codes and scales are produced by the ORACLE quantizer from seeded synthetic bf16
data, so these tests exercise the GEMM alone.  Layouts: fprop, dgrad, wgrad; scales: 1x128 on
the activation side, 128x128 tiles on the weight side, or per tensor; formats E4M3 / E5M2 mixed
("NVIDIA NeMo RL logra una aceleración del 48% ...", section "El avance técnico";
"Infraestructura de Entrenamiento FP8 ...", section "El panorama de la precisión numérica").
"""
import numpy as np
import pytest
import torch

import block_scaled_quantize_amd as bsq
import oracle
import synth
from helpers import abs_product, gemm_check, logical_to_gpu_scales

pytestmark = pytest.mark.gpu

FP, DG, WG = bsq.FPROP, bsq.DGRAD, bsq.WGRAD
B1, B128, PT = bsq.BLOCK_1x128, bsq.BLOCK_128x128, bsq.PER_TENSOR
E4, E5 = bsq.E4M3, bsq.E5M2


def quantize_operand(x: torch.Tensor, fmt, gran, mode=oracle.SCALE_FP32):
    """Oracle quantization of a stored bf16 matrix; returns (codes, logical scales)."""
    if gran == PT:
        st = oracle.DelayedState(1)
        from helpers import bits
        b = bits(x)
        oracle.delayed_step(b, fmt, mode, 0, st)       # calibrate on x itself
        q, siu = oracle.delayed_step(b, fmt, mode, 0, st)
        return q, np.array([[siu]], dtype=np.float32)
    from helpers import bits
    return oracle.quantize_blockwise(bits(x), fmt, gran, mode)


def to_device_codes(q: np.ndarray, ld: int) -> torch.Tensor:
    rows, cols = q.shape
    store = torch.full((rows, ld), 0x7F, dtype=torch.uint8)     # NaN codes in the padding
    store[:, :cols] = torch.from_numpy(q)
    return store.cuda()[:, :cols]


def device_scales(s: np.ndarray, gran) -> torch.Tensor:
    if gran == PT:
        return torch.from_numpy(s.reshape(1).astype(np.float32)).cuda()
    return logical_to_gpu_scales(s, gran)


TILES = {"A": bsq.TILE_256x128_W4, "B": bsq.TILE_256x128_W8, "C": bsq.TILE_256x256_W8,
         "D": bsq.TILE_128x128_W4}


def run_gemm(gpu, layout, M, N, K, fa, ga, fb, gb, seed=0, pad=0, rows=None, c_guard=True,
             pow2=False, tile=0):
    """pow2: power-of-2 scales (SCALE_POW2 quantization) through fp8_gemm_blockscaled_pow2."""
    mode = oracle.SCALE_POW2 if pow2 else oracle.SCALE_FP32
    ashape = (M, K) if layout != WG else (K, M)
    bshape = (N, K) if layout == FP else (K, N)
    a = synth.activations_with_outliers(*ashape, seed, f"gemm/A{layout}") if ga == B1 else \
        synth.normal(ashape, 1.0, seed, f"gemm/A{layout}")
    b = synth.normal(bshape, 0.02, seed, f"gemm/B{layout}")
    qa, sa = quantize_operand(a, fa, ga, mode)
    qb, sb = quantize_operand(b, fb, gb, mode)
    lda = -(-ashape[1] // 16) * 16 + pad
    ldb = -(-bshape[1] // 16) * 16 + pad
    ad, bd = to_device_codes(qa, lda), to_device_codes(qb, ldb)
    ldc = -(-N // 2) * 2 + (8 if c_guard else 0)   # even pitch; N odd exercises 2-byte stores
    cstore = torch.full((M + 1, ldc), -7.0, dtype=torch.bfloat16, device="cuda")
    c = cstore[:M, :N]
    gpu.gemm_blockscaled(layout, ad, fa, ga, device_scales(sa, ga), bd, fb, gb,
                         device_scales(sb, gb), c=c, pow2=pow2, tile=tile)
    torch.cuda.synchronize()
    if c_guard:
        assert torch.all(cstore[:M, N:] == -7.0) and torch.all(cstore[M] == -7.0), "guard overwritten"
    # reference on all rows or on a sample of output rows
    adq = oracle.dequantize(qa, fa, ga, sa)
    bdq = oracle.dequantize(qb, fb, gb, sb)
    if rows is not None:
        if layout == WG:
            adq = adq[:, rows]
        else:
            adq = adq[rows]
        cg = c[torch.as_tensor(rows, device="cuda")]
    else:
        cg = c
    if layout == FP:
        ref = adq @ bdq.T
    elif layout == DG:
        ref = adq @ bdq
    else:
        ref = adq.T @ bdq
    return gemm_check(cg, ref, abs_product(layout, adq, bdq), f"layout {layout} {M}x{N}x{K}")


def test_tiny_config(gpu):
    # X[64,256] ~ N(0,1) 1x128, W[256,256] ~ N(0,0.02) 128x128, Y = X W^T
    x = synth.normal((64, 256), 1.0, 0, "tiny/X")
    w = synth.normal((256, 256), 0.02, 0, "tiny/W")
    qa, sa = quantize_operand(x, E4, B1)
    qb, sb = quantize_operand(w, E4, B128)
    c = gpu.gemm_blockscaled(FP, torch.from_numpy(qa).cuda(), E4, B1, device_scales(sa, B1),
                             torch.from_numpy(qb).cuda(), E4, B128, device_scales(sb, B128))
    adq, bdq = oracle.dequantize(qa, E4, B1, sa), oracle.dequantize(qb, E4, B128, sb)
    gemm_check(c, adq @ bdq.T, abs_product(FP, adq, bdq), "tiny")


SHAPES = [(64, 128, 128), (300, 260, 200), (129, 384, 512), (1000, 1000, 1000), (4160, 256, 384),
          (1, 129, 33), (255, 127, 129)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_fprop_block_scales(gpu, M, N, K):
    run_gemm(gpu, FP, M, N, K, E4, B1, E4, B128)


@pytest.mark.parametrize("M,N,K", SHAPES[:4])
@pytest.mark.parametrize("ga,gb", [(PT, PT), (B1, PT), (PT, B128), (B128, B128)])
def test_fprop_other_scale_kinds(gpu, M, N, K, ga, gb):
    run_gemm(gpu, FP, M, N, K, E4, ga, E4, gb)


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("fa,ga,fb,gb", [(E5, B1, E4, B128), (E5, PT, E4, PT), (E4, B128, E5, PT)])
def test_dgrad(gpu, M, N, K, fa, ga, fb, gb):
    run_gemm(gpu, DG, M, N, K, fa, ga, fb, gb)


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("fa,ga,fb,gb", [(E5, PT, E4, PT), (E4, B128, E4, B128), (E5, PT, E5, B128)])
def test_wgrad(gpu, M, N, K, fa, ga, fb, gb):
    run_gemm(gpu, WG, M, N, K, fa, ga, fb, gb)


def test_padded_pitches_with_nan_padding(gpu):
    # the padding bytes hold NaN codes: they must never enter the sums
    run_gemm(gpu, FP, 200, 200, 200, E4, B1, E4, B128, pad=48)
    run_gemm(gpu, DG, 200, 200, 200, E5, B1, E4, B128, pad=32)
    run_gemm(gpu, WG, 200, 200, 200, E5, PT, E4, PT, pad=16)


def test_k_zero_and_empty(gpu):
    a = torch.zeros((5, 0), dtype=torch.uint8, device="cuda")
    b = torch.zeros((7, 0), dtype=torch.uint8, device="cuda")
    s = torch.ones(1, device="cuda")
    c = torch.full((5, 8), 3.0, dtype=torch.bfloat16, device="cuda")[:, :7]
    gpu.gemm_blockscaled(FP, a, E4, PT, s, b, E4, PT, s, c=c)
    assert torch.all(c == 0)
    e = torch.zeros((0, 16), dtype=torch.uint8, device="cuda")
    out = gpu.gemm_blockscaled(FP, e, E4, PT, s, torch.zeros((4, 16), dtype=torch.uint8, device="cuda"), E4, PT, s)
    assert out.shape == (0, 4)


@pytest.mark.parametrize("name,N,K", [("qkv", 6144, 4096), ("down", 4096, 14336)])
def test_llama8b_fprop_full_size_sampled_rows(gpu, name, N, K):
    """M = 8192 tokens, the launch configuration the benchmark times; 192 sampled rows are
    checked against the fp64 reference."""
    rows = np.sort(np.random.Generator(np.random.PCG64(1)).choice(8192, 192, replace=False))
    run_gemm(gpu, FP, 8192, N, K, E4, B1, E4, B128, rows=rows, c_guard=False)


def test_llama8b_backward_full_size_sampled(gpu):
    rows = np.sort(np.random.Generator(np.random.PCG64(2)).choice(4096, 128, replace=False))
    run_gemm(gpu, DG, 8192, 4096, 4096, E5, PT, E4, PT, rows=rows * 2, c_guard=False)
    run_gemm(gpu, WG, 4096, 4096, 8192, E5, PT, E4, PT, rows=rows, c_guard=False)


def test_deterministic(gpu):
    qa = torch.randint(0, 0x7E, (512, 1024), dtype=torch.uint8, device="cuda")
    qb = torch.randint(0, 0x7E, (768, 1024), dtype=torch.uint8, device="cuda")
    sa = torch.rand((8, 512), device="cuda") + 0.5
    sb = torch.rand((6, 8), device="cuda") + 0.5
    c1 = gpu.gemm_blockscaled(FP, qa, E4, B1, sa, qb, E4, B128, sb)
    c2 = gpu.gemm_blockscaled(FP, qa, E4, B1, sa, qb, E4, B128, sb)
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


# ----------------------------------------------------------------------------- grouped

def run_grouped(gpu, counts, N, K, seed=0, sample_rows=None, pow2=False, tile=0):
    mode = oracle.SCALE_POW2 if pow2 else oracle.SCALE_FP32
    counts = np.asarray(counts, dtype=np.int64)
    G = len(counts)
    off = synth.offsets_from_counts(counts)
    total = int(off[-1])
    x = synth.normal((total, K), 1.0, seed, "grouped/A")
    qa, sa = quantize_operand(x, E4, B1, mode)
    qbs, sbs = [], []
    for g in range(G):
        w = synth.normal((N, K), 0.02, seed, f"grouped/W{g}")
        q, s = quantize_operand(w, E4, B128, mode)
        qbs.append(q)
        sbs.append(s)
    qbs, sbs = np.stack(qbs), np.stack(sbs)
    c = gpu.grouped_gemm(torch.from_numpy(off).cuda(), torch.from_numpy(qa).cuda(),
                         logical_to_gpu_scales(sa, B1), torch.from_numpy(qbs).cuda(),
                         torch.from_numpy(sbs).cuda(), pow2=pow2, tile=tile)
    torch.cuda.synchronize()
    if sample_rows is None:
        ref = oracle.grouped_gemm(off, qa, sa, E4, qbs, sbs, E4)
        ad = oracle.dequantize(qa, E4, B1, sa)
        mag = np.zeros_like(ref)
        for g in range(G):
            r0, r1 = off[g], off[g + 1]
            if r1 > r0:
                mag[r0:r1] = np.abs(ad[r0:r1]) @ np.abs(oracle.dequantize(qbs[g], E4, B128, sbs[g])).T
        return gemm_check(c, ref, mag, f"grouped {G} groups")
    # sampled rows: the reference of each sampled row uses its own group's weight
    ad = oracle.dequantize(qa[sample_rows], E4, B1, sa[sample_rows])
    grp = np.searchsorted(off, sample_rows, side="right") - 1
    ref = np.zeros((len(sample_rows), N))
    mag = np.zeros_like(ref)
    for g in np.unique(grp):
        wd = oracle.dequantize(qbs[g], E4, B128, sbs[g])
        sel = grp == g
        ref[sel] = ad[sel] @ wd.T
        mag[sel] = np.abs(ad[sel]) @ np.abs(wd).T
    return gemm_check(c[torch.as_tensor(sample_rows, device="cuda")], ref, mag, "grouped sampled")


def test_grouped_small_with_empty_groups(gpu):
    run_grouped(gpu, [5, 0, 130, 1, 0, 257, 128], 256, 384)


def test_grouped_ragged_k_and_n(gpu):
    run_grouped(gpu, [100, 3, 0, 60], 200, 272)


def test_grouped_moe_config_sampled(gpu):
    """128 experts, 16384 tokens, top-8 Zipf(1.1) routing -> 131072 rows, gate/up 2048 -> 1536."""
    counts = synth.moe_routing(16384, 128, 8, 1.1, 0)
    rows = np.sort(np.random.Generator(np.random.PCG64(3)).choice(int(counts.sum()), 256, replace=False))
    run_grouped(gpu, counts, 1536, 2048, sample_rows=rows)


@pytest.mark.parametrize("raw", [[40, 100, 50, 300, 250, 480, -5, 470],
                                 [0, 100, 50, 300, 900, 250, -5, 470]])
@pytest.mark.parametrize("pow2", [False, True])
def test_grouped_offsets_out_of_order(gpu, raw, pow2):
    """Offsets that decrease or leave [0, total_M] are read as e[g] = min(max(offsets[0..g], 0),
    total_M): groups never overlap, rows outside [e[0], e[G]) keep their contents, and the
    result is the same on every run (no two workgroups write one row)."""
    M, N, K = 600, 256, 256
    mode = oracle.SCALE_POW2 if pow2 else oracle.SCALE_FP32
    raw = np.asarray(raw, dtype=np.int64)
    G = len(raw) - 1
    eff = np.minimum(np.maximum.accumulate(np.maximum(raw, 0)), M)
    qa, sa = quantize_operand(synth.normal((M, K), 1.0, 0, "grouped-ooo/A"), E4, B1, mode)
    qbs, sbs = zip(*[quantize_operand(synth.normal((N, K), 0.02, 0, f"grouped-ooo/W{g}"), E4,
                                      B128, mode) for g in range(G)])
    qbs, sbs = np.stack(qbs), np.stack(sbs)
    outs = []
    for _ in range(2):
        c = torch.full((M, N), -7.0, dtype=torch.bfloat16, device="cuda")
        gpu.grouped_gemm(torch.from_numpy(raw).cuda(), torch.from_numpy(qa).cuda(),
                         logical_to_gpu_scales(sa, B1), torch.from_numpy(qbs).cuda(),
                         torch.from_numpy(sbs).cuda(), c=c, pow2=pow2)
        torch.cuda.synchronize()
        outs.append(c)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), "not deterministic"
    c = outs[0]
    lo, hi = int(eff[0]), int(eff[-1])
    assert torch.all(c[:lo] == -7.0) and torch.all(c[hi:] == -7.0), "rows outside the groups written"
    ref = oracle.grouped_gemm(eff, qa, sa, E4, qbs, sbs, E4)
    ad = oracle.dequantize(qa, E4, B1, sa)
    mag = np.zeros_like(ref)
    for g in range(G):
        r0, r1 = int(eff[g]), int(eff[g + 1])
        if r1 > r0:
            mag[r0:r1] = np.abs(ad[r0:r1]) @ np.abs(oracle.dequantize(qbs[g], E4, B128, sbs[g])).T
    gemm_check(c[lo:hi], ref[lo:hi], mag[lo:hi], "grouped, offsets out of order")


def test_wrapper_rejects_bad_tensors(gpu):
    """The Python binding checks shapes, dtypes and strides before calling the library."""
    a = torch.zeros((256, 256), dtype=torch.uint8, device="cuda")
    w = torch.zeros((4, 256, 256), dtype=torch.uint8, device="cuda")
    sa = torch.ones((2, 256), device="cuda")
    sw = torch.ones((4, 2, 2), device="cuda")
    off = torch.tensor([0, 64, 128, 192, 256], dtype=torch.int64, device="cuda")
    with pytest.raises(ValueError):      # experts not N rows apart (a sliced [G, N, K] view)
        gpu.grouped_gemm(off, a, sa, w[:, :128], sw[:, :1])
    with pytest.raises(ValueError):      # offsets need G + 1 entries
        gpu.grouped_gemm(off[:4], a, sa, w, sw)
    with pytest.raises(ValueError):      # K mismatch between a and the experts
        gpu.grouped_gemm(off, a[:, :128], sa, w, sw)
    with pytest.raises(ValueError):      # weight scales of the wrong shape
        gpu.grouped_gemm(off, a, sa, w, sw[:, :, :1])
    with pytest.raises(ValueError):      # activation scales of the wrong dtype
        gpu.grouped_gemm(off, a, sa.double(), w, sw)
    with pytest.raises(ValueError):      # output of the wrong shape
        gpu.grouped_gemm(off, a, sa, w, sw, c=torch.empty((255, 256), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):      # dense: 1x128 scales of the wrong shape
        gpu.gemm_blockscaled(FP, a, E4, B1, sa[:1], a, E4, B128, torch.ones((2, 2), device="cuda"))
    with pytest.raises(ValueError):      # dense: output too small
        gpu.gemm_blockscaled(FP, a, E4, B1, sa, a, E4, B128, torch.ones((2, 2), device="cuda"),
                             c=torch.empty((256, 128), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):      # fused quantization: code output of the wrong shape
        gpu.gemm_blockscaled_qout(a, B1, sa, a, B128, torch.ones((2, 2), device="cuda"),
                                  cq=torch.empty((256, 255), dtype=torch.uint8, device="cuda"))


@pytest.mark.parametrize("variant", ["A", "B", "C", "D"])
@pytest.mark.parametrize("layout,fa,ga,fb,gb", [(FP, E4, B1, E4, B128), (DG, E5, B1, E4, B128),
                                                 (WG, E5, PT, E4, B128)])
def test_every_tile_variant(gpu, variant, layout, fa, ga, fb, gb):
    """Each tile configuration the library can pick (forced through fp8_gemm_blockscaled_tiled)."""
    run_gemm(gpu, layout, 520, 390, 392, fa, ga, fb, gb, tile=TILES[variant])
    run_gemm(gpu, layout, 256, 256, 256, fa, ga, fb, gb, tile=TILES[variant])


@pytest.mark.parametrize("K", [128, 200, 256, 640])
@pytest.mark.parametrize("layout,fa,ga,fb,gb,pow2", [(FP, E4, B1, E4, B128, False),
                                                    (FP, E4, B1, E4, B128, True),
                                                    (DG, E5, PT, E4, PT, False),
                                                    (WG, E5, PT, E4, PT, False)])
def test_dense_persistent_tile_walk(gpu, K, layout, fa, ga, fb, gb, pow2):
    """324 tiles of 256x256 on the persistent grid: a workgroup takes a second tile, formed while
    its first runs (two or more K blocks) or after it (one K block), with the next tile's first
    K block loaded during the current tile's last (two or more K blocks, ragged K included).
    Four sampled rows in each of the 18 tile rows cover every tile."""
    rows = np.array([256 * t + o for t in range(18) for o in (0, 97, 200, 255)])
    run_gemm(gpu, layout, 4608, 4608, K, fa, ga, fb, gb, pow2=pow2, rows=rows)


@pytest.mark.parametrize("K,N", [(128, 256), (256, 384), (208, 256), (640, 512)])
@pytest.mark.parametrize("pow2", [False, True])
def test_grouped_persistent_tiles(gpu, K, N, pow2):
    """More tiles than workgroups: each workgroup walks several tiles of different groups, the
    next tile's first K block loaded while the current tile finishes (K blocks per tile: 1 --
    nothing to overlap --, 2 -- the first block hands over --, 2 with a ragged K, 5)."""
    counts = [3000] * 24 + [17, 0, 700]
    run_grouped(gpu, counts, N, K, seed=K, pow2=pow2)


@pytest.mark.parametrize("G", [300, 1024])
@pytest.mark.parametrize("pow2", [False, True])
def test_grouped_many_groups(gpu, G, pow2):
    """Hundreds of groups, up to the 1024 the kernel allows (the tile's group is found 64 prefix
    entries at a time, so every 64-group chunk of the prefix is searched), many of them empty or
    a few rows long."""
    sizes = [0, 1, 7, 64, 130, 0, 256, 33, 300, 2] if G == 300 else [0, 1, 5, 17, 0, 40, 3, 0]
    counts = [sizes[(g * 7 + g // 5) % len(sizes)] for g in range(G)]
    run_grouped(gpu, counts, 128, 256, seed=G, pow2=pow2)


@pytest.mark.parametrize("variant", ["B", "C", "D"])
def test_grouped_every_tile_variant(gpu, variant):
    """Each tile configuration the grouped kernel can use (forced through fp8_grouped_gemm_tiled)."""
    run_grouped(gpu, [5, 0, 300, 1, 0, 257, 128, 513], 384, 400, tile=TILES[variant])


# ----------------------------------------------------------------------------- power-of-2 scales
# fp8_gemm_blockscaled_pow2 / fp8_grouped_gemm_pow2: power-of-2 scales ("NVIDIA NeMo RL ...",
# section "Por qué esto es importante para la economía de la IA") given to the MFMA as E8M0 block
# scales.  Same oracle and tolerance: a power-of-2 scale is exact in the fp64 reference.

@pytest.mark.parametrize("M,N,K", SHAPES)
def test_pow2_fprop_block_scales(gpu, M, N, K):
    run_gemm(gpu, FP, M, N, K, E4, B1, E4, B128, pow2=True)


@pytest.mark.parametrize("M,N,K", SHAPES[:4])
@pytest.mark.parametrize("layout,fa,ga,fb,gb", [(FP, E4, B1, E4, PT), (FP, E4, PT, E4, B128),
                                                 (FP, E4, PT, E4, PT), (FP, E4, B128, E5, B128),
                                                 (DG, E5, B1, E4, B128), (DG, E5, PT, E4, B128),
                                                 (WG, E5, PT, E4, B128), (WG, E4, B128, E4, B128)])
def test_pow2_layouts_and_scale_kinds(gpu, M, N, K, layout, fa, ga, fb, gb):
    run_gemm(gpu, layout, M, N, K, fa, ga, fb, gb, pow2=True)


def test_pow2_padded_pitches_with_nan_padding(gpu):
    run_gemm(gpu, FP, 200, 200, 200, E4, B1, E4, B128, pad=48, pow2=True)
    run_gemm(gpu, DG, 200, 200, 200, E5, B1, E4, B128, pad=32, pow2=True)


@pytest.mark.parametrize("variant", ["A", "B", "C", "D"])
@pytest.mark.parametrize("layout,fa,ga,fb,gb", [(FP, E4, B1, E4, B128), (DG, E5, B1, E4, B128),
                                                 (WG, E5, PT, E4, B128)])
def test_pow2_every_tile_variant(gpu, variant, layout, fa, ga, fb, gb):
    run_gemm(gpu, layout, 520, 390, 392, fa, ga, fb, gb, pow2=True, tile=TILES[variant])


def test_pow2_llama8b_fprop_full_size_sampled_rows(gpu):
    rows = np.sort(np.random.Generator(np.random.PCG64(4)).choice(8192, 192, replace=False))
    run_gemm(gpu, FP, 8192, 6144, 4096, E4, B1, E4, B128, rows=rows, c_guard=False, pow2=True)


def test_pow2_extreme_exponents(gpu):
    """Scales at the ends of the E8M0 range the quantizers can produce: 2^-127 (the subnormal
    power of two, E8M0 code 0) on one operand and large powers on the other; codes of +-1."""
    M, N, K = 64, 128, 256
    qa = torch.full((M, K), 0x38, dtype=torch.uint8)          # E4M3 1.0
    qa[:, 1::2] = 0xB8                                         # -1.0 on odd k
    qa[::3, :] = 0x38
    qb = torch.full((N, K), 0x38, dtype=torch.uint8)
    sa = np.full((K // 128, M), 2.0 ** 100, dtype=np.float32)
    sa[1, :] = 2.0 ** 60
    sb = np.full((1, K // 128), 2.0 ** -127, dtype=np.float32)
    sb[0, 1] = 2.0 ** -100
    c = gpu.gemm_blockscaled(FP, qa.cuda(), E4, B1, torch.from_numpy(sa).cuda(), qb.cuda(), E4,
                             B128, torch.from_numpy(sb).cuda(), pow2=True)
    ad = oracle.dequantize(qa.numpy(), E4, B1, sa.T)
    bd = oracle.dequantize(qb.numpy(), E4, B128, sb)
    gemm_check(c, ad @ bd.T, np.abs(ad) @ np.abs(bd).T, "pow2 extremes")


def test_pow2_uses_the_exponent_only(gpu):
    """A scale that is not a power of two acts as 2^floor(log2 s): compare with the fp32-scale
    entry given the rounded-down scales."""
    qa = torch.randint(0, 0x7E, (300, 512), dtype=torch.uint8, device="cuda")
    qb = torch.randint(0, 0x7E, (256, 512), dtype=torch.uint8, device="cuda")
    sa = torch.rand((4, 300), device="cuda") * 3 + 0.1
    sb = torch.rand((2, 4), device="cuda") * 3 + 0.1
    down = lambda t: (t.view(torch.int32) & 0x7F800000).view(torch.float32)
    c1 = gpu.gemm_blockscaled(FP, qa, E4, B1, sa, qb, E4, B128, sb, pow2=True).float()
    c2 = gpu.gemm_blockscaled(FP, qa, E4, B1, down(sa), qb, E4, B128, down(sb)).float()
    rel = float(torch.linalg.norm(c1 - c2) / torch.linalg.norm(c2))
    assert rel < 2e-3, rel


def test_pow2_agrees_with_fold_path(gpu):
    """Same power-of-2 inputs through both entry points: equal up to accumulation order."""
    x = synth.activations_with_outliers(1024, 2048, 5, "pow2/agree/X")
    w = synth.normal((768, 2048), 0.02, 5, "pow2/agree/W")
    qa, sa = quantize_operand(x, E4, B1, oracle.SCALE_POW2)
    qb, sb = quantize_operand(w, E4, B128, oracle.SCALE_POW2)
    args = (FP, torch.from_numpy(qa).cuda(), E4, B1, device_scales(sa, B1),
            torch.from_numpy(qb).cuda(), E4, B128, device_scales(sb, B128))
    c1 = gpu.gemm_blockscaled(*args, pow2=True).float()
    c2 = gpu.gemm_blockscaled(*args).float()
    rel = float(torch.linalg.norm(c1 - c2) / torch.linalg.norm(c2))
    assert rel < 2e-3, rel


def test_pow2_grouped_small_with_empty_groups(gpu):
    run_grouped(gpu, [5, 0, 130, 1, 0, 257, 128], 256, 384, pow2=True)


def test_pow2_grouped_moe_config_sampled(gpu):
    counts = synth.moe_routing(16384, 128, 8, 1.1, 0)
    rows = np.sort(np.random.Generator(np.random.PCG64(6)).choice(int(counts.sum()), 256, replace=False))
    run_grouped(gpu, counts, 1536, 2048, sample_rows=rows, pow2=True)


@pytest.mark.parametrize("variant", ["B", "C", "D"])
def test_pow2_grouped_every_tile_variant(gpu, variant):
    run_grouped(gpu, [5, 0, 300, 1, 0, 257, 128, 513], 384, 400, pow2=True, tile=TILES[variant])


# ----------------------------------------------------------------------------- 1x128 x 1x128
# Both operands with 1x128 scales along K (fprop layout): the blockwise weight gradient
# dW = dY^T . X with dY^T and X^T quantized columnwise over tokens ("NVIDIA NeMo RL ...",
# section "El avance técnico": one scale per 128 elements along the contracted dimension).

@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("pow2", [False, True])
def test_fprop_1x128_both_operands(gpu, M, N, K, pow2):
    run_gemm(gpu, FP, M, N, K, E5, B1, E4, B1, pow2=pow2)


@pytest.mark.parametrize("variant", ["A", "B", "C", "D"])
@pytest.mark.parametrize("pow2", [False, True])
def test_1x128_both_every_tile_variant(gpu, variant, pow2):
    run_gemm(gpu, FP, 520, 390, 392, E4, B1, E4, B1, pow2=pow2, tile=TILES[variant])
    run_gemm(gpu, FP, 256, 256, 256, E5, B1, E5, B1, pow2=pow2, tile=TILES[variant])


def wgrad_blockwise(gpu, tokens, n_out, k_in, fdy, pow2, rows=None, seed=0):
    """dW[n_out, k_in] = dY^T . X: both operands quantized columnwise over tokens on the GPU,
    multiplied by the fprop GEMM with 1x128 scales on both sides; checked against the oracle
    (columnwise quantization of the same bf16 tensors, fp64 product)."""
    mode = bsq.SCALE_POW2 if pow2 else bsq.SCALE_FP32
    dy = synth.normal((tokens, n_out), 1e-3, seed, "wgrad/dY")
    x = synth.activations_with_outliers(tokens, k_in, seed, "wgrad/X")
    ld = -(-tokens // 16) * 16                         # GEMM pitch rule: multiple of 16
    dyt = torch.empty((n_out, ld), dtype=torch.uint8, device="cuda")[:, :tokens]
    xt = torch.empty((k_in, ld), dtype=torch.uint8, device="cuda")[:, :tokens]
    _, sdy = gpu.quantize_columnwise_t(dy.cuda(), fdy, mode, qt=dyt)
    _, sx = gpu.quantize_columnwise_t(x.cuda(), E4, mode, qt=xt)
    dw = gpu.gemm_blockscaled(FP, dyt, fdy, B1, sdy, xt, E4, B1, sx, pow2=pow2)
    torch.cuda.synchronize()
    from helpers import bits
    qdy, sdy_o = oracle.quantize_columnwise_t(bits(dy), fdy, mode)
    qx, sx_o = oracle.quantize_columnwise_t(bits(x), E4, mode)
    if rows is not None:
        qdy, sdy_o = qdy[rows], sdy_o[rows]
        dw = dw[torch.as_tensor(rows, device="cuda")]
    a = oracle.dequantize(qdy, fdy, B1, sdy_o)         # dY^T rows
    b = oracle.dequantize(qx, E4, B1, sx_o)            # X^T
    return gemm_check(dw, a @ b.T, np.abs(a) @ np.abs(b).T, f"wgrad {tokens}x{n_out}x{k_in}")


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("fdy", [E4, E5])
def test_blockwise_wgrad_end_to_end(gpu, pow2, fdy):
    wgrad_blockwise(gpu, 1040, 384, 272, fdy, pow2)       # ragged last token block
    wgrad_blockwise(gpu, 300, 130, 200, fdy, pow2)        # ragged everywhere


@pytest.mark.parametrize("pow2", [False, True])
def test_blockwise_wgrad_llama8b_qkv_sampled(gpu, pow2):
    """dW of the qkv layer (6144 x 4096 over 8192 tokens), 128 sampled rows of dW."""
    rows = np.sort(np.random.Generator(np.random.PCG64(7)).choice(6144, 128, replace=False))
    wgrad_blockwise(gpu, 8192, 6144, 4096, E4, pow2, rows=rows)
