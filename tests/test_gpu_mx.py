"""Microscaling (MXFP8) path on the GPU against the oracle: fp8_quantize_mx bit for bit (codes
and E8M0 scale bytes, in the C ABI's [ceil(cols/128)][rows][4] layout), fp8_gemm_mx within the
GEMM tolerance of tests/helpers.py on seeded inputs quantized by the oracle (ragged M, N and K;
the scale bytes of chunks past K hold NaN codes, which the kernel must ignore), and the
argument checks that need device memory."""
import numpy as np
import pytest
import torch

import block_scaled_quantize_amd as bsq
import oracle
import synth
from helpers import assert_bytes_equal, gemm_check

pytestmark = pytest.mark.gpu
E4, E5 = oracle.E4M3, oracle.E5M2


def abi_scales(s: np.ndarray, pad: int) -> np.ndarray:
    """The oracle's [rows][ceil(cols/32)] scale bytes in the C ABI layout [ceil(cols/128)][rows][4]
    (chunks past the last one filled with `pad`)."""
    rows, nch = s.shape
    nb = -(-nch // 4)
    full = np.full((rows, nb * 4), pad, dtype=np.uint8)
    full[:, :nch] = s
    return np.ascontiguousarray(full.reshape(rows, nb, 4).transpose(1, 0, 2))


def run_quant(gpu, rows, cols, fmt, x=None, pitch=None, seed=0):
    if x is None:
        x = synth.activations_with_outliers(rows, cols, seed, f"mx/quant/{rows}x{cols}")
    ld = pitch if pitch is not None else cols
    store = torch.zeros((rows, ld), dtype=torch.bfloat16)
    store[:, :cols] = x
    xd = store.cuda()[:, :cols]
    scales = torch.full(bsq.mx_scale_shape(rows, cols), 0xAB, dtype=torch.uint8, device="cuda")
    q, s = gpu.quantize_mx(xd, fmt, scales=scales)
    torch.cuda.synchronize()
    qo, so = oracle.quantize_mx(x, fmt)
    assert_bytes_equal(q.cpu().numpy(), qo, f"codes {rows}x{cols}")
    # (chunks past the matrix are empty blocks: 2^0)
    assert_bytes_equal(s.cpu().numpy(), abi_scales(so, 127), f"scale bytes {rows}x{cols}")


@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 70), (37, 300), (64, 4096), (33, 128), (5, 1)])
@pytest.mark.parametrize("fmt", [E4, E5])
def test_quantize_mx_bit_exact(gpu, rows, cols, fmt):
    run_quant(gpu, rows, cols, fmt)


def test_quantize_mx_pitch(gpu):
    run_quant(gpu, 40, 512, E4, pitch=520)     # 16-byte rows
    run_quant(gpu, 40, 200, E4, pitch=264)


def test_quantize_mx_special_blocks(gpu):
    x = synth.activations_with_outliers(8, 256, 1, "mx/special")
    x[0, :32] = 0.0                                   # zero block
    x[1, 3] = float("nan")                            # NaN block
    x[2, 40] = float("inf")
    x[3, 70] = float("-inf")
    x[4, 96:128] = torch.tensor(1e-40).bfloat16()     # bf16 subnormals: the largest scale
    x[5, 130] = 3.0e38                                # huge magnitude: the smallest scale
    run_quant(gpu, 8, 256, E4, x=x)
    run_quant(gpu, 8, 256, E5, x=x)


def test_quantize_mx_full_size(gpu):
    x = synth.activations_with_outliers(8192, 4096, 0, "bench/8b/qkv/X")
    run_quant(gpu, 8192, 4096, E4, x=x)


@pytest.mark.parametrize("rows,cols", [(1, 1024), (7, 2048), (130, 14336)])
def test_quantize_mx_long_rows(gpu, rows, cols):
    for fmt in (E4, E5):
        run_quant(gpu, rows, cols, fmt)
    run_quant(gpu, rows, cols, E4, pitch=cols + 64)


def test_quantize_mx_beyond_cache_sampled(gpu):
    """Codes larger than the 256 MB last-level cache ([65540, 4096], non-temporal code stores):
    the kernel quantizes the whole tensor, the oracle checks sampled row bands (blocks are per
    row, so a band is checked exactly), the last band ragged."""
    rows, cols = 65540, 4096
    xd = torch.zeros((rows, cols), dtype=torch.bfloat16, device="cuda")
    bands = [(0, 64), (20000, 20064), (rows - 68, rows)]
    host = {}
    for lo, hi in bands:
        t = synth.activations_with_outliers(hi - lo, cols, 3, f"mx/big/{lo}")
        host[lo] = t
        xd[lo:hi] = t.cuda()
    q, s = gpu.quantize_mx(xd, E4)
    torch.cuda.synchronize()
    for lo, hi in bands:
        qo, so = oracle.quantize_mx(host[lo], E4)
        assert_bytes_equal(q[lo:hi].cpu().numpy(), qo, f"codes rows {lo}..{hi}")
        assert_bytes_equal(s[:, lo:hi].cpu().numpy(), abi_scales(so, 127), f"scales rows {lo}..{hi}")
    del xd, q, s
    torch.cuda.empty_cache()


def device_codes(q: np.ndarray, ld: int) -> torch.Tensor:
    rows, cols = q.shape
    store = torch.full((rows, ld), 0x7F, dtype=torch.uint8)      # NaN codes in the padding
    store[:, :cols] = torch.from_numpy(q)
    return store.cuda()[:, :cols]


def device_scale_bytes(s: np.ndarray, k: int) -> torch.Tensor:
    # chunks past K hold the E8M0 NaN byte: the kernel must ignore them
    return torch.from_numpy(abi_scales(s, 0xFF)).cuda()


def run_gemm_mx(gpu, M, N, K, fa=E4, fb=E4, seed=0, rows=None):
    a = synth.activations_with_outliers(M, K, seed, "mx/gemm/A")
    b = synth.normal((N, K), 0.02, seed, "mx/gemm/B")
    qa, sa = oracle.quantize_mx(a, fa)
    qb, sb = oracle.quantize_mx(b, fb)
    ad, bd = device_codes(qa, -(-K // 16) * 16), device_codes(qb, -(-K // 16) * 16 + 16)
    ldc = -(-N // 2) * 2 + 8
    cstore = torch.full((M + 1, ldc), -7.0, dtype=torch.bfloat16, device="cuda")
    c = cstore[:M, :N]
    gpu.gemm_mx(ad, device_scale_bytes(sa, K), bd, device_scale_bytes(sb, K), fa, fb, c=c)
    torch.cuda.synchronize()
    assert torch.all(cstore[:M, N:] == -7.0) and torch.all(cstore[M] == -7.0), "guard overwritten"
    adq = oracle.dequantize(qa, fa, oracle.BLOCK_1x32, oracle.e8m0_decode(sa))
    bdq = oracle.dequantize(qb, fb, oracle.BLOCK_1x32, oracle.e8m0_decode(sb))
    if rows is not None:
        adq = adq[rows]
        c = c[torch.as_tensor(rows, device="cuda")]
    ref = adq @ bdq.T
    return gemm_check(c, ref, np.abs(adq) @ np.abs(bdq).T, f"mx {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(64, 128, 128), (300, 260, 200), (129, 384, 512), (1000, 1000, 1000),
                                   (4160, 256, 384), (256, 256, 160), (100, 300, 96), (17, 33, 32)])
def test_gemm_mx(gpu, M, N, K):
    run_gemm_mx(gpu, M, N, K)


@pytest.mark.parametrize("fa,fb", [(E5, E4), (E4, E5), (E5, E5)])
def test_gemm_mx_formats(gpu, fa, fb):
    run_gemm_mx(gpu, 300, 260, 456, fa, fb)


def test_gemm_mx_matches_oracle_gemm_reference(gpu):
    # the oracle's own microscaling GEMM reference (decoded scale bytes, fp64 product)
    a = synth.activations_with_outliers(64, 256, 3, "mx/ref/A")
    b = synth.normal((128, 256), 0.02, 3, "mx/ref/B")
    qa, sa = oracle.quantize_mx(a, E4)
    qb, sb = oracle.quantize_mx(b, E4)
    c = gpu.gemm_mx(device_codes(qa, 256), device_scale_bytes(sa, 256), device_codes(qb, 256),
                    device_scale_bytes(sb, 256))
    torch.cuda.synchronize()
    ref = oracle.gemm_mx(qa, E4, sa, qb, E4, sb)
    adq = oracle.dequantize(qa, E4, oracle.BLOCK_1x32, oracle.e8m0_decode(sa))
    bdq = oracle.dequantize(qb, E4, oracle.BLOCK_1x32, oracle.e8m0_decode(sb))
    gemm_check(c, ref, np.abs(adq) @ np.abs(bdq).T, "mx vs oracle.gemm_mx")


def test_gemm_mx_full_size_sampled(gpu):
    rows = list(range(0, 8192, 97))
    run_gemm_mx(gpu, 8192, 4096, 4096, rows=rows)


def test_gemm_mx_empty_and_k0(gpu):
    a = torch.zeros((0, 64), dtype=torch.uint8, device="cuda")
    b = torch.zeros((8, 64), dtype=torch.uint8, device="cuda")
    s0 = torch.zeros(bsq.mx_scale_shape(0, 64), dtype=torch.uint8, device="cuda")
    s8 = torch.zeros(bsq.mx_scale_shape(8, 64), dtype=torch.uint8, device="cuda")
    assert gpu.gemm_mx(a, s0, b, s8).shape == (0, 8)
    a = torch.zeros((5, 0), dtype=torch.uint8, device="cuda")
    b = torch.zeros((6, 0), dtype=torch.uint8, device="cuda")
    c = torch.full((5, 6), 3.0, dtype=torch.bfloat16, device="cuda")
    lib = gpu.load()
    sa = torch.zeros((1, 5, 4), dtype=torch.uint8, device="cuda")
    sb = torch.zeros((1, 6, 4), dtype=torch.uint8, device="cuda")
    rc = lib.fp8_gemm_mx(5, 6, 0, a.data_ptr(), 16, E4, sa.data_ptr(), b.data_ptr(), 16, E4,
                         sb.data_ptr(), c.data_ptr(), 6, None)
    torch.cuda.synchronize()
    assert rc == 0 and torch.all(c == 0)


def test_mx_argument_checks(gpu):
    lib = gpu.load()
    a = torch.zeros((64, 128), dtype=torch.uint8, device="cuda")
    s = torch.zeros((1, 64, 4), dtype=torch.uint8, device="cuda")
    c = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    def call(**kw):
        v = dict(M=64, N=64, K=128, A=a.data_ptr(), lda=128, fa=E4, sa=s.data_ptr(),
                 B=a.data_ptr(), ldb=128, fb=E4, sb=s.data_ptr(), C=c.data_ptr(), ldc=64)
        v.update(kw)
        return lib.fp8_gemm_mx(v["M"], v["N"], v["K"], v["A"], v["lda"], v["fa"], v["sa"],
                               v["B"], v["ldb"], v["fb"], v["sb"], v["C"], v["ldc"], None)
    assert call() == bsq.OK
    torch.cuda.synchronize()
    assert call(fa=3) == bsq.ERR_ARG
    assert call(sa=s.data_ptr() + 2) == bsq.ERR_ALIGN
    assert call(sa=None) == bsq.ERR_NULL
    assert call(lda=100) == bsq.ERR_SHAPE
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((4, 64), dtype=torch.uint8, device="cuda")
    se = torch.zeros((1, 4, 4), dtype=torch.uint8, device="cuda")
    assert lib.fp8_quantize_mx(x.data_ptr(), 4, 64, 64, 2, q.data_ptr(), 64, se.data_ptr(), None) == bsq.ERR_ARG
    assert lib.fp8_quantize_mx(x.data_ptr(), 4, 64, 32, E4, q.data_ptr(), 64, se.data_ptr(), None) == bsq.ERR_SHAPE
    assert lib.fp8_quantize_mx(x.data_ptr(), 4, 64, 64, E4, q.data_ptr(), 64, se.data_ptr() + 1, None) == bsq.ERR_ALIGN
    assert lib.fp8_quantize_mx(None, 4, 64, 64, E4, q.data_ptr(), 64, se.data_ptr(), None) == bsq.ERR_NULL


# ------------------------------------------------------------------ columnwise (transposed) form

def run_quant_t(gpu, rows, cols, fmt, x=None, pitch=None, seed=0, fused=False):
    if x is None:
        x = synth.activations_with_outliers(rows, cols, seed, f"mx/quant_t/{rows}x{cols}")
    ld = pitch if pitch is not None else cols
    store = torch.zeros((rows, ld), dtype=torch.bfloat16)
    store[:, :cols] = x
    xd = store.cuda()[:, :cols]
    ldq = rows + (16 if pitch is not None else 0)
    qstore = torch.full((cols, ldq), 0xA5, dtype=torch.uint8, device="cuda")
    scales = torch.full(bsq.mx_scale_shape(cols, rows), 0xAB, dtype=torch.uint8, device="cuda")
    if fused:
        rstore = torch.full((rows, cols + 16), 0x5A, dtype=torch.uint8, device="cuda")
        rscales = torch.full(bsq.mx_scale_shape(rows, cols), 0xAB, dtype=torch.uint8, device="cuda")
        qr, sr, q, s = gpu.quantize_mx_and_columnwise_t(xd, fmt, q=rstore[:, :cols], scales=rscales,
                                                        qt=qstore[:, :rows], scales_t=scales)
        torch.cuda.synchronize()
        qro, sro = oracle.quantize_mx(x, fmt)
        assert_bytes_equal(qr.cpu().numpy(), qro, f"row codes {rows}x{cols}")
        assert_bytes_equal(sr.cpu().numpy(), abi_scales(sro, 127), f"row scale bytes {rows}x{cols}")
        assert torch.all(rstore[:, cols:] == 0x5A), "row codes past the columns written"
    else:
        q, s = gpu.quantize_mx_columnwise_t(xd, fmt, qt=qstore[:, :rows], scales=scales)
        torch.cuda.synchronize()
    qo, so = oracle.quantize_mx_columnwise_t(x, fmt)
    assert_bytes_equal(q.cpu().numpy(), qo, f"transposed codes {rows}x{cols}")
    assert_bytes_equal(s.cpu().numpy(), abi_scales(so, 127), f"scale bytes {rows}x{cols}")
    assert torch.all(qstore[:, rows:] == 0xA5), "codes past the transposed rows written"


FUSED = pytest.mark.parametrize("fused", [False, True], ids=["columnwise", "rows+columnwise"])


@FUSED
@pytest.mark.parametrize("rows,cols", [(1, 1), (33, 70), (300, 129), (128, 128), (4096, 256),
                                       (70, 5)])
@pytest.mark.parametrize("fmt", [E4, E5])
def test_quantize_mx_columnwise_bit_exact(gpu, rows, cols, fmt, fused):
    run_quant_t(gpu, rows, cols, fmt, fused=fused)


@FUSED
def test_quantize_mx_columnwise_pitch_and_specials(gpu, fused):
    run_quant_t(gpu, 200, 384, E4, pitch=392, fused=fused)
    x = synth.activations_with_outliers(96, 64, 5, "mx/quant_t/special")
    x[:, 3] = 0.0                                     # all-zero blocks: byte 127
    x[10, 7] = float("nan")
    x[40, 9] = float("inf")
    x[70:, 11] = torch.tensor(1e-40).bfloat16()       # bf16 subnormals: the largest scale
    x[5, 13] = 3.0e38                                 # huge magnitude: the smallest scale
    run_quant_t(gpu, 96, 64, E4, x=x, fused=fused)
    run_quant_t(gpu, 96, 64, E5, x=x, fused=fused)


@FUSED
def test_quantize_mx_columnwise_full_size(gpu, fused):
    x = synth.activations_with_outliers(8192, 4096, 0, "bench/8b/qkv/X")
    run_quant_t(gpu, 8192, 4096, E4, x=x, fused=fused)


def test_mx_backward_wgrad_and_dgrad(gpu):
    """The microscaling backward on the GPU path end to end: dW = dY^T . X from the columnwise
    codes of dY and X (blocks of 32 tokens), dX = dY . W from dY's row codes and W's columnwise
    codes (blocks of 32 output features); against the oracle's quantizers and fp64 products."""
    M, N, K = 528, 384, 256       # tokens (ragged: 16.5 blocks of 32), out features, in features
    dy = synth.normal((M, N), 1e-3, 6, "mx/bwd/dY")
    x = synth.activations_with_outliers(M, K, 6, "mx/bwd/X")
    w = synth.normal((N, K), 0.02, 6, "mx/bwd/W")
    dyd, xd, wd = dy.cuda(), x.cuda(), w.cuda()
    # weight gradient [N, K], contraction over the M tokens
    qdyt, sdyt = gpu.quantize_mx_columnwise_t(dyd, E4)
    qxt, sxt = gpu.quantize_mx_columnwise_t(xd, E4)
    dw = gpu.gemm_mx(qdyt, sdyt, qxt, sxt)
    # data gradient [M, K], contraction over the N output features
    qdy, sdy = gpu.quantize_mx(dyd, E4)
    qwt, swt = gpu.quantize_mx_columnwise_t(wd, E4)
    dx = gpu.gemm_mx(qdy, sdy, qwt, swt)
    torch.cuda.synchronize()

    def ref(qa, sa, qb, sb):
        a = oracle.dequantize(qa, E4, oracle.BLOCK_1x32, oracle.e8m0_decode(sa))
        b = oracle.dequantize(qb, E4, oracle.BLOCK_1x32, oracle.e8m0_decode(sb))
        return a @ b.T, np.abs(a) @ np.abs(b).T

    o_dyt, o_sdyt = oracle.quantize_mx_columnwise_t(dy, E4)
    o_xt, o_sxt = oracle.quantize_mx_columnwise_t(x, E4)
    r, mag = ref(o_dyt, o_sdyt, o_xt, o_sxt)
    gemm_check(dw, r, mag, "mx wgrad")
    o_dy, o_sdy = oracle.quantize_mx(dy, E4)
    o_wt, o_swt = oracle.quantize_mx_columnwise_t(w, E4)
    r, mag = ref(o_dy, o_sdy, o_wt, o_swt)
    gemm_check(dx, r, mag, "mx dgrad")


# ------------------------------------------------------------------ grouped (MoE) form

def run_grouped_mx(gpu, counts, N, K, seed, sample_rows=None):
    counts = np.asarray(counts, dtype=np.int64)
    G = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    T = int(off[-1])
    a = synth.activations_with_outliers(T, K, seed, f"mx/grouped/A/{T}x{K}")
    qa, sa = oracle.quantize_mx(a, E4)
    qbs, sbs = [], []
    for g in range(G):
        b = synth.normal((N, K), 0.02, seed + g, f"mx/grouped/B{g}/{N}x{K}")
        qb, sb = oracle.quantize_mx(b, E4)
        qbs.append(qb)
        sbs.append(sb)
    bd = torch.from_numpy(np.stack(qbs)).cuda()
    sbd = torch.stack([device_scale_bytes(s, K) for s in sbs])      # NaN bytes past K
    c = gpu.grouped_gemm_mx(torch.from_numpy(off).cuda(), device_codes(qa, K), device_scale_bytes(sa, K),
                            bd, sbd)
    torch.cuda.synchronize()
    adq = oracle.dequantize(qa, E4, oracle.BLOCK_1x32, oracle.e8m0_decode(sa))
    rows = np.arange(T) if sample_rows is None else np.asarray(sample_rows)
    group_of = np.searchsorted(off, rows, side="right") - 1
    ref = np.zeros((len(rows), N))
    mag = np.zeros((len(rows), N))
    for g in np.unique(group_of):
        sel = np.nonzero(group_of == g)[0]
        bdq = oracle.dequantize(qbs[g], E4, oracle.BLOCK_1x32, oracle.e8m0_decode(sbs[g]))
        ref[sel] = adq[rows[sel]] @ bdq.T
        mag[sel] = np.abs(adq[rows[sel]]) @ np.abs(bdq).T
    gemm_check(c[torch.as_tensor(rows, device="cuda")], ref, mag, f"grouped mx {G} groups")


def test_grouped_gemm_mx_ragged_groups(gpu):
    # empty groups, a one-row group, groups across tile boundaries, ragged K (10 chunks of 32)
    run_grouped_mx(gpu, [0, 1, 300, 0, 257, 130, 64], 384, 320, 11)


def test_grouped_gemm_mx_moe_shape_sampled(gpu):
    # 32 experts with Zipf routing, gate/up-shaped experts (N 1536, K 2048), sampled rows
    counts = synth.moe_routing(2048, 32, 8, 1.1, 5)
    rows = np.arange(0, int(counts.sum()), 37)
    run_grouped_mx(gpu, counts, 1536, 2048, 12, sample_rows=rows)
