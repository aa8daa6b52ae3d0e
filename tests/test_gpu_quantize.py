"""GPU parity of the quantizers against the CPU oracle (bit-exact codes and scales).

Blockwise 1x128 / 128x128 E4M3 / E5M2 with fp32 or power-of-2 scales ("NVIDIA NeMo RL logra una
aceleración del 48% ...", sections "El avance técnico" and "Por qué esto es importante para la
economía de la IA"); the plain fp32 cast over every fp32 bit pattern.
"""
import numpy as np
import pytest
import torch

import block_scaled_quantize_amd as bsq
import oracle
import synth
from helpers import assert_bytes_equal, bits, f32_bits, gpu_scales_to_logical

pytestmark = pytest.mark.gpu

FMTS = [bsq.E4M3, bsq.E5M2]
GRANS = [bsq.BLOCK_1x128, bsq.BLOCK_128x128]
MODES = [bsq.SCALE_FP32, bsq.SCALE_POW2]


def run_parity(gpu, x_cpu: torch.Tensor, fmt, gran, mode, pitch_pad=0, qpad=0, what=""):
    rows, cols = x_cpu.shape
    if pitch_pad:
        big = torch.zeros((rows, cols + pitch_pad), dtype=torch.bfloat16)
        big[:, :cols] = x_cpu
        xd = big.cuda()[:, :cols]
    else:
        xd = x_cpu.cuda()
    q_store = torch.full((rows, cols + qpad), 0xA5, dtype=torch.uint8, device="cuda")
    q = q_store[:, :cols]
    shape = bsq.scale_shape(rows, cols, gran)
    s_store = torch.full((int(np.prod(shape)) + 64,), 12345.0, dtype=torch.float32, device="cuda")
    s = s_store[: int(np.prod(shape))].view(shape)
    gpu.quantize_blockwise(xd, fmt, gran, mode, q=q, scale_inv=s)
    torch.cuda.synchronize()
    qo, so = oracle.quantize_blockwise(bits(x_cpu), fmt, gran, mode)
    assert_bytes_equal(q.cpu().numpy(), qo, f"codes {what}")
    assert_bytes_equal(f32_bits(gpu_scales_to_logical(s, gran)), f32_bits(so), f"scales {what}")
    # guard regions untouched
    if qpad:
        assert torch.all(q_store[:, cols:] == 0xA5)
    assert torch.all(s_store[int(np.prod(shape)):] == 12345.0)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("gran", GRANS)
@pytest.mark.parametrize("mode", MODES)
def test_tiny_config(gpu, fmt, gran, mode):
    # activation X[64,256] ~ N(0,1), weight W[256,256] ~ N(0,0.02), seed 0
    x = synth.normal((64, 256), 1.0, 0, "tiny/X")
    w = synth.normal((256, 256), 0.02, 0, "tiny/W")
    run_parity(gpu, x, fmt, gran, mode, what="tiny X")
    run_parity(gpu, w, fmt, gran, mode, what="tiny W")


@pytest.mark.parametrize("shape", [(1, 1), (3, 7), (131, 300), (129, 129), (257, 1000), (64, 4096 + 16)])
@pytest.mark.parametrize("gran", GRANS)
def test_ragged_shapes(gpu, shape, gran):
    x = synth.student_t(shape, 3.0, 1, f"ragged/{shape}")
    for fmt in FMTS:
        for mode in MODES:
            run_parity(gpu, x, fmt, gran, mode, what=f"{shape}")


@pytest.mark.parametrize("shape", [(1, 1024), (5, 2048), (131, 3072), (6, 14336), (1, 512),
                                   (300, 1536), (129, 512)])
@pytest.mark.parametrize("gran", GRANS)
def test_long_rows(gpu, shape, gran):
    """Rows of a multiple of 1024 columns take the long-row 1x128 kernel (4 rows per workgroup):
    ragged row counts, both formats and scale modes, packed and padded pitches, and an odd pitch
    that falls back to the 32-row tiles (128x128 on the same shapes: the 32-row tiles)."""
    x = synth.student_t(shape, 3.0, 4, f"long/{shape}")
    for fmt in FMTS:
        for mode in MODES:
            run_parity(gpu, x, fmt, gran, mode, what=f"long {shape}")
    run_parity(gpu, x, bsq.E4M3, gran, bsq.SCALE_FP32, pitch_pad=64, qpad=32,
               what=f"long {shape} padded pitch")
    run_parity(gpu, x, bsq.E4M3, gran, bsq.SCALE_FP32, pitch_pad=1, qpad=3,
               what=f"long {shape} odd pitch")


@pytest.mark.parametrize("gran", GRANS)
def test_strided_and_unaligned_pitch(gpu, gran):
    x = synth.normal((200, 384), 1.0, 2, "pitch")
    run_parity(gpu, x, bsq.E4M3, gran, bsq.SCALE_FP32, pitch_pad=3, qpad=5, what="odd pitch")
    run_parity(gpu, x, bsq.E4M3, gran, bsq.SCALE_FP32, pitch_pad=64, qpad=16, what="padded pitch")


@pytest.mark.parametrize("gran", GRANS)
@pytest.mark.parametrize("fmt", FMTS)
def test_all_bf16_classes(gpu, gran, fmt):
    """Uniformly random bf16 bit patterns: zeros, subnormals, huge values, inf, NaN."""
    b = synth.random_bf16_bits((256, 512), 3, "classes")
    x = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    for mode in MODES:
        run_parity(gpu, x, fmt, gran, mode, what="random bf16 patterns")


@pytest.mark.parametrize("fmt", FMTS)
def test_special_blocks(gpu, fmt):
    x = np.zeros((8, 256), dtype=np.uint16)
    x[0, 5] = 0x8000                    # -0 only
    x[1, 0], x[1, 1] = 0xFFC1, 0x4040   # NaN + 3.0
    x[2, 0], x[2, 1], x[2, 2] = 0x7F80, 0xFF80, 0xC040
    x[3, 0], x[3, 1] = 0x0001, 0x8003   # bf16 subnormals only
    x[4, 0] = 0x0460                    # scale 2^127 exactly (E4M3)
    x[5, 0] = 0x0400
    x[6, :] = 0x7F7F                    # bf16 max everywhere
    x[7, 128:] = 0x3C24                 # second block only
    t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    for gran in GRANS:
        for mode in MODES:
            run_parity(gpu, t, fmt, gran, mode, what="special")


def test_worked_example_on_gpu(gpu):
    import os
    g = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", "worked_example_1x128.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, *v = line.split()
                g[k] = [int(t, 16) for t in v]
    x = np.zeros((1, 128), dtype=np.uint16)
    x[0, :8] = g["input_bf16_hex"]
    t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    q, s = gpu.quantize_blockwise(t, bsq.E4M3, bsq.BLOCK_1x128, bsq.SCALE_FP32)
    assert q[0, :8].cpu().tolist() == g["fp32_codes_hex"]
    assert int(f32_bits(s.cpu().numpy())[0, 0]) == g["fp32_scale_inv_hex"][0]
    q, s = gpu.quantize_blockwise(t, bsq.E4M3, bsq.BLOCK_1x128, bsq.SCALE_POW2)
    assert q[0, :8].cpu().tolist() == g["pow2_codes_hex"]
    assert int(f32_bits(s.cpu().numpy())[0, 0]) == g["pow2_scale_inv_hex"][0]


def test_llama8b_activation_and_weight_full_size(gpu):
    """8B-class shapes at full size: X[8192, 4096] with outlier channels (1x128) and
    W_gate_up[28672, 4096] (128x128), every byte and scale compared."""
    x = synth.activations_with_outliers(8192, 4096, 0, "8b/X_qkv")
    run_parity(gpu, x, bsq.E4M3, bsq.BLOCK_1x128, bsq.SCALE_FP32, what="8B X 1x128")
    w = synth.normal((28672, 4096), 0.02, 0, "8b/W_gu")
    run_parity(gpu, w, bsq.E4M3, bsq.BLOCK_128x128, bsq.SCALE_FP32, what="8B W 128x128")


def test_sweep_512m_sampled(gpu):
    """The 512M-element sweep tensor [131072, 4096] (Student-t, nu = 3): the kernel runs on the
    whole tensor in the benchmark's launch configuration; the oracle checks sampled row bands
    (blocks are independent, so a band is checked exactly)."""
    rows, cols = 131072, 4096
    g = np.random.Generator(np.random.PCG64(99))
    for gran, mode in ((bsq.BLOCK_1x128, bsq.SCALE_FP32), (bsq.BLOCK_128x128, bsq.SCALE_POW2)):
        xd = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
        bands = [0, rows // 128 - 1] + list(g.integers(1, rows // 128 - 1, size=6))
        host = {}
        for b in bands:
            t = synth.student_t((128, cols), 3.0, 7, f"sweep/band{b}")
            host[b] = t
            xd[128 * b:128 * (b + 1)] = t.cuda()
        q, s = gpu.quantize_blockwise(xd, bsq.E4M3, gran, mode)
        torch.cuda.synchronize()
        for b, t in host.items():
            qo, so = oracle.quantize_blockwise(bits(t), bsq.E4M3, gran, mode)
            assert_bytes_equal(q[128 * b:128 * (b + 1)].cpu().numpy(), qo, f"band {b}")
            if gran == bsq.BLOCK_1x128:
                sg = s[:, 128 * b:128 * (b + 1)].cpu().numpy().T
            else:
                sg = s[b:b + 1].cpu().numpy()
            assert_bytes_equal(f32_bits(sg), f32_bits(so), f"band {b} scales")
        del xd, q, s
        torch.cuda.empty_cache()


def test_beyond_cache_ragged_sampled(gpu):
    """Codes larger than the 256 MB last-level cache with a ragged last tile row ([65540, 4096]:
    the 4-tile 128x128 kernel and the long-row 1x128 kernel, both with non-temporal code
    stores), fp32 scales; sampled row bands checked exactly, the last one ragged."""
    rows, cols = 65540, 4096
    xd = torch.zeros((rows, cols), dtype=torch.bfloat16, device="cuda")
    bands = [(0, 128), (30080, 30208), (rows - 4, rows)]
    host = {}
    for lo, hi in bands:
        t = synth.student_t((hi - lo, cols), 3.0, 8, f"big/{lo}")
        host[lo] = t
        xd[lo:hi] = t.cuda()
    for gran in GRANS:
        q, s = gpu.quantize_blockwise(xd, bsq.E4M3, gran, bsq.SCALE_FP32)
        torch.cuda.synchronize()
        for lo, hi in bands:
            qo, so = oracle.quantize_blockwise(bits(host[lo]), bsq.E4M3, gran, bsq.SCALE_FP32)
            assert_bytes_equal(q[lo:hi].cpu().numpy(), qo, f"codes rows {lo}..{hi}")
            if gran == bsq.BLOCK_1x128:
                sg = s[:, lo:hi].cpu().numpy().T
            else:
                sg = s[lo // 128:lo // 128 + 1].cpu().numpy()
            assert_bytes_equal(f32_bits(sg), f32_bits(so), f"scales rows {lo}..{hi}")
        del q, s
    del xd
    torch.cuda.empty_cache()


def test_deterministic(gpu):
    x = synth.student_t((1024, 4096), 3.0, 5, "det").cuda()
    for gran in GRANS:
        q1, s1 = gpu.quantize_blockwise(x, bsq.E4M3, gran)
        q2, s2 = gpu.quantize_blockwise(x, bsq.E4M3, gran)
        assert torch.equal(q1, q2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))


@pytest.mark.parametrize("fmt", FMTS)
def test_cast_all_fp32_patterns(gpu, fmt):
    """The saturating RNE cast on every one of the 2^32 fp32 bit patterns vs the oracle."""
    chunk = 1 << 28
    for base in range(0, 1 << 32, chunk):
        xb = torch.arange(base, base + chunk, dtype=torch.int64, device="cuda")
        x32 = torch.where(xb >= 2 ** 31, xb - 2 ** 32, xb).to(torch.int32).view(torch.float32)
        del xb
        q = gpu.cast_fp32(x32, fmt).cpu().numpy()
        del x32
        want = oracle.encode_bit_range(fmt, base, chunk)
        assert_bytes_equal(q, want, f"cast chunk {base:#x}")


# ----------------------------------------------------------------------------- several tensors
# fp8_quantize_blockwise_batched: one launch for several tensors ("NVIDIA NeMo RL ...", section
# "Ganancias de rendimiento en el mundo real": every layer's weight scales are recalibrated each
# step); each tensor's codes and scales equal the oracle's, bit for bit.

@pytest.mark.parametrize("fmt,mode", [(bsq.E4M3, bsq.SCALE_FP32), (bsq.E5M2, bsq.SCALE_POW2)])
def test_batched_mixed_tensors(gpu, fmt, mode):
    shapes = [(300, 260), (0, 128), (128, 128), (1, 7), (513, 1000), (64, 4096), (129, 0), (256, 384)]
    grans = [bsq.BLOCK_128x128, bsq.BLOCK_1x128, bsq.BLOCK_1x128, bsq.BLOCK_128x128,
             bsq.BLOCK_1x128, bsq.BLOCK_128x128, bsq.BLOCK_1x128, bsq.BLOCK_1x128]
    xs_cpu = [synth.student_t(s, 3.0, i, f"batched/x{i}") if s[0] * s[1] else
              torch.zeros(s, dtype=torch.bfloat16) for i, s in enumerate(shapes)]
    xs = []
    for i, x in enumerate(xs_cpu):
        if i % 3 == 2:       # an odd row pitch: the unaligned path
            big = torch.zeros((x.shape[0], x.shape[1] + 3), dtype=torch.bfloat16)
            big[:, :x.shape[1]] = x
            xs.append(big.cuda()[:, :x.shape[1]])
        else:
            xs.append(x.cuda())
    qs, ss = gpu.quantize_blockwise_batched(xs, grans, fmt, mode)
    torch.cuda.synchronize()
    for i, (x, gran) in enumerate(zip(xs_cpu, grans)):
        if x.numel() == 0:
            continue
        qo, so = oracle.quantize_blockwise(bits(x), fmt, gran, mode)
        assert_bytes_equal(qs[i].cpu().numpy(), qo, f"batched codes {i} {tuple(x.shape)}")
        assert_bytes_equal(f32_bits(gpu_scales_to_logical(ss[i], gran)), f32_bits(so),
                           f"batched scales {i}")


def test_batched_equals_single_on_8b_weights(gpu):
    """The four Llama-3.1-8B weights in one launch give what four single launches give."""
    ws = [synth.normal((n, k), 0.02, 0, f"batched8b/W{n}x{k}").cuda()
          for k, n in [(4096, 6144), (4096, 4096), (4096, 28672), (14336, 4096)]]
    grans = [bsq.BLOCK_128x128] * 4
    qs, ss = gpu.quantize_blockwise_batched(ws, grans, bsq.E4M3)
    for w, q, s in zip(ws, qs, ss):
        q1, s1 = gpu.quantize_blockwise(w, bsq.E4M3, bsq.BLOCK_128x128)
        torch.cuda.synchronize()
        assert torch.equal(q, q1) and torch.equal(s.view(torch.int32), s1.view(torch.int32))
