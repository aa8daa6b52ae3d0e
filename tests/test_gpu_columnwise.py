"""GPU parity of the columnwise (128x1 blocks, transposed output) quantizer against the oracle,
bit-exact: codes of x^T and scales in the 1x128 layout of x^T ("NVIDIA NeMo RL logra una
aceleración del 48% ...", section "El avance técnico": one scale per 128 elements along the
contracted dimension -- the token dimension for the weight gradient).  The same cases run
through the one-pass form that also writes the 1x128 row quantization
(fp8_quantize_1x128_and_columnwise_t), both outputs bit-exact.
"""
import numpy as np
import pytest
import torch

import block_scaled_quantize_amd as bsq
import oracle
import synth
from helpers import assert_bytes_equal, bits, f32_bits, gpu_scales_to_logical

pytestmark = pytest.mark.gpu

E4, E5 = bsq.E4M3, bsq.E5M2
FP32, POW2 = bsq.SCALE_FP32, bsq.SCALE_POW2


def run_parity(gpu, x_cpu: torch.Tensor, fmt, mode, pitch_pad=0, qpad=0, col_offset=0, what="",
               fused=False):
    """col_offset: the matrix starts col_offset elements into a device allocation (unaligned
    base when odd).  fused: the one-pass entry point, which also writes the 1x128 row codes."""
    if col_offset:
        xd_full = x_cpu.cuda()
        x_cpu = x_cpu[:, col_offset:].contiguous()
    rows, cols = x_cpu.shape
    if col_offset:
        xd = xd_full[:, col_offset:]
    elif pitch_pad:
        big = torch.zeros((rows, cols + pitch_pad), dtype=torch.bfloat16)
        big[:, :cols] = x_cpu
        xd = big.cuda()[:, :cols]
    else:
        xd = x_cpu.cuda()
    q_store = torch.full((cols, rows + qpad), 0xA5, dtype=torch.uint8, device="cuda")
    qt = q_store[:, :rows]
    nrb = -(-rows // 128)
    s_store = torch.full((nrb * cols + 64,), 12345.0, dtype=torch.float32, device="cuda")
    s = s_store[: nrb * cols].view(nrb, cols)
    if fused:
        r_store = torch.full((rows, cols + qpad), 0x5A, dtype=torch.uint8, device="cuda")
        q = r_store[:, :cols]
        sr = torch.full(bsq.scale_shape(rows, cols, bsq.BLOCK_1x128), 777.0, dtype=torch.float32,
                        device="cuda")
        gpu.quantize_1x128_and_columnwise_t(xd, fmt, mode, q=q, scale_inv=sr, qt=qt, scale_inv_t=s)
        torch.cuda.synchronize()
        qro, sro = oracle.quantize_blockwise(bits(x_cpu), fmt, oracle.BLOCK_1x128, mode)
        assert_bytes_equal(q.cpu().numpy(), qro, f"row codes {what}")
        assert_bytes_equal(f32_bits(gpu_scales_to_logical(sr, bsq.BLOCK_1x128)), f32_bits(sro),
                           f"row scales {what}")
        if qpad:
            assert torch.all(r_store[:, cols:] == 0x5A), "stray writes past the columns"
    else:
        gpu.quantize_columnwise_t(xd, fmt, mode, qt=qt, scale_inv=s)
        torch.cuda.synchronize()
    qo, so = oracle.quantize_columnwise_t(bits(x_cpu), fmt, mode)
    assert_bytes_equal(qt.cpu().numpy(), qo, f"codes {what}")
    assert_bytes_equal(f32_bits(s.cpu().numpy().T), f32_bits(so), f"scales {what}")
    if qpad:
        assert torch.all(q_store[:, rows:] == 0xA5), "stray writes past the rows"
    assert torch.all(s_store[nrb * cols:] == 12345.0), "stray writes past the scales"


FUSED = pytest.mark.parametrize("fused", [False, True], ids=["columnwise", "rows+columnwise"])


@FUSED
@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("mode", [FP32, POW2])
def test_tiny_and_ragged(gpu, fmt, mode, fused):
    for shape in [(64, 256), (128, 128), (1, 1), (3, 7), (130, 257), (257, 129), (1000, 72)]:
        x = synth.student_t(shape, 3.0, 1, f"colwise/{shape}")
        run_parity(gpu, x, fmt, mode, what=str(shape), fused=fused)


@FUSED
def test_pitches_and_unaligned_paths(gpu, fused):
    x = synth.normal((300, 200), 1.0, 2, "colwise/pitch")
    run_parity(gpu, x, E4, FP32, pitch_pad=8, qpad=16, what="vector path with padding", fused=fused)
    run_parity(gpu, x, E4, FP32, pitch_pad=3, qpad=5, what="odd pitches (scalar path)", fused=fused)
    run_parity(gpu, x, E5, POW2, col_offset=1, what="unaligned base", fused=fused)


@FUSED
def test_special_blocks(gpu, fused):
    rows, cols = 256, 48
    x = synth.normal((rows, cols), 1.0, 3, "colwise/special").float()
    x[:, 0] = 0.0                                  # all-zero column blocks
    x[5, 1] = float("nan")                         # NaN in block (0, 1)
    x[200, 2] = float("-nan")
    x[7, 3] = float("inf")                         # Inf -> scale 1, saturated
    x[130, 4] = float("-inf")
    x[:128, 5] = 1e-40                             # bf16-subnormal block
    x[:, 6] = 3e38                                 # near the bf16 maximum
    x[:, 7] = -x[:, 7]
    xb = x.to(torch.bfloat16)
    for fmt in (E4, E5):
        for mode in (FP32, POW2):
            run_parity(gpu, xb, fmt, mode, what=f"special fmt {fmt} mode {mode}", fused=fused)


@FUSED
def test_every_bf16_bit_class(gpu, fused):
    """Random bf16 bit patterns: every exponent, both signs, NaN/Inf/subnormal in the mix."""
    xb = synth.random_bf16_bits((512, 384), 4, "colwise/bits")
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16)
    for fmt in (E4, E5):
        run_parity(gpu, x, fmt, FP32, what=f"bits fmt {fmt}", fused=fused)


@pytest.mark.parametrize("name,rows,cols,fmt", [("X", 8192, 4096, E4), ("dY gate_up", 8192, 28672, E4),
                                                ("dY down", 8192, 4096, E5)])
def test_llama8b_backward_full_size(gpu, name, rows, cols, fmt):
    """The weight-gradient operands of the 8B-class layers, full size, bit-exact."""
    std = 1.0 if name == "X" else 1e-3
    x = synth.normal((rows, cols), std, 0, f"colwise/full/{name}")
    run_parity(gpu, x, fmt, FP32, what=name, fused=name.startswith("dY"))
