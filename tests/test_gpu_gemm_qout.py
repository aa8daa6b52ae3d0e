"""GPU parity of the fprop GEMM with the output quantized in its epilogue
(fp8_gemm_blockscaled_qout): the bf16 output equals the plain GEMM's bit for bit, and the fused
E4M3 codes and 1x128 scales equal, bit for bit, both the standalone GPU quantizer and the oracle
quantizer applied to that bf16 output ("NVIDIA NeMo RL logra una aceleración del 48% ...",
sections "El avance técnico" and "Ganancias de rendimiento en el mundo real").
"""
import numpy as np
import pytest
import torch

import block_scaled_quantize_amd as bsq
import oracle
import synth
from helpers import (abs_product, assert_bytes_equal, bits, f32_bits, gemm_check,
                     gpu_scales_to_logical, logical_to_gpu_scales)

pytestmark = pytest.mark.gpu

FP = bsq.FPROP
E4 = bsq.E4M3
B1, B128, PT = bsq.BLOCK_1x128, bsq.BLOCK_128x128, bsq.PER_TENSOR
FP32, POW2 = bsq.SCALE_FP32, bsq.SCALE_POW2


def operand(x, gran, mode):
    if gran == PT:
        st = oracle.DelayedState(1)
        b = bits(x)
        oracle.delayed_step(b, E4, mode, 0, st)
        q, siu = oracle.delayed_step(b, E4, mode, 0, st)
        return q, np.array([[siu]], dtype=np.float32), torch.tensor([siu], dtype=torch.float32).cuda()
    q, s = oracle.quantize_blockwise(bits(x), E4, gran, mode)
    return q, s, logical_to_gpu_scales(s, gran)


def device_codes(q: np.ndarray) -> torch.Tensor:
    """Codes on the device with the row pitch rounded up to 16 bytes (the GEMM's pitch rule)."""
    rows, cols = q.shape
    ld = -(-cols // 16) * 16
    store = torch.zeros((rows, ld), dtype=torch.uint8)
    store[:, :cols] = torch.from_numpy(q)
    return store.cuda()[:, :cols]


def run_qout(gpu, M, N, K, ga, gb, pow2_in, mode_out, want_bf16=True, nan_row=None, seed=0,
             check_oracle_gemm=True, tile=0):
    mode_in = POW2 if pow2_in else FP32
    a = synth.activations_with_outliers(M, K, seed, "qout/A")
    b = synth.normal((N, K), 0.02, seed, "qout/B")
    qa, sa, sad = operand(a, ga, mode_in)
    qb, sb, sbd = operand(b, gb, mode_in)
    if nan_row is not None:
        qa[nan_row, 3] = 0x7F                 # a NaN code: that output row becomes NaN
    ad, bd = device_codes(qa), device_codes(qb)
    c, cq, cqs = gpu.gemm_blockscaled_qout(ad, ga, sad, bd, gb, sbd, mode_out, pow2_in, want_bf16,
                                           tile=tile)
    c_plain = gpu.gemm_blockscaled(FP, ad, E4, ga, sad, bd, E4, gb, sbd, pow2=pow2_in, tile=tile)
    torch.cuda.synchronize()
    if want_bf16:
        assert torch.equal(c.view(torch.int16), c_plain.view(torch.int16)), "bf16 output differs"
    else:
        assert c is None
    # the fused codes are the blockwise quantization of the bf16 output
    q2, s2 = gpu.quantize_blockwise(c_plain, E4, B1, mode_out)
    torch.cuda.synchronize()
    assert_bytes_equal(cq.cpu().numpy(), q2.cpu().numpy(), f"codes vs GPU quantizer {M}x{N}x{K}")
    assert_bytes_equal(f32_bits(cqs.cpu().numpy()), f32_bits(s2.cpu().numpy()), "scales vs GPU quantizer")
    qo, so = oracle.quantize_blockwise(bits(c_plain.cpu()), E4, B1, mode_out)
    assert_bytes_equal(cq.cpu().numpy(), qo, f"codes vs oracle {M}x{N}x{K}")
    assert_bytes_equal(f32_bits(gpu_scales_to_logical(cqs, B1)), f32_bits(so), "scales vs oracle")
    if check_oracle_gemm and nan_row is None:
        adq, bdq = oracle.dequantize(qa, E4, ga, sa), oracle.dequantize(qb, E4, gb, sb)
        gemm_check(c_plain, adq @ bdq.T, abs_product(FP, adq, bdq), "qout gemm")


SHAPES = [(64, 128, 128), (300, 260, 200), (129, 384, 512), (1000, 1000, 1000), (1, 129, 33),
          (255, 127, 129), (520, 390, 392)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("mode_out", [FP32, POW2])
def test_fused_output_quantization(gpu, M, N, K, mode_out):
    run_qout(gpu, M, N, K, B1, B128, False, mode_out)


@pytest.mark.parametrize("ga,gb,pow2_in", [(B1, B128, True), (PT, PT, False), (B128, PT, False),
                                           (PT, B128, True)])
def test_scale_kinds_and_pow2_inputs(gpu, ga, gb, pow2_in):
    run_qout(gpu, 300, 260, 384, ga, gb, pow2_in, FP32)
    run_qout(gpu, 300, 260, 384, ga, gb, pow2_in, POW2)


def test_quantized_output_only_and_nan_rows(gpu):
    run_qout(gpu, 300, 260, 200, B1, B128, False, FP32, want_bf16=False)
    run_qout(gpu, 300, 260, 200, B1, B128, False, FP32, nan_row=17)


def test_k_zero(gpu):
    a = torch.zeros((5, 0), dtype=torch.uint8, device="cuda")
    b = torch.zeros((130, 0), dtype=torch.uint8, device="cuda")
    s = torch.ones(1, device="cuda")
    c, cq, cqs = gpu.gemm_blockscaled_qout(a, PT, s, b, PT, s)
    torch.cuda.synchronize()
    assert torch.all(c == 0) and torch.all(cq == 0) and torch.all(cqs == 1.0)


@pytest.mark.parametrize("variant", ["A", "B", "C", "D"])
def test_every_tile_variant(gpu, variant):
    tile = {"A": bsq.TILE_256x128_W4, "B": bsq.TILE_256x128_W8, "C": bsq.TILE_256x256_W8,
            "D": bsq.TILE_128x128_W4}[variant]
    run_qout(gpu, 520, 390, 392, B1, B128, False, FP32, tile=tile)
    run_qout(gpu, 256, 256, 256, B1, B128, True, POW2, tile=tile)


def test_llama8b_qkv_full_size(gpu):
    """M = 8192 tokens, qkv 4096 -> 6144: every code and scale of the full output checked."""
    run_qout(gpu, 8192, 6144, 4096, B1, B128, False, FP32, check_oracle_gemm=False)
