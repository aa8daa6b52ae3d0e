// Block-scaled FP8 fprop GEMM with the output quantized in the epilogue: besides (or instead of)
// the bf16 output, the kernel writes the output's E4M3 codes and 1x128 dequantization factors
// -- the operand the next layer's fprop GEMM takes -- so no separate quantization pass reads
// the output back.  Device code in gemm_impl.h (quantize_out).
//
// Method: "NVIDIA NeMo RL logra una aceleración del 48% con entrenamiento de precisión FP8 de
// extremo a extremo", section "Ganancias de rendimiento en el mundo real" (the overhead of the
// separate quantization kernels) and section "El avance técnico" (1x128 activation blocks,
// E4M3); section "Por qué esto es importante para la economía de la IA" (power-of-2 scales).
#include "gemm_impl.h"

using namespace fp8bs;

namespace {

int gemm_qout(int tile, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int ga,
              const float* scale_inv_a, const void* B, int64_t ldb, int gb,
              const float* scale_inv_b, int pow2_inputs, void* C_bf16, int64_t ldc,
              int mode_out, void* Cq, int64_t ldcq, float* cq_scale_inv, hipStream_t st) {
  if ((mode_out != FP8BS_SCALE_FP32 && mode_out != FP8BS_SCALE_POW2) ||
      (pow2_inputs != 0 && pow2_inputs != 1) || !tile_ok(tile))
    return FP8BS_ERR_ARG;
  GemmParams p{};
  bool tensor_only = false, empty = false, b_rows = false;
  const int s = dense_params(FP8BS_FPROP, M, N, K, A, lda, FP8BS_E4M3, ga, scale_inv_a, B, ldb,
                             FP8BS_E4M3, gb, scale_inv_b, C_bf16, ldc, p, tensor_only, empty,
                             b_rows, /*c_optional=*/true);
  if (s != FP8BS_OK || empty) return s;
  if (!Cq || !cq_scale_inv) return FP8BS_ERR_NULL;
  if (ldcq < N) return FP8BS_ERR_SHAPE;
  if (!aligned4(cq_scale_inv)) return FP8BS_ERR_ALIGN;
  if (b_rows) return FP8BS_ERR_UNSUPPORTED;
  p.C = static_cast<uint16_t*>(C_bf16);
  p.Cq = static_cast<uint8_t*>(Cq);
  p.ldcq = ldcq;
  p.cqs = cq_scale_inv;
  p.cq_vec = aligned4(Cq) && ldcq % 4 == 0;
  p.cq_vec16 = aligned16(Cq) && ldcq % 16 == 0;
  constexpr int E4 = FP8BS_E4M3, FP = FP8BS_FPROP;
  const bool pow2_out = mode_out == FP8BS_SCALE_POW2;
  // output codes: E4M3, 1 + 2 * format + power-of-2
  if (tensor_only)
    return pow2_out ? dispatch_variant<FP, E4, E4, kScaleTensor, 2>(p, tile, st)
                    : dispatch_variant<FP, E4, E4, kScaleTensor, 1>(p, tile, st);
  if (pow2_inputs)
    return pow2_out ? dispatch_variant<FP, E4, E4, kScaleHw, 2>(p, tile, st)
                    : dispatch_variant<FP, E4, E4, kScaleHw, 1>(p, tile, st);
  return pow2_out ? dispatch_variant<FP, E4, E4, kScaleFold, 2>(p, tile, st)
                  : dispatch_variant<FP, E4, E4, kScaleFold, 1>(p, tile, st);
}

}  // namespace

extern "C" int fp8_gemm_blockscaled_qout(int64_t M, int64_t N, int64_t K, const void* A,
                                         int64_t lda, int ga, const float* scale_inv_a,
                                         const void* B, int64_t ldb, int gb,
                                         const float* scale_inv_b, int pow2_inputs,
                                         void* C_bf16, int64_t ldc, int mode_out, void* Cq,
                                         int64_t ldcq, float* cq_scale_inv, void* stream) {
  return gemm_qout(FP8BS_TILE_AUTO, M, N, K, A, lda, ga, scale_inv_a, B, ldb, gb, scale_inv_b,
                   pow2_inputs, C_bf16, ldc, mode_out, Cq, ldcq, cq_scale_inv,
                   static_cast<hipStream_t>(stream));
}

extern "C" int fp8_gemm_blockscaled_qout_tiled(int tile, int64_t M, int64_t N, int64_t K,
                                               const void* A, int64_t lda, int ga,
                                               const float* scale_inv_a, const void* B,
                                               int64_t ldb, int gb, const float* scale_inv_b,
                                               int pow2_inputs, void* C_bf16, int64_t ldc,
                                               int mode_out, void* Cq, int64_t ldcq,
                                               float* cq_scale_inv, void* stream) {
  return gemm_qout(tile, M, N, K, A, lda, ga, scale_inv_a, B, ldb, gb, scale_inv_b, pow2_inputs,
                   C_bf16, ldc, mode_out, Cq, ldcq, cq_scale_inv, static_cast<hipStream_t>(stream));
}
