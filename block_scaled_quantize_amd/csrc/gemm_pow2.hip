// Block-scaled FP8 GEMM entry points for power-of-2 scales (dense and grouped): the scales'
// exponents are handed to the MFMA as E8M0 block scales, so the products accumulate in the
// matrix core with no fold between K blocks.  Device code in gemm_impl.h.
//
// Method: "NVIDIA NeMo RL logra una aceleración del 48% con entrenamiento de precisión FP8 de
// extremo a extremo", section "Por qué esto es importante para la economía de la IA": the option
// of power-of-2 scale factors; with them the block scales are exact exponents.
#include "gemm_impl.h"

using namespace fp8bs;

extern "C" int fp8_gemm_blockscaled_pow2(int layout, int64_t M, int64_t N, int64_t K,
                                         const void* A, int64_t lda, int fa, int ga,
                                         const float* scale_inv_a, const void* B, int64_t ldb,
                                         int fb, int gb, const float* scale_inv_b, void* C_bf16,
                                         int64_t ldc, void* stream) {
  GemmParams p{};
  bool tensor_only = false, empty = false, b_rows = false;
  const int s = dense_params(layout, M, N, K, A, lda, fa, ga, scale_inv_a, B, ldb, fb, gb,
                             scale_inv_b, C_bf16, ldc, p, tensor_only, empty, b_rows);
  if (s != FP8BS_OK || empty) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (tensor_only) return dispatch_dense<kScaleTensor>(layout, fa, fb, p, st);
  return b_rows ? dispatch_dense<kScaleHwRows>(layout, fa, fb, p, st)
                : dispatch_dense<kScaleHw>(layout, fa, fb, p, st);
}

extern "C" int fp8_grouped_gemm_pow2(int32_t num_groups, const int64_t* group_offsets,
                                     int64_t total_M, int64_t N, int64_t K, const void* A,
                                     int64_t lda, int fa, const float* scale_inv_a,
                                     const void* B, int64_t ldb, int fb,
                                     const float* scale_inv_b, void* C_bf16, int64_t ldc,
                                     void* stream) {
  GemmParams p{};
  bool empty = false;
  const int s = grouped_params(num_groups, group_offsets, total_M, N, K, A, lda, fa, scale_inv_a,
                               B, ldb, fb, scale_inv_b, C_bf16, ldc, p, empty);
  if (s != FP8BS_OK || empty) return s;
  return dispatch_grouped<kScaleHw>(fa, fb, device_cus(), p, static_cast<hipStream_t>(stream));
}
