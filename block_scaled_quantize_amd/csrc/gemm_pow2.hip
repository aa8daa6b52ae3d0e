// Block-scaled FP8 GEMM entry points for power-of-2 scales (dense and grouped): the scales'
// exponents are handed to the MFMA as E8M0 block scales, so the products accumulate in the
// matrix core with no fold between K blocks.  Device code in gemm_impl.h.
//
// Method: "NVIDIA NeMo RL logra una aceleración del 48% con entrenamiento de precisión FP8 de
// extremo a extremo", section "Por qué esto es importante para la economía de la IA": the option
// of power-of-2 scale factors; with them the block scales are exact exponents.
#include "gemm_impl.h"

namespace fp8bs {

int gemm_dense_pow2(int tile, int layout, int64_t M, int64_t N, int64_t K, const void* A,
                    int64_t lda, int fa, int ga, const float* sa, const void* B, int64_t ldb,
                    int fb, int gb, const float* sb, void* C, int64_t ldc, hipStream_t st) {
  GemmParams p{};
  bool tensor_only = false, empty = false, b_rows = false;
  const int s = dense_params(layout, M, N, K, A, lda, fa, ga, sa, B, ldb, fb, gb, sb, C, ldc, p,
                             tensor_only, empty, b_rows);
  if (s != FP8BS_OK || empty) return s;
  if (tensor_only) return dispatch_dense<kScaleTensor>(layout, fa, fb, p, tile, st);
  return b_rows ? dispatch_dense<kScaleHwRows>(layout, fa, fb, p, tile, st)
                : dispatch_dense<kScaleHw>(layout, fa, fb, p, tile, st);
}

int gemm_grouped_pow2(int tile, int32_t G, const int64_t* offsets, int64_t M, int64_t N,
                      int64_t K, const void* A, int64_t lda, int fa, const float* sa,
                      const void* B, int64_t ldb, int fb, const float* sb, void* C, int64_t ldc,
                      hipStream_t st) {
  GemmParams p{};
  bool empty = false;
  const int s = grouped_params(G, offsets, M, N, K, A, lda, fa, sa, B, ldb, fb, sb, C, ldc, p,
                               empty);
  if (s != FP8BS_OK || empty) return s;
  const int cus = device_cus();
  if (cus <= 0) return FP8BS_ERR_LAUNCH;
  return dispatch_grouped<kScaleHw>(fa, fb, cus, p, tile, st);
}

}  // namespace fp8bs

using namespace fp8bs;

extern "C" int fp8_gemm_blockscaled_pow2(int layout, int64_t M, int64_t N, int64_t K,
                                         const void* A, int64_t lda, int fa, int ga,
                                         const float* scale_inv_a, const void* B, int64_t ldb,
                                         int fb, int gb, const float* scale_inv_b, void* C_bf16,
                                         int64_t ldc, void* stream) {
  return gemm_dense_pow2(FP8BS_TILE_AUTO, layout, M, N, K, A, lda, fa, ga, scale_inv_a, B, ldb,
                         fb, gb, scale_inv_b, C_bf16, ldc, static_cast<hipStream_t>(stream));
}

extern "C" int fp8_grouped_gemm_pow2(int32_t num_groups, const int64_t* group_offsets,
                                     int64_t total_M, int64_t N, int64_t K, const void* A,
                                     int64_t lda, int fa, const float* scale_inv_a,
                                     const void* B, int64_t ldb, int fb,
                                     const float* scale_inv_b, void* C_bf16, int64_t ldc,
                                     void* stream) {
  return gemm_grouped_pow2(FP8BS_TILE_AUTO, num_groups, group_offsets, total_M, N, K, A, lda, fa,
                           scale_inv_a, B, ldb, fb, scale_inv_b, C_bf16, ldc,
                           static_cast<hipStream_t>(stream));
}
