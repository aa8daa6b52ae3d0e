// Block-scaled FP8 GEMM entry points with fp32 scales (dense and grouped), and the entry points
// that take an explicit tile configuration; the device code is in gemm_impl.h.
#include "gemm_impl.h"

namespace fp8bs {

int gemm_dense_fp32(int tile, int layout, int64_t M, int64_t N, int64_t K, const void* A,
                    int64_t lda, int fa, int ga, const float* sa, const void* B, int64_t ldb,
                    int fb, int gb, const float* sb, void* C, int64_t ldc, hipStream_t st) {
  GemmParams p{};
  bool tensor_only = false, empty = false, b_rows = false;
  const int s = dense_params(layout, M, N, K, A, lda, fa, ga, sa, B, ldb, fb, gb, sb, C, ldc, p,
                             tensor_only, empty, b_rows);
  if (s != FP8BS_OK || empty) return s;
  if (tensor_only) return dispatch_dense<kScaleTensor>(layout, fa, fb, p, tile, st);
  return b_rows ? dispatch_dense<kScaleFoldRows>(layout, fa, fb, p, tile, st)
                : dispatch_dense<kScaleFold>(layout, fa, fb, p, tile, st);
}

int gemm_grouped_fp32(int tile, int32_t G, const int64_t* offsets, int64_t M, int64_t N,
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
  return dispatch_grouped<kScaleFold>(fa, fb, cus, p, tile, st);
}

}  // namespace fp8bs

using namespace fp8bs;

extern "C" int fp8_gemm_blockscaled(int layout, int64_t M, int64_t N, int64_t K, const void* A,
                                    int64_t lda, int fa, int ga, const float* scale_inv_a,
                                    const void* B, int64_t ldb, int fb, int gb,
                                    const float* scale_inv_b, void* C_bf16, int64_t ldc,
                                    void* stream) {
  return gemm_dense_fp32(FP8BS_TILE_AUTO, layout, M, N, K, A, lda, fa, ga, scale_inv_a, B, ldb,
                         fb, gb, scale_inv_b, C_bf16, ldc, static_cast<hipStream_t>(stream));
}

extern "C" int fp8_grouped_gemm(int32_t num_groups, const int64_t* group_offsets,
                                int64_t total_M, int64_t N, int64_t K, const void* A,
                                int64_t lda, int fa, const float* scale_inv_a, const void* B,
                                int64_t ldb, int fb, const float* scale_inv_b, void* C_bf16,
                                int64_t ldc, void* stream) {
  return gemm_grouped_fp32(FP8BS_TILE_AUTO, num_groups, group_offsets, total_M, N, K, A, lda, fa,
                           scale_inv_a, B, ldb, fb, scale_inv_b, C_bf16, ldc,
                           static_cast<hipStream_t>(stream));
}

extern "C" int fp8_gemm_blockscaled_tiled(int tile, int pow2, int layout, int64_t M, int64_t N,
                                          int64_t K, const void* A, int64_t lda, int fa, int ga,
                                          const float* scale_inv_a, const void* B, int64_t ldb,
                                          int fb, int gb, const float* scale_inv_b,
                                          void* C_bf16, int64_t ldc, void* stream) {
  if (!tile_ok(tile) || (pow2 != 0 && pow2 != 1)) return FP8BS_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return pow2 ? gemm_dense_pow2(tile, layout, M, N, K, A, lda, fa, ga, scale_inv_a, B, ldb, fb,
                                gb, scale_inv_b, C_bf16, ldc, st)
              : gemm_dense_fp32(tile, layout, M, N, K, A, lda, fa, ga, scale_inv_a, B, ldb, fb,
                                gb, scale_inv_b, C_bf16, ldc, st);
}

extern "C" int fp8_grouped_gemm_tiled(int tile, int pow2, int32_t num_groups,
                                      const int64_t* group_offsets, int64_t total_M, int64_t N,
                                      int64_t K, const void* A, int64_t lda, int fa,
                                      const float* scale_inv_a, const void* B, int64_t ldb,
                                      int fb, const float* scale_inv_b, void* C_bf16,
                                      int64_t ldc, void* stream) {
  if (!grouped_tile_ok(tile) || (pow2 != 0 && pow2 != 1)) return FP8BS_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return pow2 ? gemm_grouped_pow2(tile, num_groups, group_offsets, total_M, N, K, A, lda, fa,
                                  scale_inv_a, B, ldb, fb, scale_inv_b, C_bf16, ldc, st)
              : gemm_grouped_fp32(tile, num_groups, group_offsets, total_M, N, K, A, lda, fa,
                                  scale_inv_a, B, ldb, fb, scale_inv_b, C_bf16, ldc, st);
}
