// Block-scaled FP8 GEMM entry points (dense and grouped; fp32 and power-of-2 scales; with an
// explicit tile configuration): argument checks and the choice of kernel set.  The kernels are
// instantiated per layout in gemm_fprop.hip, gemm_fprop_pow2.hip, gemm_mx.hip, gemm_dgrad.hip,
// gemm_wgrad.hip and gemm_grouped.hip; the device code is in gemm_impl.h.
//
// Method: "NVIDIA NeMo RL logra una aceleración del 48% con entrenamiento de precisión FP8 de
// extremo a extremo", section "El avance técnico" (FP8 linear layers with 128x128 weight and
// 1x128 activation scales, BF16 output) and section "Por qué esto es importante para la
// economía de la IA" (power-of-2 scales).
#include "gemm_impl.h"

namespace fp8bs {
namespace {

int gemm_dense(bool pow2, int tile, int layout, int64_t M, int64_t N, int64_t K, const void* A,
               int64_t lda, int fa, int ga, const float* sa, const void* B, int64_t ldb, int fb,
               int gb, const float* sb, void* C, int64_t ldc, hipStream_t st) {
  GemmParams p{};
  bool tensor_only = false, empty = false, b_rows = false;
  const int s = dense_params(layout, M, N, K, A, lda, fa, ga, sa, B, ldb, fb, gb, sb, C, ldc, p,
                             tensor_only, empty, b_rows);
  if (s != FP8BS_OK || empty) return s;
  // 1x128 weight scales need a K-major weight operand, which dense_params accepts for fprop only
  const int sm = tensor_only ? kScaleTensor
                 : pow2      ? (b_rows ? kScaleHwRows : kScaleHw)
                             : (b_rows ? kScaleFoldRows : kScaleFold);
  switch (layout) {
    case FP8BS_FPROP:
      return (sm == kScaleHw || sm == kScaleHwRows) ? gemm_fprop_pow2(sm, fa, fb, p, tile, st)
                                                    : gemm_fprop_fp32(sm, fa, fb, p, tile, st);
    case FP8BS_DGRAD: return gemm_dgrad(sm, fa, fb, p, tile, st);
    default: return gemm_wgrad(sm, fa, fb, p, tile, st);
  }
}

// Microscaling GEMM (fprop): the dense checks with per-tensor stand-ins for the scales, then
// the scale words of both operands: row r, K block kb at word kb * rows + r (the 1x128 layout).
int gemm_mx_entry(int tile, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int fa,
                  const void* sa, const void* B, int64_t ldb, int fb, const void* sb, void* C,
                  int64_t ldc, hipStream_t st) {
  GemmParams p{};
  bool tensor_only = false, empty = false, b_rows = false;
  const float* fa_s = static_cast<const float*>(sa);
  const float* fb_s = static_cast<const float*>(sb);
  int s = dense_params(FP8BS_FPROP, M, N, K, A, lda, fa, FP8BS_PER_TENSOR, fa_s, B, ldb, fb,
                       FP8BS_PER_TENSOR, fb_s, C, ldc, p, tensor_only, empty, b_rows);
  if (s != FP8BS_OK || empty) return s;
  if (K == 0) return gemm_fprop_fp32(kScaleTensor, fa, fb, p, tile, st);   // zeros
  if (!aligned4(sa) || !aligned4(sb)) return FP8BS_ERR_ALIGN;
  const int64_t nkb = ceil_div(K, 128);
  // scale arrays below 4 GiB (the kernels size their scale DMA in 32 bits)
  if (nkb * M * 4 >= (int64_t(1) << 32) || nkb * N * 4 >= (int64_t(1) << 32)) return FP8BS_ERR_SHAPE;
  p.sa_ks = M; p.sa_rs = 1; p.sa_rshift = 0; p.sa_bytes = nkb * M * 4;
  p.sb_ks = N; p.sb_rs = 1; p.sb_bytes = nkb * N * 4;
  return gemm_fprop_mx(fa, fb, p, tile, st);
}

int grouped_mx_entry(int tile, int32_t G, const int64_t* offsets, int64_t M, int64_t N, int64_t K,
                     const void* A, int64_t lda, int fa, const void* sa, const void* B,
                     int64_t ldb, int fb, const void* sb, void* C, int64_t ldc, hipStream_t st) {
  GemmParams p{};
  bool empty = false;
  const int s = grouped_params(G, offsets, M, N, K, A, lda, fa, static_cast<const float*>(sa), B,
                               ldb, fb, static_cast<const float*>(sb), C, ldc, p, empty);
  if (s != FP8BS_OK || empty) return s;
  if (!aligned4(sa) || !aligned4(sb)) return FP8BS_ERR_ALIGN;
  // expert g's weight scale words: [ceil(K/128)][N] from sb + g * ceil(K/128) * N
  p.sb_ks = N; p.sb_rs = 1;
  p.sb_group_stride = ceil_div(K, 128) * N;
  p.sb_bytes = p.sb_group_stride * 4;
  if (p.sb_bytes >= (int64_t(1) << 32)) return FP8BS_ERR_SHAPE;
  const int cus = device_cus();
  if (cus <= 0) return FP8BS_ERR_LAUNCH;
  return gemm_grouped_mx(fa, fb, cus, p, tile, st);
}

int gemm_grouped_entry(bool pow2, int tile, int32_t G, const int64_t* offsets, int64_t M,
                       int64_t N, int64_t K, const void* A, int64_t lda, int fa, const float* sa,
                       const void* B, int64_t ldb, int fb, const float* sb, void* C, int64_t ldc,
                       hipStream_t st) {
  GemmParams p{};
  bool empty = false;
  const int s = grouped_params(G, offsets, M, N, K, A, lda, fa, sa, B, ldb, fb, sb, C, ldc, p,
                               empty);
  if (s != FP8BS_OK || empty) return s;
  const int cus = device_cus();
  if (cus <= 0) return FP8BS_ERR_LAUNCH;
  return gemm_grouped(pow2, fa, fb, cus, p, tile, st);
}

}  // namespace
}  // namespace fp8bs

using namespace fp8bs;

extern "C" int fp8_gemm_mx(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int fa,
                           const void* scale_e8m0_a, const void* B, int64_t ldb, int fb,
                           const void* scale_e8m0_b, void* C_bf16, int64_t ldc, void* stream) {
  return gemm_mx_entry(FP8BS_TILE_AUTO, M, N, K, A, lda, fa, scale_e8m0_a, B, ldb, fb,
                       scale_e8m0_b, C_bf16, ldc, static_cast<hipStream_t>(stream));
}

extern "C" int fp8_grouped_gemm_mx(int32_t num_groups, const int64_t* group_offsets,
                                   int64_t total_M, int64_t N, int64_t K, const void* A,
                                   int64_t lda, int fa, const void* scale_e8m0_a, const void* B,
                                   int64_t ldb, int fb, const void* scale_e8m0_b, void* C_bf16,
                                   int64_t ldc, void* stream) {
  return grouped_mx_entry(FP8BS_TILE_AUTO, num_groups, group_offsets, total_M, N, K, A, lda, fa,
                          scale_e8m0_a, B, ldb, fb, scale_e8m0_b, C_bf16, ldc,
                          static_cast<hipStream_t>(stream));
}

extern "C" int fp8_gemm_blockscaled(int layout, int64_t M, int64_t N, int64_t K, const void* A,
                                    int64_t lda, int fa, int ga, const float* scale_inv_a,
                                    const void* B, int64_t ldb, int fb, int gb,
                                    const float* scale_inv_b, void* C_bf16, int64_t ldc,
                                    void* stream) {
  return gemm_dense(false, FP8BS_TILE_AUTO, layout, M, N, K, A, lda, fa, ga, scale_inv_a, B, ldb,
                    fb, gb, scale_inv_b, C_bf16, ldc, static_cast<hipStream_t>(stream));
}

extern "C" int fp8_gemm_blockscaled_pow2(int layout, int64_t M, int64_t N, int64_t K,
                                         const void* A, int64_t lda, int fa, int ga,
                                         const float* scale_inv_a, const void* B, int64_t ldb,
                                         int fb, int gb, const float* scale_inv_b, void* C_bf16,
                                         int64_t ldc, void* stream) {
  return gemm_dense(true, FP8BS_TILE_AUTO, layout, M, N, K, A, lda, fa, ga, scale_inv_a, B, ldb,
                    fb, gb, scale_inv_b, C_bf16, ldc, static_cast<hipStream_t>(stream));
}

extern "C" int fp8_grouped_gemm(int32_t num_groups, const int64_t* group_offsets,
                                int64_t total_M, int64_t N, int64_t K, const void* A,
                                int64_t lda, int fa, const float* scale_inv_a, const void* B,
                                int64_t ldb, int fb, const float* scale_inv_b, void* C_bf16,
                                int64_t ldc, void* stream) {
  return gemm_grouped_entry(false, FP8BS_TILE_AUTO, num_groups, group_offsets, total_M, N, K, A,
                            lda, fa, scale_inv_a, B, ldb, fb, scale_inv_b, C_bf16, ldc,
                            static_cast<hipStream_t>(stream));
}

extern "C" int fp8_grouped_gemm_pow2(int32_t num_groups, const int64_t* group_offsets,
                                     int64_t total_M, int64_t N, int64_t K, const void* A,
                                     int64_t lda, int fa, const float* scale_inv_a,
                                     const void* B, int64_t ldb, int fb,
                                     const float* scale_inv_b, void* C_bf16, int64_t ldc,
                                     void* stream) {
  return gemm_grouped_entry(true, FP8BS_TILE_AUTO, num_groups, group_offsets, total_M, N, K, A,
                            lda, fa, scale_inv_a, B, ldb, fb, scale_inv_b, C_bf16, ldc,
                            static_cast<hipStream_t>(stream));
}

extern "C" int fp8_gemm_blockscaled_tiled(int tile, int pow2, int layout, int64_t M, int64_t N,
                                          int64_t K, const void* A, int64_t lda, int fa, int ga,
                                          const float* scale_inv_a, const void* B, int64_t ldb,
                                          int fb, int gb, const float* scale_inv_b,
                                          void* C_bf16, int64_t ldc, void* stream) {
  if (!tile_ok(tile) || (pow2 != 0 && pow2 != 1)) return FP8BS_ERR_ARG;
  return gemm_dense(pow2 != 0, tile, layout, M, N, K, A, lda, fa, ga, scale_inv_a, B, ldb, fb, gb,
                    scale_inv_b, C_bf16, ldc, static_cast<hipStream_t>(stream));
}

extern "C" int fp8_grouped_gemm_tiled(int tile, int pow2, int32_t num_groups,
                                      const int64_t* group_offsets, int64_t total_M, int64_t N,
                                      int64_t K, const void* A, int64_t lda, int fa,
                                      const float* scale_inv_a, const void* B, int64_t ldb,
                                      int fb, const float* scale_inv_b, void* C_bf16,
                                      int64_t ldc, void* stream) {
  if (!grouped_tile_ok(tile) || (pow2 != 0 && pow2 != 1)) return FP8BS_ERR_ARG;
  return gemm_grouped_entry(pow2 != 0, tile, num_groups, group_offsets, total_M, N, K, A, lda, fa,
                            scale_inv_a, B, ldb, fb, scale_inv_b, C_bf16, ldc,
                            static_cast<hipStream_t>(stream));
}
