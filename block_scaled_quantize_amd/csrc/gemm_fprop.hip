// Dense fprop kernels (C = A . B^T, both operands K-major) with fp32 block scales folded between
// K blocks, 1x128 scales on both operands, or per-tensor scales; device code in gemm_impl.h.
#include "gemm_impl.h"

namespace fp8bs {

int gemm_fprop_fp32(int sm, int fa, int fb, const GemmParams& p, int tile, hipStream_t st) {
  switch (sm) {
    case kScaleFold: return dispatch_formats<FP8BS_FPROP, kScaleFold>(fa, fb, p, tile, st);
    case kScaleTensor: return dispatch_formats<FP8BS_FPROP, kScaleTensor>(fa, fb, p, tile, st);
    case kScaleFoldRows: return dispatch_formats<FP8BS_FPROP, kScaleFoldRows>(fa, fb, p, tile, st);
    default: return FP8BS_ERR_UNSUPPORTED;
  }
}

}  // namespace fp8bs
