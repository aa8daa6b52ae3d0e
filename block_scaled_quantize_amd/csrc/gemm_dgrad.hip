// Dense dgrad kernels (FP8BS_DGRAD layout) for fp32 block scales, per-tensor scales and power-of-2
// (E8M0) block scales; device code in gemm_impl.h.
#include "gemm_impl.h"

namespace fp8bs {

int gemm_dgrad(int sm, int fa, int fb, const GemmParams& p, int tile, hipStream_t st) {
  switch (sm) {
    case kScaleFold: return dispatch_formats<FP8BS_DGRAD, kScaleFold>(fa, fb, p, tile, st);
    case kScaleTensor: return dispatch_formats<FP8BS_DGRAD, kScaleTensor>(fa, fb, p, tile, st);
    case kScaleHw: return dispatch_formats<FP8BS_DGRAD, kScaleHw>(fa, fb, p, tile, st);
    default: return FP8BS_ERR_UNSUPPORTED;
  }
}

}  // namespace fp8bs
