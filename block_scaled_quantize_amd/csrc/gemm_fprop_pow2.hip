// Dense fprop kernels with power-of-2 block scales given to the MFMA as E8M0 scales (128x128 or
// 1x128 weight scales); device code in gemm_impl.h.
//
// Method: "NVIDIA NeMo RL logra una aceleración del 48% con entrenamiento de precisión FP8 de
// extremo a extremo", section "Por qué esto es importante para la economía de la IA": the option
// of power-of-2 scale factors; with them the block scales are exact exponents.
#include "gemm_impl.h"

namespace fp8bs {

int gemm_fprop_pow2(int sm, int fa, int fb, const GemmParams& p, int tile, hipStream_t st) {
  switch (sm) {
    case kScaleHw: return dispatch_formats<FP8BS_FPROP, kScaleHw>(fa, fb, p, tile, st);
    case kScaleHwRows: return dispatch_formats<FP8BS_FPROP, kScaleHwRows>(fa, fb, p, tile, st);
    default: return FP8BS_ERR_UNSUPPORTED;
  }
}

}  // namespace fp8bs
