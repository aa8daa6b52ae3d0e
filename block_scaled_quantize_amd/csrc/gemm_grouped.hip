// Grouped (MoE) GEMM kernels: fp32 block scales folded between K blocks, or power-of-2 scales
// given to the MFMA as E8M0 scales; device code in gemm_impl.h.
//
// Method: "NVIDIA NeMo RL logra una aceleración del 48% con entrenamiento de precisión FP8 de
// extremo a extremo", section "Ganancias de rendimiento en el mundo real" (the FP8 recipe on an
// MoE model's experts) and section "Por qué esto es importante para la economía de la IA"
// (power-of-2 scales).
#include "gemm_impl.h"

namespace fp8bs {

int gemm_grouped(bool pow2, int fa, int fb, int cus, const GemmParams& p, int tile,
                 hipStream_t st) {
  return pow2 ? dispatch_grouped<kScaleHw>(fa, fb, cus, p, tile, st)
              : dispatch_grouped<kScaleFold>(fa, fb, cus, p, tile, st);
}

}  // namespace fp8bs
