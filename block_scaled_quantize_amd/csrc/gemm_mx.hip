// Dense fprop and grouped (MoE) kernels with microscaling (MXFP8) scales: one E8M0 byte per 32 K
// elements of every row of both operands, given to the MFMA lane by lane; device code in
// gemm_impl.h.
//
// Method: "Infraestructura de Entrenamiento FP8: Precisión Numérica de Nueva Generación",
// section "Estrategias de escalado y estabilidad" (block scaling, MXFP8: separate scale factors
// for blocks within a tensor) and section "Blackwell MXFP8 y NVFP4: mirando hacia adelante"
// (block scaling accelerated by the hardware).  The pages give neither the block size nor the
// scale format: 32-element blocks with E8M0 scales are the microscaling layout that the scaled
// MFMA of gfx950 consumes directly.
#include "gemm_impl.h"

namespace fp8bs {

int gemm_fprop_mx(int fa, int fb, const GemmParams& p, int tile, hipStream_t st) {
  return dispatch_formats<FP8BS_FPROP, kScaleMx>(fa, fb, p, tile, st);
}

// The grouped (MoE) form: every expert's weights carry their own scale words.
int gemm_grouped_mx(int fa, int fb, int cus, const GemmParams& p, int tile, hipStream_t st) {
  return dispatch_grouped<kScaleMx>(fa, fb, cus, p, tile, st);
}

}  // namespace fp8bs
