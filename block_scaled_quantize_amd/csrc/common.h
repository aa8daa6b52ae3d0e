// Internal device and host helpers of the FP8 library (gfx950 only).
//
// Numerics follow the formats of "Infraestructura de Entrenamiento FP8: Precisión Numérica de
// Nueva Generación", section "El panorama de la precisión numérica" (E4M3 up to +-448, E5M2
// with the wider range).  Conversion uses the gfx950 packed FP8 convert instructions, which
// round to nearest even and keep subnormals; they do not saturate (E4M3 overflows to NaN from
// 464 up, E5M2 to infinity from 61440 up) and do not always keep a NaN's sign, so callers
// clamp to +-FMAX first wherever |y| can exceed it and patch NaN codes explicitly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

#include "fp8bs.h"

namespace fp8bs {

template <int FMT>
struct Format;
template <>
struct Format<FP8BS_E4M3> {
  static constexpr float fmax = 448.0f;
  static constexpr uint32_t max_code = 0x7Eu;
};
template <>
struct Format<FP8BS_E5M2> {
  static constexpr float fmax = 57344.0f;
  static constexpr uint32_t max_code = 0x7Bu;
};

// Four fp32 values -> four codes packed little-endian (value k in byte k), hardware RNE.
template <int FMT>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  if constexpr (FMT == FP8BS_E4M3) {
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  } else {
    uint32_t w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    return __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  }
}

// bf16 pair packed in a dword -> the two fp32 values (exact).
__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// Largest bf16 magnitude pattern over a dword pair: max(bits & 0x7FFF) of both halves packed.
// Unsigned order of magnitude bits is the order of |x|; NaN patterns sort above infinity.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2 mag2(uint32_t d) {
  return __builtin_bit_cast(u16x2, d & 0x7FFF7FFFu);
}
__device__ __forceinline__ u16x2 max2(u16x2 a, u16x2 b) { return __builtin_elementwise_max(a, b); }
__device__ __forceinline__ uint32_t hmax(u16x2 a) { return a.x > a.y ? a.x : a.y; }

// Max over the 8 lanes of an aligned group (lanes 8g .. 8g+7) via DPP.
__device__ __forceinline__ uint32_t group8_max(uint32_t v) {
  uint32_t t = __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  v = v > t ? v : t;
  t = __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);           // quad_perm [2,3,0,1]
  v = v > t ? v : t;
  t = __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);          // row_half_mirror
  return v > t ? v : t;
}

// Max over a whole wave (64 lanes); the result is valid in every lane.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = group8_max(v);
  uint32_t t = __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false);  // row_mirror (16 lanes)
  v = v > t ? v : t;
  t = (uint32_t)__shfl_xor((int)v, 16);
  v = v > t ? v : t;
  t = (uint32_t)__shfl_xor((int)v, 32);
  return v > t ? v : t;
}

// Scale of a block from its largest bf16 magnitude pattern (0 .. 0x7FFF):
// amax == 0 or non-finite -> 1; s = fl32(FMAX / amax) (IEEE division); +inf -> FLT_MAX;
// power-of-2 mode keeps the exponent only, i.e. rounds s down to 2^floor(log2 s).
template <int FMT, bool POW2>
__device__ __forceinline__ float scale_from_amax_bits(uint32_t amax16) {
  if (amax16 == 0u || amax16 >= 0x7F80u) return 1.0f;
  float amax = __uint_as_float(amax16 << 16);
  float s = Format<FMT>::fmax / amax;
  if (__float_as_uint(s) == 0x7F800000u) s = __uint_as_float(0x7F7FFFFFu);
  if constexpr (POW2) s = __uint_as_float(__float_as_uint(s) & 0xFF800000u);
  return s;
}

// Same rule for an fp32 amax (delayed scaling keeps fp32 history entries).
template <int FMT>
__device__ __forceinline__ float scale_from_amax_f32(float amax, int margin, bool pow2,
                                                     float keep) {
  uint32_t b = __float_as_uint(amax);
  if (!(amax > 0.0f) || b >= 0x7F800000u) return keep;  // zero, NaN, inf: keep the old scale
  float s = Format<FMT>::fmax / amax;
  s = s / __uint_as_float((uint32_t)(127 + margin) << 23);  // exact power of two 2^margin
  if (__float_as_uint(s) == 0x7F800000u) s = __uint_as_float(0x7F7FFFFFu);
  if (pow2) s = __uint_as_float(__float_as_uint(s) & 0xFF800000u);
  return s;
}

// Replace the codes of NaN inputs by 0x7F with the input's sign.  `d` holds two bf16 inputs
// that produced bytes (2*pair, 2*pair+1) of `codes`.
__device__ __forceinline__ uint32_t patch_nan_pair(uint32_t codes, uint32_t d, int pair) {
  uint32_t lo = d & 0xFFFFu, hi = d >> 16;
  if ((lo & 0x7FFFu) > 0x7F80u)
    codes = (codes & ~(0xFFu << (16 * pair))) | ((0x7Fu | ((lo >> 8) & 0x80u)) << (16 * pair));
  if ((hi & 0x7FFFu) > 0x7F80u)
    codes = (codes & ~(0xFFu << (16 * pair + 8))) | ((0x7Fu | ((hi >> 8) & 0x80u)) << (16 * pair + 8));
  return codes;
}

// Encode 16 bf16 inputs (8 dwords) scaled by s into 16 codes (4 dwords).
// FAST: the caller guarantees every |x * s| <= FMAX * (1 + 2^-23) and no NaN/Inf input,
// which is the case for a finite block with s derived from that block's own amax: then the
// hardware convert alone is exact.  Otherwise the product is clamped to +-FMAX (saturation)
// and NaN inputs are patched.
template <int FMT, bool FAST>
__device__ __forceinline__ uint4 encode16(const uint32_t (&d)[8], float s) {
  uint32_t out[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float y0 = bf16_lo(d[2 * w]) * s, y1 = bf16_hi(d[2 * w]) * s;
    float y2 = bf16_lo(d[2 * w + 1]) * s, y3 = bf16_hi(d[2 * w + 1]) * s;
    if constexpr (!FAST) {
      constexpr float F = Format<FMT>::fmax;
      y0 = __builtin_amdgcn_fmed3f(y0, -F, F);
      y1 = __builtin_amdgcn_fmed3f(y1, -F, F);
      y2 = __builtin_amdgcn_fmed3f(y2, -F, F);
      y3 = __builtin_amdgcn_fmed3f(y3, -F, F);
    }
    out[w] = cvt4<FMT>(y0, y1, y2, y3);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// NaN patch for 16 inputs (slow path only).
__device__ __forceinline__ uint4 patch_nan16(uint4 q, const uint32_t (&d)[8]) {
  q.x = patch_nan_pair(patch_nan_pair(q.x, d[0], 0), d[1], 1);
  q.y = patch_nan_pair(patch_nan_pair(q.y, d[2], 0), d[3], 1);
  q.z = patch_nan_pair(patch_nan_pair(q.z, d[4], 0), d[5], 1);
  q.w = patch_nan_pair(patch_nan_pair(q.w, d[6], 0), d[7], 1);
  return q;
}

// Magnitude-bits maximum of 16 bf16 inputs.
__device__ __forceinline__ uint32_t amax16_bits(const uint32_t (&d)[8]) {
  u16x2 m = mag2(d[0]);
#pragma unroll
  for (int i = 1; i < 8; ++i) m = max2(m, mag2(d[i]));
  return hmax(m);
}

// ------------------------------------------------------------------ host-side helpers
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline bool fmt_ok(int f) { return f == FP8BS_E4M3 || f == FP8BS_E5M2; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Launch through hipLaunchKernel so that the status of THIS launch is returned (a pending
// error from unrelated earlier work is neither reported nor cleared).
template <typename... KArgs, typename... Args>
inline int launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                  Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<KArgs...> values(static_cast<KArgs>(args)...);
  void* ptrs[sizeof...(KArgs)];
  std::apply([&](auto&... v) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&v)), ...);
  }, values);
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0,
                                 stream);
  return e == hipSuccess ? FP8BS_OK : FP8BS_ERR_LAUNCH;
}

}  // namespace fp8bs
