// Columnwise (128x1) FP8 quantization with transposed output, for gfx950.
//
// Method: "NVIDIA NeMo RL logra una aceleración del 48% con entrenamiento de precisión FP8 de
// extremo a extremo", section "El avance técnico": activations carry one scale per 128
// consecutive elements along the dimension a GEMM contracts.  The weight gradient contracts
// over tokens, so there the blocks of an activation or gradient X[tokens, features] run down a
// column: 128 consecutive rows of one column.  This kernel computes those blocks and writes the
// codes of X transposed, [features][tokens], so the weight-gradient GEMM reads them K-major
// (tokens contiguous) with the scales in the 1x128 layout of the transposed matrix:
// scale_inv[row block][column].  Scale rule, rounding, saturation and NaN handling are those
// of the blockwise quantizer (power-of-2 option: section "Por qué esto es importante para la
// economía de la IA").
//
// Design (HBM-bound, one pass): a workgroup of 256 lanes takes a 128-row x 128-column tile;
// lane (row group g, column chunk c) loads rows 8g .. 8g+7 of columns 8c .. 8c+7 with 16-byte
// loads, so each lane ends with the 8 codes of 8 consecutive rows per column.  The column
// maxima are reduced over the lane's 8 rows in registers (packed 16-bit max of magnitude bits),
// across the 4 row groups of a wave by lane shuffles and across the 4 waves through 1 KiB of
// LDS.  The codes are staged in LDS as [column][row] (column pitch 136 bytes, so the 8-byte
// writes of a wave spread over the banks) and leave as whole 128-byte rows of the transposed
// matrix, 16 bytes per lane.
//
// The microscaling form (fp8_quantize_mx_columnwise_t) takes blocks of 32 rows of one column
// with E8M0 scale bytes ("Infraestructura de Entrenamiento FP8: Precisión Numérica de Nueva
// Generación", sections "Estrategias de escalado y estabilidad" and "Blackwell MXFP8 y NVFP4:
// mirando hacia adelante"): the weight- and data-gradient operands of the microscaling GEMM.
#include <float.h>

#include "common.h"

namespace fp8bs {
namespace {

constexpr int kThreadsT = 256;

// 8 consecutive bf16 of row r from column c on (elements outside the matrix read as +0).
// VEC: 16-byte aligned rows.
template <bool VEC>
__device__ __forceinline__ uint4 load8(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                       int64_t ld, int64_t r, int64_t c) {
  if (r >= rows || c >= cols) return make_uint4(0u, 0u, 0u, 0u);
  const uint16_t* p = x + r * ld + c;
  if (VEC && c + 8 <= cols) return *reinterpret_cast<const uint4*>(p);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (c + 2 * i < cols) ? (uint32_t)p[2 * i] : 0u;
    const uint32_t hi = (c + 2 * i + 1 < cols) ? (uint32_t)p[2 * i + 1] : 0u;
    w[i] = lo | (hi << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// ROWS: the same pass also quantizes x in 1x128 blocks along its rows (fp8_quantize_blockwise's
// codes q[rows][ld_q] and scales scale_inv_rows[ceil(cols/128)][rows]): a tile row spans the 16
// lanes of one row group -- one DPP row of the wave -- 8 columns each, so its maximum is four
// DPP steps, and each lane stores its 8 codes of the row as one 8-byte run.
template <int FMT, bool POW2, bool VEC, bool ROWS = false>
__global__ __launch_bounds__(kThreadsT) void quant_128x1_t_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ qt, int64_t ld_qt, float* __restrict__ scale_inv,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scale_inv_rows) {
  __shared__ uint32_t s_max[4][16][4];   // [wave][column chunk][column pair], packed 16-bit
  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const int cg = t & 15, rg = t >> 4;
  const int64_t nbc = (cols + 127) >> 7;
  const int64_t rb = blockIdx.x / nbc, cb = blockIdx.x % nbc;
  const int64_t r0 = rb * 128 + 8 * rg;
  const int64_t c0 = cb * 128 + 8 * cg;

  uint32_t d[8][4];   // d[k][p]: row r0 + k, columns c0 + 2p (low half) and c0 + 2p + 1
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint4 v = load8<VEC>(x, rows, cols, ld_x, r0 + k, c0);
    d[k][0] = v.x; d[k][1] = v.y; d[k][2] = v.z; d[k][3] = v.w;
  }

  if constexpr (ROWS) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t r = r0 + k;
      uint32_t a = hmax(max2(max2(mag2(d[k][0]), mag2(d[k][1])), max2(mag2(d[k][2]), mag2(d[k][3]))));
      a = group8_max(a);
      const uint32_t o = __builtin_amdgcn_mov_dpp(a, 0x140, 0xF, 0xF, false);   // row_mirror
      a = a > o ? a : o;
      const float sr = scale_from_amax_bits<FMT, POW2>(a);
      float y[8];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        y[2 * p] = bf16_lo(d[k][p]) * sr;
        y[2 * p + 1] = bf16_hi(d[k][p]) * sr;
      }
      const bool fin = a < 0x7F80u;
      if (!fin) {
        constexpr float F = Format<FMT>::fmax;
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = __builtin_amdgcn_fmed3f(y[i], -F, F);
      }
      uint32_t lo = cvt4<FMT>(y[0], y[1], y[2], y[3]);
      uint32_t hi = cvt4<FMT>(y[4], y[5], y[6], y[7]);
      if (!fin) {
        lo = patch_nan_pair(patch_nan_pair(lo, d[k][0], 0), d[k][1], 1);
        hi = patch_nan_pair(patch_nan_pair(hi, d[k][2], 0), d[k][3], 1);
      }
      if (r < rows && c0 < cols) {
        uint8_t* dst = q + r * ld_q + c0;
        if (VEC && c0 + 8 <= cols) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (c0 + i < cols) dst[i] = (uint8_t)((i < 4 ? lo : hi) >> (8 * (i & 3)));
        }
        if (cg == 0) scale_inv_rows[cb * rows + r] = 1.0f / sr;
      }
    }
  }

  // Column maxima: over this lane's 8 rows, then over the wave's 4 row groups (lanes that
  // differ in bits 4 and 5 share the column chunk), then over the 4 waves.
  uint32_t m[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    u16x2 v = mag2(d[0][p]);
#pragma unroll
    for (int k = 1; k < 8; ++k) v = max2(v, mag2(d[k][p]));
    uint32_t b = __builtin_bit_cast(uint32_t, v);
    b = __builtin_bit_cast(uint32_t, max2(__builtin_bit_cast(u16x2, b),
                                           __builtin_bit_cast(u16x2, (uint32_t)__shfl_xor((int)b, 16))));
    b = __builtin_bit_cast(uint32_t, max2(__builtin_bit_cast(u16x2, b),
                                           __builtin_bit_cast(u16x2, (uint32_t)__shfl_xor((int)b, 32))));
    m[p] = b;
  }
  if (lane < 16) {
#pragma unroll
    for (int p = 0; p < 4; ++p) s_max[wv][cg][p] = m[p];
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    u16x2 v = __builtin_bit_cast(u16x2, s_max[0][cg][p]);
#pragma unroll
    for (int w = 1; w < 4; ++w) v = max2(v, __builtin_bit_cast(u16x2, s_max[w][cg][p]));
    m[p] = __builtin_bit_cast(uint32_t, v);
  }

  float s[8];
  bool finite = true;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t a = (j & 1) ? (m[j >> 1] >> 16) : (m[j >> 1] & 0xFFFFu);
    s[j] = scale_from_amax_bits<FMT, POW2>(a);
    finite = finite && a < 0x7F80u;
  }

  // Encode column by column into an LDS tile [128 columns][128 rows] (column pitch 136 bytes),
  // then write whole 128-byte column rows of the transposed matrix, 16 bytes per lane.
  __shared__ __attribute__((aligned(16))) uint8_t s_t[128 * 136];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int p = j >> 1;
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = ((j & 1) ? bf16_hi(d[k][p]) : bf16_lo(d[k][p])) * s[j];
    if (!finite) {
      constexpr float F = Format<FMT>::fmax;
#pragma unroll
      for (int k = 0; k < 8; ++k) y[k] = __builtin_amdgcn_fmed3f(y[k], -F, F);
    }
    uint32_t lo = cvt4<FMT>(y[0], y[1], y[2], y[3]);
    uint32_t hi = cvt4<FMT>(y[4], y[5], y[6], y[7]);
    if (!finite) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t b = ((j & 1) ? (d[k][p] >> 16) : d[k][p]) & 0xFFFFu;
        if ((b & 0x7FFFu) > 0x7F80u) {
          const uint32_t code = 0x7Fu | ((b >> 8) & 0x80u);
          const int sh = 8 * (k & 3);
          if (k < 4) lo = (lo & ~(0xFFu << sh)) | (code << sh);
          else hi = (hi & ~(0xFFu << sh)) | (code << sh);
        }
      }
    }
    *reinterpret_cast<uint2*>(s_t + (8 * cg + j) * 136 + 8 * rg) = make_uint2(lo, hi);
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int col = (t >> 3) + 32 * u, chunk = t & 7;
    const int64_t c = cb * 128 + col;
    const int64_t r = rb * 128 + 16 * chunk;
    if (c >= cols || r >= rows) continue;
    const uint8_t* src = s_t + col * 136 + 16 * chunk;
    const uint2 a = *reinterpret_cast<const uint2*>(src);
    const uint2 b = *reinterpret_cast<const uint2*>(src + 8);
    uint8_t* dst = qt + c * ld_qt + r;
    if (VEC && r + 16 <= rows) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(a.x, a.y, b.x, b.y);
    } else {
      const uint32_t w4[4] = {a.x, a.y, b.x, b.y};
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (r + k < rows) dst[k] = (uint8_t)(w4[k >> 2] >> (8 * (k & 3)));
    }
  }
  if (rg == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < cols) scale_inv[rb * cols + c0 + j] = 1.0f / s[j];
  }
}

// Microscaling form (blocks of 32 rows of one column, power-of-2 scales stored as E8M0 bytes, as
// fp8_quantize_mx does along rows): the same tile, lanes and transposed code stores.  A wave's
// four row groups are exactly one 32-row block, so a column's block maximum needs only the
// shuffles inside the wave.  The E8M0 byte is 254 minus the exponent field of s (the exponent of
// 1/s), and the four blocks of a tile column (one per wave) leave as one 4-byte word at
// [128-row block][column]: the microscaling scale layout of x^T.
// ROWS: the same pass also quantizes x along its rows as fp8_quantize_mx does (codes
// q[rows][ld_q], scale words se_rows[ceil(cols/128)][rows]): a 32-column row block is one quad
// of the row group's 16 lanes (two DPP steps), and lane 0 of the row group gathers the four
// blocks' bytes of its 128 columns into one word.
template <int FMT, bool VEC, bool ROWS = false>
__global__ __launch_bounds__(kThreadsT) void quant_mx_t_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ qt, int64_t ld_qt, uint32_t* __restrict__ se,
    uint8_t* __restrict__ q, int64_t ld_q, uint32_t* __restrict__ se_rows) {
  __shared__ uint32_t s_e8[128];   // per tile column, byte w = the factor of wave w's block
  __shared__ __attribute__((aligned(16))) uint8_t s_t[128 * 136];
  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const int cg = t & 15, rg = t >> 4;
  const int64_t nbc = (cols + 127) >> 7;
  const int64_t rb = blockIdx.x / nbc, cb = blockIdx.x % nbc;
  const int64_t r0 = rb * 128 + 8 * rg;
  const int64_t c0 = cb * 128 + 8 * cg;

  uint32_t d[8][4];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint4 v = load8<VEC>(x, rows, cols, ld_x, r0 + k, c0);
    d[k][0] = v.x; d[k][1] = v.y; d[k][2] = v.z; d[k][3] = v.w;
  }
  if constexpr (ROWS) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t r = r0 + k;
      uint32_t a = hmax(max2(max2(mag2(d[k][0]), mag2(d[k][1])), max2(mag2(d[k][2]), mag2(d[k][3]))));
      uint32_t o = __builtin_amdgcn_mov_dpp(a, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
      a = a > o ? a : o;
      o = __builtin_amdgcn_mov_dpp(a, 0x4E, 0xF, 0xF, false);            // quad_perm [2,3,0,1]
      a = a > o ? a : o;
      const float sr = scale_from_amax_bits<FMT, true>(a);
      float y[8];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        y[2 * p] = bf16_lo(d[k][p]) * sr;
        y[2 * p + 1] = bf16_hi(d[k][p]) * sr;
      }
      const bool fin = a < 0x7F80u;
      if (!fin) {
        constexpr float F = Format<FMT>::fmax;
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = __builtin_amdgcn_fmed3f(y[i], -F, F);
      }
      uint32_t lo = cvt4<FMT>(y[0], y[1], y[2], y[3]);
      uint32_t hi = cvt4<FMT>(y[4], y[5], y[6], y[7]);
      if (!fin) {
        lo = patch_nan_pair(patch_nan_pair(lo, d[k][0], 0), d[k][1], 1);
        hi = patch_nan_pair(patch_nan_pair(hi, d[k][2], 0), d[k][3], 1);
      }
      // the bytes of the row's four 32-column blocks, from lanes 0, 4, 8, 12 of the row group
      const uint32_t byte = 254u - ((__float_as_uint(sr) >> 23) & 0xFFu);
      const uint32_t word = byte | ((uint32_t)__shfl_down((int)byte, 4) << 8) |
                            ((uint32_t)__shfl_down((int)byte, 8) << 16) |
                            ((uint32_t)__shfl_down((int)byte, 12) << 24);
      if (r < rows && c0 < cols) {
        uint8_t* dst = q + r * ld_q + c0;
        if (VEC && c0 + 8 <= cols) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (c0 + i < cols) dst[i] = (uint8_t)((i < 4 ? lo : hi) >> (8 * (i & 3)));
        }
        if (cg == 0) se_rows[cb * rows + r] = word;
      }
    }
  }
  uint32_t m[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    u16x2 v = mag2(d[0][p]);
#pragma unroll
    for (int k = 1; k < 8; ++k) v = max2(v, mag2(d[k][p]));
    uint32_t b = __builtin_bit_cast(uint32_t, v);
    b = __builtin_bit_cast(uint32_t, max2(__builtin_bit_cast(u16x2, b),
                                           __builtin_bit_cast(u16x2, (uint32_t)__shfl_xor((int)b, 16))));
    b = __builtin_bit_cast(uint32_t, max2(__builtin_bit_cast(u16x2, b),
                                           __builtin_bit_cast(u16x2, (uint32_t)__shfl_xor((int)b, 32))));
    m[p] = b;
  }
  float s[8];
  bool finite = true;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t a = (j & 1) ? (m[j >> 1] >> 16) : (m[j >> 1] & 0xFFFFu);
    s[j] = scale_from_amax_bits<FMT, true>(a);
    finite = finite && a < 0x7F80u;
  }
  if (lane < 16) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      reinterpret_cast<uint8_t*>(s_e8)[4 * (8 * cg + j) + wv] =
          (uint8_t)(254u - ((__float_as_uint(s[j]) >> 23) & 0xFFu));
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int p = j >> 1;
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = ((j & 1) ? bf16_hi(d[k][p]) : bf16_lo(d[k][p])) * s[j];
    if (!finite) {
      constexpr float F = Format<FMT>::fmax;
#pragma unroll
      for (int k = 0; k < 8; ++k) y[k] = __builtin_amdgcn_fmed3f(y[k], -F, F);
    }
    uint32_t lo = cvt4<FMT>(y[0], y[1], y[2], y[3]);
    uint32_t hi = cvt4<FMT>(y[4], y[5], y[6], y[7]);
    if (!finite) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t b = ((j & 1) ? (d[k][p] >> 16) : d[k][p]) & 0xFFFFu;
        if ((b & 0x7FFFu) > 0x7F80u) {
          const uint32_t code = 0x7Fu | ((b >> 8) & 0x80u);
          const int sh = 8 * (k & 3);
          if (k < 4) lo = (lo & ~(0xFFu << sh)) | (code << sh);
          else hi = (hi & ~(0xFFu << sh)) | (code << sh);
        }
      }
    }
    *reinterpret_cast<uint2*>(s_t + (8 * cg + j) * 136 + 8 * rg) = make_uint2(lo, hi);
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int col = (t >> 3) + 32 * u, chunk = t & 7;
    const int64_t c = cb * 128 + col;
    const int64_t r = rb * 128 + 16 * chunk;
    if (c >= cols || r >= rows) continue;
    const uint8_t* src = s_t + col * 136 + 16 * chunk;
    const uint2 a = *reinterpret_cast<const uint2*>(src);
    const uint2 b = *reinterpret_cast<const uint2*>(src + 8);
    uint8_t* dst = qt + c * ld_qt + r;
    if (VEC && r + 16 <= rows) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(a.x, a.y, b.x, b.y);
    } else {
      const uint32_t w4[4] = {a.x, a.y, b.x, b.y};
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (r + k < rows) dst[k] = (uint8_t)(w4[k >> 2] >> (8 * (k & 3)));
    }
  }
  if (t < 128 && cb * 128 + t < cols) se[rb * cols + cb * 128 + t] = s_e8[t];
}

template <int FMT>
int dispatch_columnwise_t(bool pow2, bool vec, const uint16_t* x, int64_t rows, int64_t cols,
                          int64_t ld_x, uint8_t* qt, int64_t ld_qt, float* s, hipStream_t st) {
  const dim3 grid((unsigned)(ceil_div(rows, 128) * ceil_div(cols, 128)));
  const dim3 block(kThreadsT);
  auto go = [&](auto kernel) {
    return launch(kernel, grid, block, st, x, rows, cols, ld_x, qt, ld_qt, s, (uint8_t*)nullptr,
                  (int64_t)0, (float*)nullptr);
  };
  if (pow2)
    return vec ? go(quant_128x1_t_kernel<FMT, true, true>) : go(quant_128x1_t_kernel<FMT, true, false>);
  return vec ? go(quant_128x1_t_kernel<FMT, false, true>) : go(quant_128x1_t_kernel<FMT, false, false>);
}

}  // namespace
}  // namespace fp8bs

using namespace fp8bs;

extern "C" int fp8_quantize_columnwise_t(const void* x_bf16, int64_t rows, int64_t cols,
                                         int64_t ld_x, int fmt, int mode, void* qt_out,
                                         int64_t ld_qt, float* scale_inv_out, void* stream) {
  if (!fmt_ok(fmt) || (mode != FP8BS_SCALE_FP32 && mode != FP8BS_SCALE_POW2)) return FP8BS_ERR_ARG;
  if (rows < 0 || cols < 0 || ld_x < cols || ld_qt < rows) return FP8BS_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP8BS_OK;
  if (!x_bf16 || !qt_out || !scale_inv_out) return FP8BS_ERR_NULL;
  if (ceil_div(rows, 128) * ceil_div(cols, 128) > 0x7FFFFFFF) return FP8BS_ERR_SHAPE;
  if (rows > INT64_MAX / ld_x || cols > INT64_MAX / ld_qt) return FP8BS_ERR_SHAPE;
  if (!aligned4(scale_inv_out)) return FP8BS_ERR_ALIGN;
  const bool vec = aligned16(x_bf16) && aligned16(qt_out) && ld_x % 8 == 0 && ld_qt % 16 == 0;
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  uint8_t* qt = static_cast<uint8_t*>(qt_out);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool pow2 = mode == FP8BS_SCALE_POW2;
  if (fmt == FP8BS_E4M3)
    return dispatch_columnwise_t<FP8BS_E4M3>(pow2, vec, x, rows, cols, ld_x, qt, ld_qt,
                                             scale_inv_out, st);
  return dispatch_columnwise_t<FP8BS_E5M2>(pow2, vec, x, rows, cols, ld_x, qt, ld_qt,
                                           scale_inv_out, st);
}

extern "C" int fp8_quantize_mx_columnwise_t(const void* x_bf16, int64_t rows, int64_t cols,
                                            int64_t ld_x, int fmt, void* qt_out, int64_t ld_qt,
                                            void* scale_e8m0_out, void* stream) {
  if (!fmt_ok(fmt)) return FP8BS_ERR_ARG;
  if (rows < 0 || cols < 0 || ld_x < cols || ld_qt < rows) return FP8BS_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP8BS_OK;
  if (!x_bf16 || !qt_out || !scale_e8m0_out) return FP8BS_ERR_NULL;
  if (ceil_div(rows, 128) * ceil_div(cols, 128) > 0x7FFFFFFF) return FP8BS_ERR_SHAPE;
  if (rows > INT64_MAX / ld_x || cols > INT64_MAX / ld_qt) return FP8BS_ERR_SHAPE;
  if (!aligned4(scale_e8m0_out)) return FP8BS_ERR_ALIGN;
  const bool vec = aligned16(x_bf16) && aligned16(qt_out) && ld_x % 8 == 0 && ld_qt % 16 == 0;
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  uint8_t* qt = static_cast<uint8_t*>(qt_out);
  uint32_t* se = static_cast<uint32_t*>(scale_e8m0_out);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(ceil_div(rows, 128) * ceil_div(cols, 128)));
  const dim3 block(kThreadsT);
  auto go = [&](auto kernel) {
    return launch(kernel, grid, block, st, x, rows, cols, ld_x, qt, ld_qt, se, (uint8_t*)nullptr,
                  (int64_t)0, (uint32_t*)nullptr);
  };
  if (fmt == FP8BS_E4M3)
    return vec ? go(quant_mx_t_kernel<FP8BS_E4M3, true>) : go(quant_mx_t_kernel<FP8BS_E4M3, false>);
  return vec ? go(quant_mx_t_kernel<FP8BS_E5M2, true>) : go(quant_mx_t_kernel<FP8BS_E5M2, false>);
}

extern "C" int fp8_quantize_mx_and_columnwise_t(const void* x_bf16, int64_t rows, int64_t cols,
                                                int64_t ld_x, int fmt, void* q_out, int64_t ld_q,
                                                void* scale_e8m0_out, void* qt_out, int64_t ld_qt,
                                                void* scale_e8m0_t_out, void* stream) {
  if (!fmt_ok(fmt)) return FP8BS_ERR_ARG;
  if (rows < 0 || cols < 0 || ld_x < cols || ld_q < cols || ld_qt < rows) return FP8BS_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP8BS_OK;
  if (!x_bf16 || !q_out || !scale_e8m0_out || !qt_out || !scale_e8m0_t_out) return FP8BS_ERR_NULL;
  if (ceil_div(rows, 128) * ceil_div(cols, 128) > 0x7FFFFFFF) return FP8BS_ERR_SHAPE;
  if (rows > INT64_MAX / ld_x || rows > INT64_MAX / ld_q || cols > INT64_MAX / ld_qt)
    return FP8BS_ERR_SHAPE;
  if (!aligned4(scale_e8m0_out) || !aligned4(scale_e8m0_t_out)) return FP8BS_ERR_ALIGN;
  const bool vec = aligned16(x_bf16) && aligned16(qt_out) && ld_x % 8 == 0 && ld_qt % 16 == 0 &&
                   (reinterpret_cast<uintptr_t>(q_out) & 7u) == 0 && ld_q % 8 == 0;
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  uint8_t* q = static_cast<uint8_t*>(q_out);
  uint8_t* qt = static_cast<uint8_t*>(qt_out);
  uint32_t* se = static_cast<uint32_t*>(scale_e8m0_out);
  uint32_t* set = static_cast<uint32_t*>(scale_e8m0_t_out);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(ceil_div(rows, 128) * ceil_div(cols, 128)));
  const dim3 block(kThreadsT);
  auto go = [&](auto kernel) {
    return launch(kernel, grid, block, st, x, rows, cols, ld_x, qt, ld_qt, set, q, ld_q, se);
  };
  if (fmt == FP8BS_E4M3)
    return vec ? go(quant_mx_t_kernel<FP8BS_E4M3, true, true>)
               : go(quant_mx_t_kernel<FP8BS_E4M3, false, true>);
  return vec ? go(quant_mx_t_kernel<FP8BS_E5M2, true, true>)
             : go(quant_mx_t_kernel<FP8BS_E5M2, false, true>);
}

extern "C" int fp8_quantize_1x128_and_columnwise_t(const void* x_bf16, int64_t rows, int64_t cols,
                                                   int64_t ld_x, int fmt, int mode, void* q_out,
                                                   int64_t ld_q, float* scale_inv_out,
                                                   void* qt_out, int64_t ld_qt,
                                                   float* scale_inv_t_out, void* stream) {
  if (!fmt_ok(fmt) || (mode != FP8BS_SCALE_FP32 && mode != FP8BS_SCALE_POW2)) return FP8BS_ERR_ARG;
  if (rows < 0 || cols < 0 || ld_x < cols || ld_q < cols || ld_qt < rows) return FP8BS_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP8BS_OK;
  if (!x_bf16 || !q_out || !scale_inv_out || !qt_out || !scale_inv_t_out) return FP8BS_ERR_NULL;
  if (ceil_div(rows, 128) * ceil_div(cols, 128) > 0x7FFFFFFF) return FP8BS_ERR_SHAPE;
  if (rows > INT64_MAX / ld_x || rows > INT64_MAX / ld_q || cols > INT64_MAX / ld_qt)
    return FP8BS_ERR_SHAPE;
  if (!aligned4(scale_inv_out) || !aligned4(scale_inv_t_out)) return FP8BS_ERR_ALIGN;
  const bool vec = aligned16(x_bf16) && aligned16(qt_out) && ld_x % 8 == 0 && ld_qt % 16 == 0 &&
                   (reinterpret_cast<uintptr_t>(q_out) & 7u) == 0 && ld_q % 8 == 0;
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  uint8_t* q = static_cast<uint8_t*>(q_out);
  uint8_t* qt = static_cast<uint8_t*>(qt_out);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(ceil_div(rows, 128) * ceil_div(cols, 128)));
  const dim3 block(kThreadsT);
  auto go = [&](auto kernel) {
    return launch(kernel, grid, block, st, x, rows, cols, ld_x, qt, ld_qt, scale_inv_t_out, q, ld_q,
                  scale_inv_out);
  };
  const bool pow2 = mode == FP8BS_SCALE_POW2;
  if (fmt == FP8BS_E4M3) {
    if (pow2) return vec ? go(quant_128x1_t_kernel<FP8BS_E4M3, true, true, true>)
                         : go(quant_128x1_t_kernel<FP8BS_E4M3, true, false, true>);
    return vec ? go(quant_128x1_t_kernel<FP8BS_E4M3, false, true, true>)
               : go(quant_128x1_t_kernel<FP8BS_E4M3, false, false, true>);
  }
  if (pow2) return vec ? go(quant_128x1_t_kernel<FP8BS_E5M2, true, true, true>)
                       : go(quant_128x1_t_kernel<FP8BS_E5M2, true, false, true>);
  return vec ? go(quant_128x1_t_kernel<FP8BS_E5M2, false, true, true>)
             : go(quant_128x1_t_kernel<FP8BS_E5M2, false, false, true>);
}
