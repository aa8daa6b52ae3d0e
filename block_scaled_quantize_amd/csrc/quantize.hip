// FP8 quantization kernels for gfx950: blockwise (1x128 / 128x128) and per-tensor delayed.
//
// Method: "NVIDIA NeMo RL logra una aceleración del 48% con entrenamiento de precisión FP8 de
// extremo a extremo", section "El avance técnico" (E4M3 blocks: 1x128 for activations,
// 128x128 for weights) and section "Por qué esto es importante para la economía de la IA"
// (power-of-2 scales); "Infraestructura de Entrenamiento FP8: Precisión Numérica de Nueva
// Generación", section "Transformer Engine: la base de software" (delayed scaling with an amax
// history) and section "El panorama de la precisión numérica" (E4M3 / E5M2).
//
// Design (HBM-bound, one pass): each block is read once into registers, its amax is reduced
// in registers (packed 16-bit max over magnitude bits, then DPP across the lanes that share
// the block), the scale is computed in the same pass, and the scaled values are converted
// with the packed hardware FP8 convert and written once.  Every lane moves 32 bytes of input
// (two 16-byte loads) and 16 bytes of output (one 16-byte store) per 16 elements.
#include <float.h>

#include <atomic>

#include "common.h"

namespace fp8bs {
namespace {

constexpr int kThreads = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The long-row kernels write their codes with non-temporal stores when the codes alone exceed
// the 256 MB last-level cache (then they cannot stay there for the GEMM that reads them next,
// and streaming them past it measured 4% faster); smaller outputs are stored normally, since
// the next GEMM finds them in that cache (non-temporal stores measured 4% slower inside the
// 8B step).  Non-temporal loads were slower in both cases.
constexpr int64_t kNtStoreBytes = int64_t(256) << 20;

// ---------------------------------------------------------------- element access
// Load 16 consecutive bf16 of row r starting at column c0 into 8 dwords.  Elements outside the
// matrix read as +0 (they do not change an amax).  VEC: 16-byte aligned rows.
template <bool VEC>
__device__ __forceinline__ void load16(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                       int64_t ld, int64_t r, int64_t c0, uint32_t (&d)[8]) {
  if (r >= rows || c0 >= cols) {
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = 0u;
    return;
  }
  const uint16_t* p = x + r * ld + c0;
  if (VEC && c0 + 16 <= cols) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint4 b = *reinterpret_cast<const uint4*>(p + 8);
    d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w;
    d[4] = b.x; d[5] = b.y; d[6] = b.z; d[7] = b.w;
    return;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t lo = (c0 + 2 * i < cols) ? (uint32_t)p[2 * i] : 0u;
    uint32_t hi = (c0 + 2 * i + 1 < cols) ? (uint32_t)p[2 * i + 1] : 0u;
    d[i] = lo | (hi << 16);
  }
}

// Store 16 codes of row r starting at column c0 (only those inside the matrix).  NT:
// non-temporal stores.
template <bool VEC, bool NT = false>
__device__ __forceinline__ void store16(uint8_t* __restrict__ q, int64_t rows, int64_t cols,
                                        int64_t ld, int64_t r, int64_t c0, uint4 v) {
  if (r >= rows || c0 >= cols) return;
  uint8_t* p = q + r * ld + c0;
  if (VEC && c0 + 16 <= cols) {
    if constexpr (NT) {
      const u32x4 w = {v.x, v.y, v.z, v.w};
      __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
    } else {
      *reinterpret_cast<uint4*>(p) = v;
    }
    return;
  }
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (c0 + i < cols) p[i] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
}

template <int FMT>
__device__ __forceinline__ uint4 encode_block_values(const uint32_t (&d)[8], float s,
                                                     bool finite_block) {
  if (finite_block) return encode16<FMT, true>(d, s);
  return patch_nan16(encode16<FMT, false>(d, s), d);
}

// ---------------------------------------------------------------- 1x128 blocks
// Workgroup tile: kRows1 rows x one 128-column block.  8 lanes share a row block (16 elements
// each); each thread handles kRowsPerThread row blocks kRows1/kRowsPerThread rows apart.
// Scales go to scale_inv[colblock][row]: the tile's kRows1 scales are contiguous.  The 1-D
// grid runs column blocks fastest, so workgroups in flight together stream contiguous rows.
constexpr int kRowsPerThread = 1;
constexpr int kRows1 = (kThreads / 8) * kRowsPerThread;  // 32

template <int FMT, bool POW2, bool VEC>
__device__ __forceinline__ void quant_1x128_body(const uint16_t* __restrict__ x, int64_t rows,
                                                 int64_t cols, int64_t ld_x,
                                                 uint8_t* __restrict__ q, int64_t ld_q,
                                                 float* __restrict__ scale_inv, int64_t bid) {
  const int t = threadIdx.x;
  const int64_t nbc = (cols + 127) >> 7;
  const int64_t cb = bid % nbc;
  const int64_t c0 = cb * 128 + (t & 7) * 16;
  const int64_t r0 = (bid / nbc) * kRows1 + (t >> 3);
  uint32_t d[kRowsPerThread][8];
#pragma unroll
  for (int j = 0; j < kRowsPerThread; ++j)
    load16<VEC>(x, rows, cols, ld_x, r0 + j * (kThreads / 8), c0, d[j]);
#pragma unroll
  for (int j = 0; j < kRowsPerThread; ++j) {
    const int64_t r = r0 + j * (kThreads / 8);
    const uint32_t amax = group8_max(amax16_bits(d[j]));
    const float s = scale_from_amax_bits<FMT, POW2>(amax);
    const uint4 v = encode_block_values<FMT>(d[j], s, amax < 0x7F80u);
    store16<VEC>(q, rows, cols, ld_q, r, c0, v);
    if ((t & 7) == 0 && r < rows) scale_inv[cb * rows + r] = 1.0f / s;
  }
}

template <int FMT, bool POW2, bool VEC>
__global__ __launch_bounds__(kThreads) void quant_1x128_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scale_inv) {
  quant_1x128_body<FMT, POW2, VEC>(x, rows, cols, ld_x, q, ld_q, scale_inv, blockIdx.x);
}

// Long rows (a multiple of 1024 columns, 16-byte aligned rows): each wave streams 2 KiB of one
// row -- 8 consecutive 128-column blocks, 8 lanes each as above -- and a workgroup takes 4
// rows.  For the same traffic a plain copy in this geometry streams 6% faster on this GPU than
// in the 32-row tile above (every wave's accesses are one contiguous run).
constexpr int kRowsL = kThreads / 64;   // 4
template <int FMT, bool POW2, bool NTS>
__global__ __launch_bounds__(kThreads) void quant_1x128_rows_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scale_inv) {
  const int t = threadIdx.x;
  const int64_t nbc = cols >> 10;
  const int64_t bid = blockIdx.x;
  const int64_t c0 = (bid % nbc) * 1024 + (t & 63) * 16;
  const int64_t r = (bid / nbc) * kRowsL + (t >> 6);
  uint32_t d[8];
  load16<true>(x, rows, cols, ld_x, r, c0, d);
  const uint32_t amax = group8_max(amax16_bits(d));
  const float s = scale_from_amax_bits<FMT, POW2>(amax);
  store16<true, NTS>(q, rows, cols, ld_q, r, c0, encode_block_values<FMT>(d, s, amax < 0x7F80u));
  if ((t & 7) == 0 && r < rows) scale_inv[(c0 >> 7) * rows + r] = 1.0f / s;
}

// ---------------------------------------------------------------- microscaling (1x32) blocks
// The 1x128 geometry (32 rows x 128 columns per workgroup, 16 elements per lane) with a block
// per pair of lanes: the pair's amax, the power-of-2 scale, and as the stored dequantization
// factor its E8M0 byte (the binary exponent of 1/s, biased by 127).  The four bytes of a row's
// 128 columns are gathered into the group's first lane and leave as one 4-byte word at
// [column block][row] (the blocks of a column block contiguous over the rows, as the 1x128
// scales); chunks past the matrix are empty blocks: 127 (2^0).
// LONG: the long-row geometry of quant_1x128_rows_kernel (VEC, cols a multiple of 1024); NTS:
// non-temporal code stores.
template <int FMT, bool VEC, bool LONG, bool NTS>
__global__ __launch_bounds__(kThreads) void quant_mx_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, uint32_t* __restrict__ se) {
  const int t = threadIdx.x;
  const int64_t bid = blockIdx.x;
  int64_t c0, r;
  if constexpr (LONG) {
    const int64_t nbc = cols >> 10;
    c0 = (bid % nbc) * 1024 + (t & 63) * 16;
    r = (bid / nbc) * kRowsL + (t >> 6);
  } else {
    const int64_t nbc = (cols + 127) >> 7;
    c0 = (bid % nbc) * 128 + (t & 7) * 16;
    r = (bid / nbc) * kRows1 + (t >> 3);
  }
  const int64_t cb = c0 >> 7;
  uint32_t d[8];
  load16<VEC>(x, rows, cols, ld_x, r, c0, d);
  uint32_t amax = amax16_bits(d);
  const uint32_t other = __builtin_amdgcn_mov_dpp(amax, 0xB1, 0xF, 0xF, false);   // lane t ^ 1
  amax = amax > other ? amax : other;
  const float s = scale_from_amax_bits<FMT, true>(amax);
  store16<VEC, NTS>(q, rows, cols, ld_q, r, c0, encode_block_values<FMT>(d, s, amax < 0x7F80u));
  // s = 2^e with e in [-120, 127]: 1/s has the biased exponent 254 - field(s) (0 for 2^-127)
  const uint32_t code = 254u - ((__float_as_uint(s) >> 23) & 0xFFu);
  uint32_t w = code | ((uint32_t)__shfl_xor((int)code, 2) << 8);
  w |= (uint32_t)__shfl_xor((int)w, 4) << 16;
  if ((t & 7) == 0 && r < rows) se[cb * rows + r] = w;
}

// ---------------------------------------------------------------- 128x128 tiles
// One workgroup per tile.  Thread t covers columns (t % 8) * 16 .. +16 of rows
// t / 8 + 32 * i, i = 0..3; the tile amax is reduced across the workgroup through LDS.
template <int FMT, bool POW2, bool VEC>
__device__ __forceinline__ void quant_128x128_body(const uint16_t* __restrict__ x, int64_t rows,
                                                   int64_t cols, int64_t ld_x,
                                                   uint8_t* __restrict__ q, int64_t ld_q,
                                                   float* __restrict__ scale_inv, int64_t bid,
                                                   uint32_t* wave_amax) {
  const int t = threadIdx.x;
  const int64_t nbc = (cols + 127) >> 7;
  const int64_t tr = bid / nbc, tc = bid % nbc;
  const int64_t c0 = tc * 128 + (t & 7) * 16;
  const int64_t rbase = tr * 128 + (t >> 3);
  uint32_t d[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) load16<VEC>(x, rows, cols, ld_x, rbase + 32 * i, c0, d[i]);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t a = amax16_bits(d[i]);
    m = m > a ? m : a;
  }
  m = wave_max(m);
  if ((t & 63) == 0) wave_amax[t >> 6] = m;
  __syncthreads();
  uint32_t amax = wave_amax[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) amax = amax > wave_amax[w] ? amax : wave_amax[w];
  const float s = scale_from_amax_bits<FMT, POW2>(amax);
  const bool finite = amax < 0x7F80u;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    store16<VEC>(q, rows, cols, ld_q, rbase + 32 * i, c0, encode_block_values<FMT>(d[i], s, finite));
  if (t == 0) scale_inv[tr * nbc + tc] = 1.0f / s;
}

template <int FMT, bool POW2, bool VEC>
__global__ __launch_bounds__(kThreads) void quant_128x128_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scale_inv) {
  __shared__ uint32_t wave_amax[kThreads / 64];
  quant_128x128_body<FMT, POW2, VEC>(x, rows, cols, ld_x, q, ld_q, scale_inv, blockIdx.x,
                                     wave_amax);
}

// Tensors whose codes exceed the 256 MB last-level cache, rows of a multiple of 512 columns
// (16-byte aligned): a 512-lane workgroup takes 4 tiles side by side (128 rows x 512 columns)
// and stores its codes non-temporally.  Each half-wave streams 1 KiB of one row (4 tiles x 8 lanes
// x 16 elements), a wave two rows, the 8 waves 16 rows per pass, 8 passes; a lane keeps its 8
// pieces (one per pass) in registers until the tiles' maxima are known.  Tile maxima: over the
// lane's pieces, the 8 lanes of the tile's row segment (DPP), the two half-waves (one shuffle)
// and the 8 waves (LDS).  Measured 10-12% faster than the 32-row tiles from 512M elements up,
// but 8-11% slower at 16M (a quarter as many workgroups: one per CU), about equal at 128M.
constexpr int kThreadsW = 512;
template <int FMT, bool POW2, bool NTS>
__global__ __launch_bounds__(kThreadsW) void quant_128x128_wide_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scale_inv) {
  __shared__ uint32_t s_amax[kThreadsW / 64][4];
  const int t = threadIdx.x;
  const int w = t >> 6, h = (t >> 5) & 1, li = t & 31;
  const int64_t nbc = cols >> 9;                       // 512-column groups
  const int64_t tr = blockIdx.x / nbc, cg = blockIdx.x % nbc;
  const int64_t c0 = cg * 512 + li * 16;
  const int64_t r0 = tr * 128 + 2 * w + h;
  uint32_t d[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) load16<true>(x, rows, cols, ld_x, r0 + 16 * i, c0, d[i]);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t a = amax16_bits(d[i]);
    m = m > a ? m : a;
  }
  m = group8_max(m);
  const uint32_t o = (uint32_t)__shfl_xor((int)m, 32);
  m = m > o ? m : o;
  if ((t & 39) == 0) s_amax[w][li >> 3] = m;          // lanes 0, 8, 16, 24 of the wave
  __syncthreads();
  uint32_t amax = s_amax[0][li >> 3];
#pragma unroll
  for (int v = 1; v < kThreadsW / 64; ++v) amax = amax > s_amax[v][li >> 3] ? amax : s_amax[v][li >> 3];
  const float s = scale_from_amax_bits<FMT, POW2>(amax);
  const bool finite = amax < 0x7F80u;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    store16<true, NTS>(q, rows, cols, ld_q, r0 + 16 * i, c0, encode_block_values<FMT>(d[i], s, finite));
  if (t < 32 && (t & 7) == 0) scale_inv[tr * (cols >> 7) + cg * 4 + (t >> 3)] = 1.0f / s;
}

// ---------------------------------------------------------------- several tensors, one launch
// Up to kMaxBatch tensors quantized by one grid: workgroup b belongs to the tensor whose range
// of the prefix-summed workgroup counts holds b and runs that tensor's 1x128 or 128x128 body
// (the same code as the single-tensor kernels, so the results are identical).  One launch for
// all of a step's weights spares the ramp and tail of each small launch.
constexpr int kMaxBatch = 16;

struct QuantTensor {
  const uint16_t* x;
  int64_t rows, cols, ld_x;
  uint8_t* q;
  int64_t ld_q;
  float* s;
  int64_t first;   // first workgroup of the tensor
  int gran, vec;
};
struct QuantBatch {
  QuantTensor t[kMaxBatch];
  int count;
};

template <int FMT, bool POW2>
__global__ __launch_bounds__(kThreads) void quant_batched_kernel(QuantBatch b) {
  __shared__ uint32_t wave_amax[kThreads / 64];
  const int64_t bid = blockIdx.x;
  int k = 0;
  for (int i = 1; i < b.count; ++i)
    if (b.t[i].first <= bid) k = i;
  const QuantTensor& t = b.t[k];
  const int64_t local = bid - t.first;
  if (t.gran == FP8BS_BLOCK_1x128) {
    if (t.vec) quant_1x128_body<FMT, POW2, true>(t.x, t.rows, t.cols, t.ld_x, t.q, t.ld_q, t.s, local);
    else quant_1x128_body<FMT, POW2, false>(t.x, t.rows, t.cols, t.ld_x, t.q, t.ld_q, t.s, local);
  } else {
    if (t.vec) quant_128x128_body<FMT, POW2, true>(t.x, t.rows, t.cols, t.ld_x, t.q, t.ld_q, t.s, local, wave_amax);
    else quant_128x128_body<FMT, POW2, false>(t.x, t.rows, t.cols, t.ld_x, t.q, t.ld_q, t.s, local, wave_amax);
  }
}

// ---------------------------------------------------------------- delayed per-tensor
// Pass 1: cast with the scale held in the state and reduce this tensor's amax into one
// partial per workgroup (no atomics, so the result is deterministic).  Grid-stride loop over
// 16-element chunks; the grid is capped at kDelayedBlocks workgroups.
constexpr int kDelayedBlocks = 2048;

template <int FMT, bool VEC>
__global__ __launch_bounds__(kThreads) void delayed_cast_kernel(
    const uint16_t* __restrict__ x, int64_t numel, const float* __restrict__ scale,
    uint8_t* __restrict__ q, uint32_t* __restrict__ partial) {
  __shared__ uint32_t wave_amax[kThreads / 64];
  const float s = *scale;
  const int64_t nchunks = (numel + 15) / 16;
  uint32_t m = 0;
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < nchunks;
       c += (int64_t)gridDim.x * kThreads) {
    uint32_t d[8];
    load16<VEC>(x, 1, numel, numel, 0, c * 16, d);
    const uint32_t a = amax16_bits(d);
    m = m > a ? m : a;
    uint4 v = encode16<FMT, false>(d, s);
    if (a > 0x7F80u) v = patch_nan16(v, d);
    store16<VEC>(q, 1, numel, numel, 0, c * 16, v);
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) wave_amax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = wave_amax[0];
    for (int w = 1; w < kThreads / 64; ++w) r = r > wave_amax[w] ? r : wave_amax[w];
    partial[blockIdx.x] = r;
  }
}

// Pass 2 (one workgroup): reduce the partials, push the amax into the history (newest first),
// reduce the history with "max" and derive the scale for the next step.
template <int FMT>
__global__ __launch_bounds__(kThreads) void delayed_finalize_kernel(
    const uint32_t* __restrict__ partial, int nparts, int margin, int pow2, int hist_len,
    float* __restrict__ history, float* __restrict__ scale, float* __restrict__ scale_inv_used) {
  __shared__ uint32_t red[kThreads / 64];
  __shared__ float hist_max[kThreads / 64];
  __shared__ int hist_nan[kThreads / 64];
  const int t = threadIdx.x;
  uint32_t m = 0;
  for (int i = t; i < nparts; i += kThreads) m = m > partial[i] ? m : partial[i];
  m = wave_max(m);
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  uint32_t a16 = red[0];
  for (int w = 1; w < kThreads / 64; ++w) a16 = a16 > red[w] ? a16 : red[w];
  const float a = __uint_as_float(a16 << 16);   // NaN pattern if any input was NaN
  const float s_old = *scale;

  // Shift the history by one (read everything before anyone writes).
  float mine[4];
  int cnt = 0;
  for (int i = t; i < hist_len && cnt < 4; i += kThreads, ++cnt) mine[cnt] = i == 0 ? a : history[i - 1];
  __syncthreads();
  float hm = 0.0f;
  int hn = 0;
  cnt = 0;
  for (int i = t; i < hist_len && cnt < 4; i += kThreads, ++cnt) {
    history[i] = mine[cnt];
    const float v = mine[cnt];
    if (v != v) hn = 1;
    else if (v > hm) hm = v;
  }
  // block-reduce max and NaN flag
  for (int off = 32; off >= 1; off >>= 1) {
    float o = __shfl_xor(hm, off);
    hm = hm > o ? hm : o;
    hn |= __shfl_xor(hn, off);
  }
  if ((t & 63) == 0) {
    hist_max[t >> 6] = hm;
    hist_nan[t >> 6] = hn;
  }
  __syncthreads();
  if (t == 0) {
    float r = hist_max[0];
    int nan = hist_nan[0];
    for (int w = 1; w < kThreads / 64; ++w) {
      r = r > hist_max[w] ? r : hist_max[w];
      nan |= hist_nan[w];
    }
    *scale_inv_used = 1.0f / s_old;
    *scale = nan ? s_old : scale_from_amax_f32<FMT>(r, margin, pow2 != 0, s_old);
  }
}

// ---------------------------------------------------------------- plain cast of fp32
template <int FMT>
__global__ __launch_bounds__(kThreads) void cast_fp32_kernel(const float* __restrict__ x,
                                                            int64_t n, uint8_t* __restrict__ q) {
  const int64_t n4 = (n + 3) / 4;
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < n4;
       c += (int64_t)gridDim.x * kThreads) {
    float v[4];
    const int64_t i0 = c * 4;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = i0 + k < n ? x[i0 + k] : 0.0f;
    constexpr float F = Format<FMT>::fmax;
    uint32_t w = cvt4<FMT>(__builtin_amdgcn_fmed3f(v[0], -F, F), __builtin_amdgcn_fmed3f(v[1], -F, F),
                           __builtin_amdgcn_fmed3f(v[2], -F, F), __builtin_amdgcn_fmed3f(v[3], -F, F));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t b = __float_as_uint(v[k]);
      if ((b & 0x7FFFFFFFu) > 0x7F800000u)
        w = (w & ~(0xFFu << (8 * k))) | ((0x7Fu | ((b >> 24) & 0x80u)) << (8 * k));
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (i0 + k < n) q[i0 + k] = (uint8_t)(w >> (8 * k));
  }
}

template <int FMT, bool POW2, bool VEC>
int launch_blockwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int gran,
                     uint8_t* q, int64_t ld_q, float* s, hipStream_t st) {
  if (gran == FP8BS_BLOCK_1x128) {
    if (VEC && cols % 1024 == 0) {
      dim3 grid((unsigned)(ceil_div(rows, kRowsL) * (cols >> 10)));
      if (rows * cols > kNtStoreBytes)
        return launch(quant_1x128_rows_kernel<FMT, POW2, true>, grid, dim3(kThreads), st, x, rows,
                      cols, ld_x, q, ld_q, s);
      return launch(quant_1x128_rows_kernel<FMT, POW2, false>, grid, dim3(kThreads), st, x, rows,
                    cols, ld_x, q, ld_q, s);
    }
    dim3 grid((unsigned)(ceil_div(rows, kRows1) * ceil_div(cols, 128)));
    return launch(quant_1x128_kernel<FMT, POW2, VEC>, grid, dim3(kThreads), st, x, rows, cols,
                  ld_x, q, ld_q, s);
  }
  if (VEC && cols % 512 == 0 && rows * cols > kNtStoreBytes) {
    dim3 grid((unsigned)(ceil_div(rows, 128) * (cols >> 9)));
    return launch(quant_128x128_wide_kernel<FMT, POW2, true>, grid, dim3(kThreadsW), st, x, rows,
                  cols, ld_x, q, ld_q, s);
  }
  dim3 grid((unsigned)(ceil_div(rows, 128) * ceil_div(cols, 128)));
  return launch(quant_128x128_kernel<FMT, POW2, VEC>, grid, dim3(kThreads), st, x, rows, cols,
                ld_x, q, ld_q, s);
}

template <int FMT>
int dispatch_blockwise(bool pow2, bool vec, const uint16_t* x, int64_t rows, int64_t cols,
                       int64_t ld_x, int gran, uint8_t* q, int64_t ld_q, float* s,
                       hipStream_t st) {
  if (pow2)
    return vec ? launch_blockwise<FMT, true, true>(x, rows, cols, ld_x, gran, q, ld_q, s, st)
               : launch_blockwise<FMT, true, false>(x, rows, cols, ld_x, gran, q, ld_q, s, st);
  return vec ? launch_blockwise<FMT, false, true>(x, rows, cols, ld_x, gran, q, ld_q, s, st)
             : launch_blockwise<FMT, false, false>(x, rows, cols, ld_x, gran, q, ld_q, s, st);
}

}  // namespace
}  // namespace fp8bs

using namespace fp8bs;

extern "C" int fp8_quantize_mx(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                               int fmt, void* q_out, int64_t ld_q, void* scale_e8m0_out,
                               void* stream) {
  if (!fmt_ok(fmt)) return FP8BS_ERR_ARG;
  if (rows < 0 || cols < 0 || ld_x < cols || ld_q < cols) return FP8BS_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP8BS_OK;
  if (!x_bf16 || !q_out || !scale_e8m0_out) return FP8BS_ERR_NULL;
  if (ceil_div(rows, kRows1) * ceil_div(cols, 128) > 0x7FFFFFFF ||
      ceil_div(rows, kRowsL) * ceil_div(cols, 1024) > 0x7FFFFFFF)
    return FP8BS_ERR_SHAPE;
  if (rows > INT64_MAX / ld_x || rows > INT64_MAX / ld_q) return FP8BS_ERR_SHAPE;
  if (!aligned4(scale_e8m0_out)) return FP8BS_ERR_ALIGN;
  const bool vec = aligned16(x_bf16) && aligned16(q_out) && ld_x % 8 == 0 && ld_q % 16 == 0;
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  uint8_t* q = static_cast<uint8_t*>(q_out);
  uint32_t* se = static_cast<uint32_t*>(scale_e8m0_out);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool long_rows = vec && cols % 1024 == 0;
  const dim3 grid((unsigned)(long_rows ? ceil_div(rows, kRowsL) * (cols >> 10)
                                       : ceil_div(rows, kRows1) * ceil_div(cols, 128)));
  auto go = [&](auto kernel) { return launch(kernel, grid, dim3(kThreads), st, x, rows, cols, ld_x, q, ld_q, se); };
  const bool nts = long_rows && rows * cols > kNtStoreBytes;
  if (fmt == FP8BS_E4M3)
    return nts       ? go(quant_mx_kernel<FP8BS_E4M3, true, true, true>)
           : long_rows ? go(quant_mx_kernel<FP8BS_E4M3, true, true, false>)
           : vec     ? go(quant_mx_kernel<FP8BS_E4M3, true, false, false>)
                     : go(quant_mx_kernel<FP8BS_E4M3, false, false, false>);
  return nts       ? go(quant_mx_kernel<FP8BS_E5M2, true, true, true>)
         : long_rows ? go(quant_mx_kernel<FP8BS_E5M2, true, true, false>)
         : vec     ? go(quant_mx_kernel<FP8BS_E5M2, true, false, false>)
                   : go(quant_mx_kernel<FP8BS_E5M2, false, false, false>);
}

extern "C" int fp8_quantize_blockwise(const void* x_bf16, int64_t rows, int64_t cols,
                                      int64_t ld_x, int fmt, int gran, int mode, void* q_out,
                                      int64_t ld_q, float* scale_inv_out, void* stream) {
  if (!fmt_ok(fmt) || (gran != FP8BS_BLOCK_1x128 && gran != FP8BS_BLOCK_128x128) ||
      (mode != FP8BS_SCALE_FP32 && mode != FP8BS_SCALE_POW2))
    return FP8BS_ERR_ARG;
  if (rows < 0 || cols < 0 || ld_x < cols || ld_q < cols) return FP8BS_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP8BS_OK;
  if (!x_bf16 || !q_out || !scale_inv_out) return FP8BS_ERR_NULL;
  const int64_t nb_rows = gran == FP8BS_BLOCK_1x128 ? ceil_div(rows, kRows1) : ceil_div(rows, 128);
  if (nb_rows * ceil_div(cols, 128) > 0x7FFFFFFF) return FP8BS_ERR_SHAPE;
  if (gran == FP8BS_BLOCK_1x128 && ceil_div(rows, kRowsL) * ceil_div(cols, 1024) > 0x7FFFFFFF)
    return FP8BS_ERR_SHAPE;
  if (rows > INT64_MAX / ld_x) return FP8BS_ERR_SHAPE;
  if (!aligned4(scale_inv_out)) return FP8BS_ERR_ALIGN;
  const bool vec = aligned16(x_bf16) && aligned16(q_out) && ld_x % 8 == 0 && ld_q % 16 == 0;
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  uint8_t* q = static_cast<uint8_t*>(q_out);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool pow2 = mode == FP8BS_SCALE_POW2;
  if (fmt == FP8BS_E4M3)
    return dispatch_blockwise<FP8BS_E4M3>(pow2, vec, x, rows, cols, ld_x, gran, q, ld_q,
                                          scale_inv_out, st);
  return dispatch_blockwise<FP8BS_E5M2>(pow2, vec, x, rows, cols, ld_x, gran, q, ld_q,
                                        scale_inv_out, st);
}

extern "C" int fp8_quantize_blockwise_batched(int count, const void* const* x_bf16,
                                              const int64_t* rows, const int64_t* cols,
                                              const int64_t* ld_x, const int* gran, int fmt,
                                              int mode, void* const* q_out, const int64_t* ld_q,
                                              float* const* scale_inv_out, void* stream) {
  if (!fmt_ok(fmt) || (mode != FP8BS_SCALE_FP32 && mode != FP8BS_SCALE_POW2) || count < 0 ||
      count > kMaxBatch)
    return FP8BS_ERR_ARG;
  if (count == 0) return FP8BS_OK;
  if (!x_bf16 || !rows || !cols || !ld_x || !gran || !q_out || !ld_q || !scale_inv_out)
    return FP8BS_ERR_NULL;
  QuantBatch b{};
  int64_t total = 0;
  for (int i = 0; i < count; ++i) {
    const int64_t r = rows[i], c = cols[i];
    if (gran[i] != FP8BS_BLOCK_1x128 && gran[i] != FP8BS_BLOCK_128x128) return FP8BS_ERR_ARG;
    if (r < 0 || c < 0 || ld_x[i] < c || ld_q[i] < c) return FP8BS_ERR_SHAPE;
    if (r > 0 && c > 0) {
      if (!x_bf16[i] || !q_out[i] || !scale_inv_out[i]) return FP8BS_ERR_NULL;
      if (r > INT64_MAX / ld_x[i]) return FP8BS_ERR_SHAPE;
      if (!aligned4(scale_inv_out[i])) return FP8BS_ERR_ALIGN;
    }
    QuantTensor& t = b.t[b.count];
    const int64_t nb_rows = gran[i] == FP8BS_BLOCK_1x128 ? ceil_div(r, kRows1) : ceil_div(r, 128);
    const int64_t blocks = (r > 0 && c > 0) ? nb_rows * ceil_div(c, 128) : 0;
    if (blocks == 0) continue;   // an empty tensor takes no workgroup
    t.x = static_cast<const uint16_t*>(x_bf16[i]);
    t.rows = r; t.cols = c; t.ld_x = ld_x[i];
    t.q = static_cast<uint8_t*>(q_out[i]);
    t.ld_q = ld_q[i];
    t.s = scale_inv_out[i];
    t.first = total;
    t.gran = gran[i];
    t.vec = aligned16(x_bf16[i]) && aligned16(q_out[i]) && ld_x[i] % 8 == 0 && ld_q[i] % 16 == 0;
    total += blocks;
    ++b.count;
  }
  if (total > 0x7FFFFFFF) return FP8BS_ERR_SHAPE;
  if (total == 0) return FP8BS_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)total), block(kThreads);
  const bool pow2 = mode == FP8BS_SCALE_POW2;
  if (fmt == FP8BS_E4M3)
    return pow2 ? launch(quant_batched_kernel<FP8BS_E4M3, true>, grid, block, st, b)
                : launch(quant_batched_kernel<FP8BS_E4M3, false>, grid, block, st, b);
  return pow2 ? launch(quant_batched_kernel<FP8BS_E5M2, true>, grid, block, st, b)
              : launch(quant_batched_kernel<FP8BS_E5M2, false>, grid, block, st, b);
}

extern "C" size_t fp8_quantize_delayed_workspace_size(void) {
  return sizeof(uint32_t) * kDelayedBlocks;
}

namespace fp8bs {
namespace {

// Argument checks shared by the delayed entry points (the workspace is checked by the caller).
int delayed_args_ok(const void* x_bf16, int64_t numel, int fmt, int mode, int margin,
                    int hist_len, const float* amax_history, const float* scale, const void* q_out,
                    const float* scale_inv_used) {
  if (!fmt_ok(fmt) || (mode != FP8BS_SCALE_FP32 && mode != FP8BS_SCALE_POW2) ||
      hist_len < 1 || hist_len > 1024 || margin < 0 || margin > 64)
    return FP8BS_ERR_ARG;
  if (numel < 0) return FP8BS_ERR_SHAPE;
  if (!amax_history || !scale || !scale_inv_used || (numel > 0 && (!x_bf16 || !q_out)))
    return FP8BS_ERR_NULL;
  if (!aligned4(amax_history) || !aligned4(scale) || !aligned4(scale_inv_used))
    return FP8BS_ERR_ALIGN;
  return FP8BS_OK;
}

// Cast + finalize of one delayed step; `part` holds at least delayed_blocks(numel) words.
int delayed_blocks(int64_t numel) {
  const int64_t nchunks = (numel + 15) / 16;
  return (int)std::min<int64_t>(kDelayedBlocks, std::max<int64_t>(1, ceil_div(nchunks, kThreads)));
}

int delayed_launch(const void* x_bf16, int64_t numel, int fmt, int mode, int margin,
                   int hist_len, float* amax_history, float* scale, void* q_out,
                   float* scale_inv_used, uint32_t* part, hipStream_t st) {
  const int blocks = delayed_blocks(numel);
  const bool vec = aligned16(x_bf16) && aligned16(q_out);
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  uint8_t* q = static_cast<uint8_t*>(q_out);
  int rc;
  if (fmt == FP8BS_E4M3)
    rc = vec ? launch(delayed_cast_kernel<FP8BS_E4M3, true>, dim3(blocks), dim3(kThreads), st, x, numel, scale, q, part)
             : launch(delayed_cast_kernel<FP8BS_E4M3, false>, dim3(blocks), dim3(kThreads), st, x, numel, scale, q, part);
  else
    rc = vec ? launch(delayed_cast_kernel<FP8BS_E5M2, true>, dim3(blocks), dim3(kThreads), st, x, numel, scale, q, part)
             : launch(delayed_cast_kernel<FP8BS_E5M2, false>, dim3(blocks), dim3(kThreads), st, x, numel, scale, q, part);
  if (rc != FP8BS_OK) return rc;
  const int pow2 = mode == FP8BS_SCALE_POW2;
  if (fmt == FP8BS_E4M3)
    return launch(delayed_finalize_kernel<FP8BS_E4M3>, dim3(1), dim3(kThreads), st,
                  (const uint32_t*)part, blocks, margin, pow2, hist_len, amax_history, scale,
                  scale_inv_used);
  return launch(delayed_finalize_kernel<FP8BS_E5M2>, dim3(1), dim3(kThreads), st,
                (const uint32_t*)part, blocks, margin, pow2, hist_len, amax_history, scale,
                scale_inv_used);
}

// Scratch memory of fp8_quantize_delayed_noalloc: the cast kernel's per-workgroup amax partials
// (one word per workgroup; the cast grid never exceeds kDelayedBlocks workgroups, so its size
// does not depend on the tensor).  Each device holds its own copy; host code reaches it only
// through the address hipGetSymbolAddress returns on that device (the array's name is a host
// stand-in there, not a device address).
constexpr int kScratchWords = kDelayedBlocks;
__device__ __align__(256) uint32_t scratch[kScratchWords];

constexpr int kMaxDevices = 64;
std::atomic<uint32_t*> g_scratch[kMaxDevices];

// The device address of `scratch` on the current device, looked up on the first call there.
uint32_t* scratch_on_current_device(int* status) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = FP8BS_ERR_LAUNCH;
    return nullptr;
  }
  uint32_t* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* addr = nullptr;
  if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) {
    *status = FP8BS_ERR_LAUNCH;
    return nullptr;
  }
  p = static_cast<uint32_t*>(addr);
  g_scratch[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace
}  // namespace fp8bs

extern "C" int fp8_quantize_delayed(const void* x_bf16, int64_t numel, int fmt, int mode,
                                    int margin, int hist_len, float* amax_history, float* scale,
                                    void* q_out, float* scale_inv_used, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  const int s = delayed_args_ok(x_bf16, numel, fmt, mode, margin, hist_len, amax_history, scale,
                                q_out, scale_inv_used);
  if (s != FP8BS_OK) return s;
  if (!workspace || workspace_bytes < fp8_quantize_delayed_workspace_size())
    return FP8BS_ERR_WORKSPACE;
  if (!aligned4(workspace)) return FP8BS_ERR_ALIGN;
  return delayed_launch(x_bf16, numel, fmt, mode, margin, hist_len, amax_history, scale, q_out,
                        scale_inv_used, static_cast<uint32_t*>(workspace),
                        static_cast<hipStream_t>(stream));
}

extern "C" int fp8_quantize_delayed_noalloc(const void* x_bf16, int64_t numel, int fmt, int mode,
                                            int margin, int hist_len, float* amax_history,
                                            float* scale, void* q_out, float* scale_inv_used,
                                            void* stream) {
  const int s = delayed_args_ok(x_bf16, numel, fmt, mode, margin, hist_len, amax_history, scale,
                                q_out, scale_inv_used);
  if (s != FP8BS_OK) return s;
  static_assert(kScratchWords >= kDelayedBlocks, "scratch holds one partial per workgroup");
  if (delayed_blocks(numel) > kScratchWords) return FP8BS_ERR_WORKSPACE;   // (never: capped)
  int status = FP8BS_OK;
  uint32_t* part = scratch_on_current_device(&status);
  if (!part) return status;
  return delayed_launch(x_bf16, numel, fmt, mode, margin, hist_len, amax_history, scale, q_out,
                        scale_inv_used, part, static_cast<hipStream_t>(stream));
}

extern "C" int fp8_cast_fp32(const float* x, int64_t n, int fmt, void* q_out, void* stream) {
  if (!fmt_ok(fmt)) return FP8BS_ERR_ARG;
  if (n < 0) return FP8BS_ERR_SHAPE;
  if (n == 0) return FP8BS_OK;
  if (!x || !q_out) return FP8BS_ERR_NULL;
  if (!aligned4(x)) return FP8BS_ERR_ALIGN;
  const int blocks = (int)std::min<int64_t>(8192, std::max<int64_t>(1, ceil_div(ceil_div(n, 4), kThreads)));
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* q = static_cast<uint8_t*>(q_out);
  if (fmt == FP8BS_E4M3)
    return launch(cast_fp32_kernel<FP8BS_E4M3>, dim3(blocks), dim3(kThreads), st, x, n, q);
  return launch(cast_fp32_kernel<FP8BS_E5M2>, dim3(blocks), dim3(kThreads), st, x, n, q);
}

extern "C" const char* fp8bs_status_string(int status) {
  switch (status) {
    case FP8BS_OK: return "ok";
    case FP8BS_ERR_NULL: return "a required pointer is NULL";
    case FP8BS_ERR_SHAPE: return "invalid size or pitch";
    case FP8BS_ERR_ALIGN: return "pointer or pitch misaligned";
    case FP8BS_ERR_UNSUPPORTED: return "unsupported operand/scale combination";
    case FP8BS_ERR_LAUNCH: return "kernel launch failed";
    case FP8BS_ERR_WORKSPACE: return "workspace missing or too small";
    case FP8BS_ERR_ARG: return "argument out of range";
    default: return "unknown status";
  }
}
