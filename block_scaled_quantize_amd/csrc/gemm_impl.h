// Block-scaled FP8 GEMM for gfx950 (CDNA4): device code and launch helpers shared by the dense
// and grouped entry points (gemm.hip: fp32 scales; gemm_pow2.hip: power-of-2 scales applied by
// the MFMA itself).
//
// Method: "NVIDIA NeMo RL logra una aceleración del 48% con entrenamiento de precisión FP8 de
// extremo a extremo", section "El avance técnico": linear layers run FP8 math on 128x128 weight
// tiles and 1x128 activation blocks, output BF16; section "Ganancias de rendimiento en el
// mundo real": the same recipe on an MoE model's experts; section "Por qué esto es importante
// para la economía de la IA": power-of-2 scale factors.  Gradients may be E5M2 ("Infraestructura
// de Entrenamiento FP8 ...", section "El panorama de la precisión numérica").
//
// Design
//  * Output tile BM x BN per workgroup (256x256 with 8 waves, 256x128 with 8 or 4 waves, 128x128
//    with 4 waves), 128-byte K blocks, so one K block is exactly one scale block.  Each wave owns
//    a (BM / waves_m) x (BN / waves_n) sub-tile made of 16x16 pieces.
//  * One V_MFMA_F32_16X16X128_F8F6F4 consumes a full 128-wide K block.  Three ways to apply the
//    scales: fp32 block scales -- the MFMA result P is the partial sum of one scale block, folded
//    as acc += P * (sa[m, kb] * sb[n-block, kb]); per-tensor scales on both operands -- the MFMA
//    accumulates directly and the product of the two scales is applied once in the epilogue;
//    power-of-2 block scales -- their exponents go to the MFMA's own E8M0 scale operands (one
//    per lane: the lane's row and 32-wide k chunk) and the MFMA accumulates directly.
//  * The MFMA's "A" operand is the weight side (rows = n) and its "B" operand the activation side
//    (columns = m), so each lane ends with 4 consecutive n of one output row: 8-byte bf16 stores.
//  * Global -> LDS by buffer_load ... lds (no VGPR staging), 2 or 3 LDS stages; bounds come from
//    the buffer descriptors (rows past the matrix read as zero).
//  * LDS tiles are rows of 128 bytes with a 16-byte-chunk XOR swizzle chosen so that the lanes
//    the 64-bank LDS serves together hit distinct banks: ds_read_b128 serves 16 lanes (16
//    consecutive rows of a K-major tile) per pass, ds_read_b64_tr_b8 32 lanes (rows k0+j and
//    k0+32+j, j < 8, of an MN-major tile).
//    K-major operands (rows = m or n) are read with ds_read_b128; MN-major operands (rows = k,
//    dgrad / wgrad) are read with ds_read_b64_tr_b8, which transposes 8x8 byte blocks across
//    lanes, so no separate transpose pass is needed.
//  * Workgroup ids are remapped so that each XCD (ids round-robin over 8 XCDs) works on a
//    compact group of tiles and its L2 is reused.
#pragma once

#include <float.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"

namespace fp8bs {

// Arguments of one GEMM launch, as the kernels read them.
struct GemmParams {
  int64_t M, N, K;
  const uint8_t* A;   // activation side (rows m)
  int64_t lda;
  const uint8_t* B;   // weight side (rows n)
  int64_t ldb;
  const float* sa;    // sa(m, kb) = sa[kb * sa_ks + (m >> sa_rshift) * sa_rs]
  int64_t sa_ks, sa_rs, sa_bytes;
  int sa_rshift;
  const float* sb;    // sb(n, kb) = sb[kb * sb_ks + (n / 128) * sb_rs]
  int64_t sb_ks, sb_rs, sb_bytes;
  uint16_t* C;        // may be null when the output is only wanted quantized
  int64_t ldc;
  int tiles_m, tiles_n;
  int c_vec;          // 8-byte output stores are aligned
  int c_vec16;        // 16-byte output stores are aligned
  // fused output quantization (1x128 blocks along N): codes Cq[M, N] (pitch ldcq) and
  // dequantization factors cqs[ceil(N/128)][M]
  uint8_t* Cq;
  int64_t ldcq;
  float* cqs;
  int cq_vec;         // 4-byte code stores are aligned
  int cq_vec16;       // 16-byte code stores are aligned
  // grouped GEMM only
  const int64_t* offsets;
  int num_groups;
  int64_t b_group_stride;   // bytes between experts' weights
  int64_t sb_group_stride;  // floats between experts' scales
};

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// How the block scales are applied (see the design notes above).
constexpr int kScaleFold = 0;     // fp32 block scales, folded between K blocks
constexpr int kScaleTensor = 1;   // per-tensor scales on both operands, applied in the epilogue
constexpr int kScaleHw = 2;       // power-of-2 block scales, applied by the MFMA (E8M0)
// The same two block-scale modes with 1x128 weight-side scales (one per weight row and K block,
// the layout of a transposed columnwise-quantized operand): the fold multiplies each output
// element by its own sa[m] * sb[n]; the MFMA takes a per-lane E8M0 weight scale.
constexpr int kScaleFoldRows = 3;
constexpr int kScaleHwRows = 4;
// Microscaling: E8M0 scale bytes, one per 32 K elements of every row of both operands.  The
// four bytes of a row and K block travel as one word (as the 1x128 scales of kScaleHwRows do),
// and each lane gives the MFMA the byte of its own 32-wide k chunk.
constexpr int kScaleMx = 5;

constexpr int kGroupM = 4;      // tile-rows per L2 group in the dense tile order (2, 4, 6, 8, 16 measured)
constexpr int kGroupMGrouped = 8;   // ... in the grouped (MoE) order (4 and 8 measured)
constexpr int kLdsBytes = 160 * 1024;
constexpr int kStaticLdsReserve = 8448;   // the grouped kernel's group bounds and prefixes
constexpr bool kPersistentDense = true;   // two-stage dense tiles on a persistent grid

// Tile configuration: BM x BN output tile, WAVES_M x WAVES_N waves, each wave owning a
// (BM / WAVES_M) x (BN / WAVES_N) block of 16x16 pieces.  Three LDS stages when they fit in
// the 160 KiB of a CU, else two.
template <int BM_, int BN_, int WAVES_M, int WAVES_N>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kWavesM = WAVES_M, kWavesN = WAVES_N;
  static constexpr int kWTM = BM / WAVES_M;   // m extent of a wave
  static constexpr int kWTN = BN / WAVES_N;   // n extent of a wave
  static constexpr int kNJ = kWTM / 16;       // 16-wide m pieces per wave
  static constexpr int kNI = kWTN / 16;       // 16-wide n pieces per wave
  static constexpr int kXBytes = BM * 128;
  static constexpr int kWBytes = BN * 128;
  static constexpr int kSbWords = BN;   // one weight scale per tile column at most (1x128)
  static constexpr int kSaBytes = (BM + kSbWords) * 4;  // BM activation scales, weight scales
  static constexpr int kStage = kXBytes + kWBytes + kSaBytes;
  static constexpr int kDummyBytes = 256;   // target of the scale DMAs of non-loading waves
  static constexpr int kStages = 3 * kStage + kDummyBytes <= kLdsBytes ? 3 : 2;
  static constexpr int kDummy = kStage * kStages;   // offset of the dummy slot
  // Epilogue staging: per wave 16 output rows x 64 columns of bf16 (128 bytes, pitch 144), when
  // it fits next to the stages and the grouped kernel's static LDS.
  static constexpr int kEpiPitch = 144;
  static constexpr int kEpiWaveBytes = 16 * kEpiPitch;
  static constexpr int kEpi = kDummy + kDummyBytes;
  static constexpr bool kStagedEpi =
      kWTN == 64 && kEpi + kWaves * kEpiWaveBytes + kStaticLdsReserve <= kLdsBytes;
  static constexpr int kLds = kEpi + (kStagedEpi ? kWaves * kEpiWaveBytes : 0);
  static constexpr int kXLoads = BM / 8 / kWaves;   // 1 KB DMA blocks of the X tile per wave
  static constexpr int kWLoads = BN / 8 / kWaves;   // ... of the W tile per wave
  static constexpr int kSaWaves = BM / 64;          // waves that load 64 scale words each
  static constexpr int kSbWave = (BM / 64) % kWaves;  // wave that loads the weight scales
  // 1x128 weight scales (one per tile column): BN / 64 waves load 64 words each.
  static constexpr int kSbRowWaves = BN / 64;
  static constexpr int kSbRowWave0 = (BM / 64) % kWaves;
  static_assert(kSbRowWave0 + kSbRowWaves <= kWaves, "weight-scale loaders");
  static_assert(BM % (8 * kWaves) == 0 && BN % (8 * kWaves) == 0, "DMA split");
  static_assert(kSaWaves <= kWaves, "scale loaders");
  static_assert(kWTN <= 128 && 128 % kWTN == 0, "a wave's n range lies in one 128 block");
  static_assert(2 * kStage + kDummyBytes <= kLdsBytes, "LDS");
};


// ------------------------------------------------------------------ low-level helpers
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint64_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t n = (uint32_t)(nbytes >> 32) != 0u ? 0xFFFFFFFFu : (uint32_t)nbytes;
  u32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));   // stride 0
  r.z = __builtin_amdgcn_readfirstlane(n);
  r.w = 0x00020000u;                                           // raw 32-bit data format
  return r;
}

// The descriptor size of a DMA source with avail readable bytes from its base (none when
// avail <= 0 or the block is not live), clamped to 32 bits.
__device__ __forceinline__ uint64_t dma_bytes(int64_t avail, bool live) {
  const uint32_t hi = (uint32_t)((uint64_t)avail >> 32), lo = (uint32_t)avail;
  const uint32_t n = (int32_t)hi < 0 ? 0u : (hi != 0u ? 0xFFFFFFFFu : lo);
  return live ? n : 0u;
}

// Descriptor of a K-major operand's K block at byte offset k0 from the tile's K block 0: av0 = the
// bytes readable from the tile's K block 0, clamped to 32 bits once per tile (0 when none); the
// block's size is av0 - k0, in 32 bits.  The same reads as the exact size: a block's DMA stays
// below 256 rows of the pitch (< 2^31), and a clamped size minus k0 (< 2^23) stays above that.
// A nonzero av0 is at least one row's pitch, which is at least K > k0 for every block inside K,
// so the subtraction does not wrap.  Scale arrays (below 4 GiB, never clamped) use the same form:
// a tile's live K blocks read words of the array.
__device__ __forceinline__ uint32_t clamp_bytes(int64_t v) {
  return v <= 0 ? 0u : (v >= (int64_t)0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)v);
}
__device__ __forceinline__ u32x4 make_rsrc_k(const void* base, uint32_t av0, uint32_t k0,
                                             bool live) {
  return make_rsrc(base, (live && av0 != 0u) ? av0 - k0 : 0u);
}

// 16 bytes per lane from buffer offset voff to LDS address lds + 16 * lane.  Offsets at or past
// the descriptor's size read as zero.
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(lds) : "memory", "m0");
}
// 4 bytes per lane to LDS address lds + 4 * lane.
__device__ __forceinline__ void dma4(u32x4 rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(lds) : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are outstanding (N < 64).  The
// empty asm statements keep the compiler from moving LDS accesses across the wait.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
  asm volatile("" ::: "memory");
}

// Workgroup barrier without the memory fence of __syncthreads (outstanding LDS DMA is tracked
// explicitly with wait_vm); also a compiler barrier for memory accesses.
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Physical 16-byte chunk of logical chunk c in tile row r (chunk c ^ swz(r)), chosen by measuring
// the LDS read rate of the fragment patterns below.  K-major tiles: a 16-byte fragment read
// covers 16 consecutive rows at one logical chunk pair; XOR with r % 8 spreads 8 rows over the 8
// chunk positions and the extra flip by bit 3 separates the two 8-row halves, which makes the
// read conflict-free (about 240 B/clk per CU measured, against 128 for a permutation by r / 2).
// MN-major tiles: one transpose read takes one chunk from each of 8 consecutive rows in each of
// 4 bands 32 rows apart; the permutation by (k / 2) % 4 and bit 2 from bit 5 ^ bit 0 of k gives the best
// measured rate of the forms tried (about 190 B/clk, against 172 without the bit-0 term).
__device__ __forceinline__ int swz_k(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_mn(int k) { return ((k >> 1) & 3) | ((((k >> 5) ^ k) & 1) << 2); }
template <bool KMAJOR>
__device__ __forceinline__ int swz(int r) { return KMAJOR ? swz_k(r) : swz_mn(r); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

// Per-lane parts of the fragment addresses of one wave's pieces of a tile side, computed once
// per tile.  The wave's pieces start at row (K-major) or column (MN-major) u0 and follow every
// 16; the swizzle then depends on the lane only.  K-major: piece r is at the lane's address
// + 2048 r, an immediate offset of the LDS read.  MN-major (tile [halves][128 k][128 columns],
// a wave's columns inside one half): piece r is at the lane's address XOR 16 r, the chunk bits
// 4..6 (u0 % 128 is a multiple of the wave's column span, so it and 16 r share no bit).
template <bool KMAJOR>
struct FragBase {
  uint32_t a[KMAJOR ? 2 : 4];
};
__device__ __forceinline__ FragBase<true> frag_base_k(int li, int g, int u0) {
  const int sw = swz_k(li);
  const uint32_t r = (uint32_t)(u0 + li) * 128u;
  return FragBase<true>{{r + ((((2 * g) ^ sw) << 4)), r + ((((2 * g + 1) ^ sw) << 4))}};
}
// The K order of the 16x16x128 FP8 MFMA as its block scales see it: a lane's first 16 bytes are
// k = 16 g .. 16 g + 15 and its last 16 bytes k = 64 + 16 g .., so the 32-wide scale chunk c
// (the scale byte of lane 16 c + row) covers k = 32 c .. 32 c + 31 only when the fragments are
// read in that order (16-byte chunks g and g + 4).  Products summed without per-chunk scales do
// not depend on the order, so only the microscaling path reads its K-major fragments this way.
__device__ __forceinline__ FragBase<true> frag_base_k_mx(int li, int g, int u0) {
  const int sw = swz_k(li);
  const uint32_t r = (uint32_t)(u0 + li) * 128u;
  return FragBase<true>{{r + (((g ^ sw) << 4)), r + ((((g + 4) ^ sw) << 4))}};
}
__device__ __forceinline__ FragBase<false> frag_base_mn(int li, int g, int u0) {
  FragBase<false> b;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int k = 32 * g + 8 * t + (li >> 1);
    // bits 4..6 of k * 128 + 8 (li & 1) are 0
    const uint32_t lane = (uint32_t)((k * 128 + 8 * (li & 1)) | (swz_mn(k) << 4));
    b.a[t] = (lane ^ (uint32_t)(u0 & 0x70)) + (uint32_t)(u0 >> 7) * 16384u;
  }
  return b;
}
template <bool KMAJOR>
__device__ __forceinline__ FragBase<KMAJOR> frag_base(int li, int g, int u0) {
  if constexpr (KMAJOR) return frag_base_k(li, g, u0);
  else return frag_base_mn(li, g, u0);
}
// The bases in the LDS tile at address tile_lds (a multiple of 128, so that the MN-major XOR
// stays inside the lane's part), made opaque so that the compiler keeps one address per base
// and reaches the pieces by immediate offsets (K-major) or one XOR (MN-major).
template <bool KMAJOR>
__device__ __forceinline__ FragBase<KMAJOR> frag_at_tile(FragBase<KMAJOR> b, uint32_t tile_lds) {
#pragma unroll
  for (int t = 0; t < (KMAJOR ? 2 : 4); ++t) {
    b.a[t] += tile_lds;
    asm volatile("" : "+v"(b.a[t]));
  }
  return b;
}
typedef __attribute__((address_space(3))) const u32x4 lds_u4_t;
typedef __attribute__((address_space(3))) const float lds_f32_t;
__device__ __forceinline__ float lds_f32(uint32_t a) { return *(lds_f32_t*)a; }
// One byte of LDS, zero-extended, carried in a float's bits (the microscaling scale bytes).
typedef __attribute__((address_space(3))) const uint8_t lds_u8_t;
__device__ __forceinline__ float lds_u8_bits(uint32_t a) { return __uint_as_float(*(lds_u8_t*)a); }
// The 32-byte MFMA fragment of lane (li, g) for the wave's piece r: bytes k = 32g .. 32g+31 of
// the piece's row li (K-major tile), or of its column li in an MN-major tile, gathered by four
// 8x8 byte transposes across lanes (source lane 2j + h of each 16-lane group points at row
// k0 + j, bytes 8h .. 8h + 7 of the chunk).
template <bool KMAJOR>
__device__ __forceinline__ v8i frag_piece(const FragBase<KMAJOR>& b, int r) {
  v8i v;
  if constexpr (KMAJOR) {
    const u32x4 lo = *(lds_u4_t*)(b.a[0] + 2048u * (uint32_t)r);
    const u32x4 hi = *(lds_u4_t*)(b.a[1] + 2048u * (uint32_t)r);
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) v2i*)(b.a[t] ^ (16u * (uint32_t)r)));
      v[2 * t] = x.x;
      v[2 * t + 1] = x.y;
    }
  }
  return v;
}


// Per-lane DMA source offsets for a tile side.  K-major: rows of the tile are matrix rows
// (m or n), the K block starts at the descriptor base.  MN-major: rows of the tile are k, the
// 128-column halves sit at +128 * h.  Instruction q of the tile covers LDS bytes
// [1024 q, 1024 q + 1024) = 8 rows of 128 bytes; lane i fills row 8q' + i / 8 at physical
// chunk i % 8, which holds logical chunk (i % 8) ^ swz(row).
template <bool KMAJOR>
__device__ __forceinline__ uint32_t dma_voffset(int q, int lane, int64_t ld) {
  const int rl = lane >> 3;
  if constexpr (KMAJOR) {
    const int row = 8 * q + rl;
    const int c = (lane & 7) ^ swz_k(row);
    return (uint32_t)((int64_t)row * ld + 16 * c);
  } else {
    const int h = q >> 4, qq = q & 15;
    const int row = 8 * qq + rl;
    const int c = (lane & 7) ^ swz_mn(row);
    return (uint32_t)((int64_t)row * ld + 128 * h + 16 * c);
  }
}

// Zero the bytes of a K-major tile whose k is at or beyond krem (last, partial K block).
template <int ROWS, int THREADS>
__device__ __forceinline__ void zero_k_tail(uint8_t* tile, int krem) {
  for (int id = threadIdx.x; id < ROWS * 8; id += THREADS) {
    const int r = id >> 3, c = id & 7;
    uint8_t* p = tile + r * 128 + ((c ^ swz_k(r)) << 4);
    if (16 * c >= krem) {
      *reinterpret_cast<uint4*>(p) = make_uint4(0, 0, 0, 0);
    } else if (16 * c + 16 > krem) {
      for (int b = krem - 16 * c; b < 16; ++b) p[b] = 0;
    }
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  bf2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Wait until every LDS access of this wave has completed.
__device__ __forceinline__ void wait_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));   // lgkmcnt 0, others unchanged
  asm volatile("" ::: "memory");
}

// Wait until at most min(n, HI) vector-memory operations are outstanding, for LO <= min(n, HI)
// (n wave-uniform): a binary search over the waitcnt immediates, a handful of scalar branches
// instead of one per value.
template <int LO, int HI>
__device__ __forceinline__ void wait_vm_range(int n) {
  if constexpr (LO >= HI) {
    wait_vm<HI>();
  } else {
    constexpr int MID = (LO + HI + 1) / 2;
    if (n >= MID) wait_vm_range<MID, HI>(n);
    else wait_vm_range<LO, MID - 1>(n);
  }
}
// Wait until at most min(n, N) are outstanding (n >= 0); FAST, a count that is checked first
// (the one a whole tile gives).
template <int N, int FAST = N>
__device__ __forceinline__ void wait_vm_atmost(int n) {
  n = __builtin_amdgcn_readfirstlane(n);
  if (n == FAST) wait_vm<FAST>();
  else wait_vm_range<0, N>(n);
}

// One output tile: group g (0 for a dense GEMM), rows [m0, m_end), columns from n0.
struct Tile {
  int g, m0, m_end, n0;
};
// Pipeline state a persistent workgroup carries from one tile to the next: the LDS stage that
// holds the tile's first K block, whether that block was issued during the previous tile, and
// how many store instructions (at least) the previous tile's epilogue issued after it.  Vector
// memory operations complete in issue order (one vmcnt for loads, stores and LDS DMA), so
// waiting until at most that many are outstanding means the block has landed while the stores
// may still drain.
struct Carry {
  int stage0, prefetched, stores;
};

// The epilogue store of one 16x16 piece: this lane's 4 consecutive outputs of row m, rounded to
// bf16 (round to nearest even) and stored with one 8-byte store when aligned.
template <class C>
__device__ __forceinline__ void store_piece(const GemmParams& p, const Tile& t, int wm, int wn,
                                            int li, int g, int i, int j, v4f v) {
  const int64_t m = (int64_t)t.m0 + wm * C::kWTM + 16 * j + li;
  if (m >= t.m_end) return;
  uint16_t* crow = p.C + m * p.ldc;
  const int64_t n = (int64_t)t.n0 + wn * C::kWTN + 16 * i + 4 * g;
  const uint32_t lo = pack_bf16x2(v[0], v[1]);
  const uint32_t hi = pack_bf16x2(v[2], v[3]);
  if (p.c_vec && n + 4 <= p.N) {
    *reinterpret_cast<uint2*>(crow + n) = make_uint2(lo, hi);
  } else {
    const uint16_t h[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (n + e < p.N) crow[n + e] = h[e];
  }
}

// The epilogue store of the 16 rows of m piece j (this wave's 64 columns): the lane's bf16
// values go to the wave's own LDS rows, come back as 16-byte row chunks, and leave as whole
// 128-byte row segments (8 rows per store instruction) instead of 32-byte pieces of 16 rows.
template <class C>
__device__ __forceinline__ void store_rows_staged(const GemmParams& p, const Tile& t, int wm,
                                                  int wn, int lane, int j, const v4f (&v)[C::kNI],
                                                  uint8_t* region) {
  static_assert(C::kWTN == 64 && C::kNI == 4, "a wave's rows are 128 bytes");
  const int li = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < C::kNI; ++i)
    *reinterpret_cast<uint2*>(region + li * C::kEpiPitch + 32 * i + 8 * g) =
        make_uint2(pack_bf16x2(v[i][0], v[i][1]), pack_bf16x2(v[i][2], v[i][3]));
  wait_lds();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 8 * h + (lane >> 3), c = lane & 7;
    const uint4 d = *reinterpret_cast<const uint4*>(region + r * C::kEpiPitch + 16 * c);
    const int64_t m = (int64_t)t.m0 + wm * C::kWTM + 16 * j + r;
    const int64_t n = (int64_t)t.n0 + wn * C::kWTN + 8 * c;
    if (m < t.m_end) {
      uint16_t* crow = p.C + m * p.ldc;
      if (n + 8 <= p.N) {
        // non-temporal: full lines go straight to memory instead of filling the caches with
        // dirty output that the next kernel would have to write back
        __builtin_nontemporal_store(u32x4{d.x, d.y, d.z, d.w}, reinterpret_cast<u32x4*>(crow + n));
      } else {
        const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n + e < p.N) crow[n + e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
  wait_lds();   // (the next round rewrites the region)
}

// LDS accesses of one wave stay in issue order, so a wave can exchange data between its own
// lanes through LDS with no wait: this only keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The staged epilogue of a wave whose 64 columns lie inside the output (16-byte aligned rows):
// the same LDS round trip and full-line stores as store_rows_staged, without per-lane column
// tests, with the row address stepped instead of recomputed, and with piece j + 1 written to the
// region while piece j's stores go out (the accumulators are zero when K is empty, so no zeroing
// is needed).  ROWS_CUT: only the wave's first `rows` rows are inside (a lane stores its row if
// it is); otherwise all 128 are.
template <class C, int SM, bool ROWS_CUT, class Acc>
__device__ __forceinline__ void store_wave_staged(const GemmParams& p, const Tile& t, int wm, int wn,
                                                  int lane, const Acc& acc, float post,
                                                  uint8_t* region, int rows) {
  static_assert(C::kWTN == 64 && C::kNI == 4, "a wave's rows are 128 bytes");
  constexpr int NI = C::kNI, NJ = C::kNJ;
  const int li = lane & 15, g = lane >> 4;
  const int r = lane >> 3, c = lane & 7;
  uint16_t* base = p.C + ((int64_t)t.m0 + wm * C::kWTM + r) * p.ldc + (t.n0 + wn * C::kWTN + 8 * c);
  const int64_t row8 = 8 * p.ldc;
  uint8_t* wr = region + li * C::kEpiPitch + 8 * g;
  const uint8_t* rd = region + r * C::kEpiPitch + 16 * c;
  auto put = [&](int j) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      v4f v = acc[i][j];
      if constexpr (SM == kScaleTensor) v = v * post;
      *reinterpret_cast<uint2*>(wr + 32 * i) =
          make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
  };
  uint4 d[2];
  auto get = [&]() {
#pragma unroll
    for (int h = 0; h < 2; ++h) d[h] = *reinterpret_cast<const uint4*>(rd + 8 * h * C::kEpiPitch);
  };
  put(0);
  wave_lds_fence();
  get();
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const uint4 e0 = d[0], e1 = d[1];
    if (j + 1 < NJ) {
      wave_lds_fence();   // (the reads of piece j precede these writes in the LDS queue)
      put(j + 1);
    }
    if (!ROWS_CUT || r + 16 * j < rows)
      __builtin_nontemporal_store(u32x4{e0.x, e0.y, e0.z, e0.w},
                                  reinterpret_cast<u32x4*>(base + (2 * j) * row8));
    if (!ROWS_CUT || r + 16 * j + 8 < rows)
      __builtin_nontemporal_store(u32x4{e1.x, e1.y, e1.z, e1.w},
                                  reinterpret_cast<u32x4*>(base + (2 * j + 1) * row8));
    if (j + 1 < NJ) {
      wave_lds_fence();
      get();
    }
  }
}

// E8M0 code of a power-of-two scale: its binary32 exponent field (2^-127, the one subnormal
// power of two a scale can take, has field 0 and is E8M0 code 0 as well).
__device__ __forceinline__ int e8m0_of(float s) {
  return (int)((__builtin_bit_cast(uint32_t, s) >> 23) & 0xFF);
}

// Fused output quantization: the tile's bf16 output values (exactly those the epilogue stores)
// quantized in 1x128 blocks along N -- the blockwise quantizer's rule applied to the bf16
// output, so the codes and scales equal those of quantizing the stored bf16 matrix.  A 128-column
// block of a row spans the 64-column ranges of two waves (wn even / odd): each lane reduces its
// values, the 4 lanes of a row reduce by shuffles, the two waves meet in LDS.
template <class C, int SM, int QO, class Acc>
__device__ __forceinline__ void quantize_out(const GemmParams& p, uint8_t* smem, const Acc& acc,
                                             float post, int nkb, int64_t m0, int64_t m_end,
                                             int64_t n0) {
  constexpr int QF = (QO - 1) >> 1;
  constexpr bool QP = ((QO - 1) & 1) != 0;
  constexpr int NI = C::kNI, NJ = C::kNJ, BM = C::BM;
  static_assert(C::kWTN == 64 && C::BN % 128 == 0, "a 128-column block spans two waves");
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w % C::kWavesM, wn = w / C::kWavesM;
  const int li = lane & 15, g = lane >> 4;
  // bf16 values of the lane: bv[i][j] = (v0, v1), (v2, v3)
  uint32_t bv[NI][NJ][2];
  uint32_t amax[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    u16x2 mx = {0, 0};
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      v4f v = acc[i][j];
      if constexpr (SM == kScaleTensor) v = v * post;   // as the bf16 epilogue does
      if (nkb == 0) v = v4f{0.f, 0.f, 0.f, 0.f};
      bv[i][j][0] = pack_bf16x2(v[0], v[1]);
      bv[i][j][1] = pack_bf16x2(v[2], v[3]);
      mx = max2(mx, max2(mag2(bv[i][j][0]), mag2(bv[i][j][1])));
    }
    uint32_t a = hmax(mx);
    a = max(a, (uint32_t)__shfl_xor((int)a, 16));
    a = max(a, (uint32_t)__shfl_xor((int)a, 32));
    amax[j] = a;
  }
  // every wave is past its last read of the operand stages: reuse them for the exchange
  __syncthreads();
  uint32_t* s_amax = reinterpret_cast<uint32_t*>(smem);   // [waves along n][BM]
  if (g == 0) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) s_amax[wn * BM + wm * C::kWTM + 16 * j + li] = amax[j];
  }
  __syncthreads();
  const int64_t blk = (n0 >> 7) + (wn >> 1);   // 128-column block of this wave
  // Codes of a tile whose columns all lie inside the output (16-byte aligned rows) are gathered
  // in the free operand stages as [row][column] (pitch kTPitch, after the amax words) and leave
  // as whole 256-byte tile rows, 4 rows per store instruction.  Otherwise they leave through the
  // wave's epilogue region when 16-byte stores are aligned: the 16 rows of a piece as 64-byte row
  // segments, 16 rows per store instruction, instead of 4 bytes per lane and piece.
  constexpr int kQPitch = 80;
  constexpr int kTPitch = C::BN + 16;   // (4-byte writes of a piece: 64 distinct banks)
  static_assert(C::kWavesN * BM * 4 + BM * kTPitch <= C::kStages * C::kStage, "codes tile");
  uint8_t* const tile_codes = smem + C::kWavesN * BM * 4;
  const bool whole_cols = p.cq_vec16 && n0 + C::BN <= p.N;
  const bool staged = C::kStagedEpi && p.cq_vec16 && !whole_cols;
  uint8_t* region = smem + C::kEpi + w * C::kEpiWaveBytes;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int row = wm * C::kWTM + 16 * j + li;
    const int64_t m = m0 + row;
    const uint32_t a = max(s_amax[(wn & ~1) * BM + row], s_amax[(wn | 1) * BM + row]);
    const float s = scale_from_amax_bits<QF, QP>(a);
    const bool finite = a < 0x7F80u;
    uint32_t codes[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float y0 = bf16_lo(bv[i][j][0]) * s, y1 = bf16_hi(bv[i][j][0]) * s;
      float y2 = bf16_lo(bv[i][j][1]) * s, y3 = bf16_hi(bv[i][j][1]) * s;
      if (!finite) {
        constexpr float F = Format<QF>::fmax;
        y0 = __builtin_amdgcn_fmed3f(y0, -F, F);
        y1 = __builtin_amdgcn_fmed3f(y1, -F, F);
        y2 = __builtin_amdgcn_fmed3f(y2, -F, F);
        y3 = __builtin_amdgcn_fmed3f(y3, -F, F);
      }
      codes[i] = cvt4<QF>(y0, y1, y2, y3);
      if (!finite) codes[i] = patch_nan_pair(patch_nan_pair(codes[i], bv[i][j][0], 0), bv[i][j][1], 1);
    }
    if (whole_cols) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
        *reinterpret_cast<uint32_t*>(tile_codes + row * kTPitch + wn * C::kWTN + 16 * i + 4 * g) =
            codes[i];
    } else if (staged) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
        *reinterpret_cast<uint32_t*>(region + li * kQPitch + 16 * i + 4 * g) = codes[i];
      wait_lds();
      const int r = lane >> 2, c = lane & 3;
      const uint4 d = *reinterpret_cast<const uint4*>(region + r * kQPitch + 16 * c);
      const int64_t mr = m0 + wm * C::kWTM + 16 * j + r;
      const int64_t n = n0 + wn * C::kWTN + 16 * c;
      if (mr < m_end) {
        uint8_t* qrow = p.Cq + mr * p.ldcq;
        if (n + 16 <= p.N) {
          __builtin_nontemporal_store(u32x4{d.x, d.y, d.z, d.w}, reinterpret_cast<u32x4*>(qrow + n));
        } else {
          const uint32_t wd[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (n + e < p.N) qrow[n + e] = (uint8_t)(wd[e >> 2] >> (8 * (e & 3)));
        }
      }
      wait_lds();   // (the next piece rewrites the region)
    } else if (m < m_end) {
      uint8_t* qrow = p.Cq + m * p.ldcq;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int64_t n = n0 + wn * C::kWTN + 16 * i + 4 * g;
        if (p.cq_vec && n + 4 <= p.N) {
          *reinterpret_cast<uint32_t*>(qrow + n) = codes[i];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < p.N) qrow[n + e] = (uint8_t)(codes[i] >> (8 * e));
        }
      }
    }
    if (m < m_end && g == 0 && (wn & 1) == 0 && blk * 128 < p.N) p.cqs[blk * p.M + m] = 1.0f / s;
  }
  if (whole_cols) {
    __syncthreads();   // every wave's codes are in the tile
    constexpr int kRowsPerWave = BM / C::kWaves;
    constexpr int kLanesPerRow = C::BN / 16;
    static_assert(64 % kLanesPerRow == 0 && kRowsPerWave % (64 / kLanesPerRow) == 0, "code rows");
    const int c = lane % kLanesPerRow;
#pragma unroll
    for (int q = 0; q < kRowsPerWave / (64 / kLanesPerRow); ++q) {
      const int row = w * kRowsPerWave + q * (64 / kLanesPerRow) + lane / kLanesPerRow;
      const uint4 d = *reinterpret_cast<const uint4*>(tile_codes + row * kTPitch + 16 * c);
      if (m0 + row < m_end)
        __builtin_nontemporal_store(u32x4{d.x, d.y, d.z, d.w},
                                    reinterpret_cast<u32x4*>(p.Cq + (m0 + row) * p.ldcq + n0 + 16 * c));
    }
  }
}

// ------------------------------------------------------------------ one output tile
// Computes C[m0 .. m_end) x [n0 .. n0 + BN) of tile t (columns clipped to N) with the operand
// roles of LAYOUT: A is the activation-side matrix; the weight side and its scales are those of
// the tile's group (p.B + g * b_group_stride, p.sb + g * sb_group_stride, sb_bytes bytes).
// QO: fused quantization of the output into 1x128 blocks along N, 0 = none, else
// 1 + 2 * format + (power-of-2 scale ? 1 : 0).
// PF (persistent workgroups, two LDS stages, no fused quantization): when has_next and the tile
// has at least two K blocks, the next tile's first K block is loaded into the free stage while
// this tile's last block runs, and the next tile starts without waiting for this tile's stores.
// The next tile, nt = next_tile(), is then formed at the start of the tile's last-but-one block
// (its lookup overlaps the K loop instead of following the epilogue); nt is left as it was
// otherwise.
// CUT_ROWS (grouped GEMM: every expert's last tile is cut): waves whose rows end inside the tile
// also take the epilogue without column tests.
template <class C, int LAYOUT, int FA, int FB, int SM, int QO = 0, bool PF = false,
          bool PERSIST = PF, bool CUT_ROWS = false, class NextTile>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, uint8_t* smem, const Tile& t,
                                          Tile& nt, const NextTile& next_tile, bool has_next,
                                          Carry& cy) {
  static_assert(!PF || (C::kStages == 2 && QO == 0), "cross-tile prefetch: two stages, bf16 out");
  const int64_t m0 = t.m0, m_end = t.m_end, n0 = t.n0;
  const uint8_t* Bw = p.B + (int64_t)t.g * p.b_group_stride;
  const float* sbw = p.sb + (int64_t)t.g * p.sb_group_stride;
  const int64_t sb_bytes = p.sb_bytes;
  constexpr bool XK = LAYOUT != FP8BS_WGRAD;   // activation side K-major?
  constexpr bool WK = LAYOUT == FP8BS_FPROP;   // weight side K-major?
  // per-row weight scale words: 1x128 weight scales, or the microscaling bytes
  constexpr bool ROWS = SM == kScaleFoldRows || SM == kScaleHwRows || SM == kScaleMx;
  constexpr bool FOLD = SM == kScaleFold || SM == kScaleFoldRows;
  constexpr bool HW = SM == kScaleHw || SM == kScaleHwRows || SM == kScaleMx;
  constexpr bool MX = SM == kScaleMx;
  constexpr bool STAGED = SM != kScaleTensor;   // block scales staged in LDS with the operands
  constexpr int BM = C::BM, BN = C::BN, NI = C::kNI, NJ = C::kNJ;
  // (PERSIST, a loop over tiles: the thread id is made opaque per tile, so that values derived
  // from it are recomputed for each tile instead of being kept live across the whole loop)
  int tid = (int)threadIdx.x;
  if constexpr (PERSIST) asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wm = w % C::kWavesM, wn = w / C::kWavesM;
  const int li = lane & 15, g = lane >> 4;
  const int64_t K = p.K;
  const int nkb = (int)((K + 127) >> 7);
  const int krem = (int)(K - (int64_t)(nkb - 1) * 128);
  const uint32_t lds0 = lds_addr(smem);
  const int st0 = PF ? cy.stage0 : 0;   // LDS stage of block 0
  // the next tile's first K block is loaded during this tile (as "block nkb")
  const bool pf_live = PF && has_next && nkb >= 2;

  // DMA source offsets relative to a tile's origin (the same for every K block and tile).
  uint32_t xoff[C::kXLoads], woff[C::kWLoads];
#pragma unroll
  for (int q = 0; q < C::kXLoads; ++q) xoff[q] = dma_voffset<XK>(w * C::kXLoads + q, lane, p.lda);
#pragma unroll
  for (int q = 0; q < C::kWLoads; ++q) woff[q] = dma_voffset<WK>(w * C::kWLoads + q, lane, p.ldb);
  const int wu = __builtin_amdgcn_readfirstlane(w);   // (the wave index, as a scalar)
  const bool sa_loader = wu < C::kSaWaves;
  const bool sb_loader = ROWS ? (wu >= C::kSbRowWave0 && wu < C::kSbRowWave0 + C::kSbRowWaves)
                              : wu == C::kSbWave;
  // Scale words: tile row w * 64 + lane, and the weight scales of the tile's 128-column blocks
  // (1x128 weight scales: tile column 64 (w - w0) + lane).  Rows past m_end and columns past N
  // read other tiles' scales or, past the array, zeros; their outputs are never stored.  The
  // tile's first scale row (m0 is a multiple of 128 whenever rows share a scale) and column
  // block are added to the descriptor base.
  uint32_t saoff = (uint32_t)((int64_t)((w * 64 + lane) >> p.sa_rshift) * p.sa_rs * 4);
  uint32_t sboff = 0xFFFFFFFFu;
  if constexpr (ROWS) {
    if (sb_loader) sboff = (uint32_t)((int64_t)((w - C::kSbRowWave0) * 64 + lane) * p.sb_rs * 4);
  } else {
    if (lane < BN / 128) sboff = (uint32_t)((int64_t)lane * p.sb_rs * 4);
  }

  // DMA instructions per K block issued by each wave (vmcnt is counted per wave).
  // Scale DMA instructions per wave and block: one when the activation-scale loaders and the
  // weight-scale loaders are different waves (every tile configuration with 8 waves), else two.
  // The fold with 1x128 weight scales keeps two (its block DMA goes out in one burst; one
  // instruction per wave measured 10-19% slower there, 2-4% faster everywhere else).
  constexpr bool kOneScale =
      !(ROWS && FOLD) && C::kSaWaves + (ROWS ? C::kSbRowWaves : 1) <= C::kWaves;
  constexpr int kPerStage = C::kXLoads + C::kWLoads + (STAGED ? (kOneScale ? 1 : 2) : 0);
  // A block's DMA starts as soon as its slot is free, right after the barrier that ends the
  // slot's previous block: one instruction after each MFMA unit of the last piece before the
  // hand-over, the rest one per MFMA unit at the start of the next block.  (A burst would leave
  // waves waiting to issue while the CU's address unit drains it; a later start lands later.)
  // With 1x128 weight scales the fold doubles its VALU work per MFMA, and issuing the whole
  // block after the hand-over piece's MFMAs measured faster.
  constexpr bool kBurst = ROWS;
  static_assert(kPerStage - NI <= (NJ - 1) * NI, "every DMA part precedes the next turn");
  // readable bytes of the K-major sides from the tile's K block 0
  const uint32_t x_av0 = __builtin_amdgcn_readfirstlane(XK ? clamp_bytes((m_end - m0) * p.lda) : 0u);
  const uint32_t w_av0 = __builtin_amdgcn_readfirstlane(WK ? clamp_bytes((p.N - n0) * p.ldb) : 0u);
  // ... and of the scale arrays from the tile's first scale word
  const uint32_t sa_av0 = __builtin_amdgcn_readfirstlane(
      STAGED ? clamp_bytes(p.sa_bytes - 4 * ((m0 >> p.sa_rshift) * p.sa_rs)) : 0u);
  const uint32_t sb_av0 = __builtin_amdgcn_readfirstlane(
      STAGED ? clamp_bytes(sb_bytes - 4 * ((ROWS ? n0 : (n0 >> 7)) * p.sb_rs)) : 0u);
  // DMA of one K block: the buffer descriptors (empty for blocks past the last: they read
  // zeros into a slot no block reads) and the LDS stage; dma_part(d, q) issues this wave's q-th
  // DMA instruction of the block (compile-time q once the callers' loops are unrolled).
  struct BlockDma {
    u32x4 x, w, sa, sb;
    uint32_t sbase;
  };
  // NX (PF only): the block is "block nkb", the next tile's first block; its descriptors are
  // built only in the two blocks that issue it, so the next tile adds no live registers to the
  // common block.
  auto block_dma = [&](int kb, auto nx_tag) {
    constexpr bool NX = decltype(nx_tag)::value;
    BlockDma d;
    d.sbase = lds0 + ((uint32_t)(kb + st0) % C::kStages) * C::kStage;
    const bool live = NX ? pf_live : kb < nkb;
    int64_t tm0 = m0, tme = m_end, tn0 = n0, kk = kb;
    const uint8_t* tBw = Bw;
    const float* tsb = sbw;
    if constexpr (NX) {
      tm0 = nt.m0; tme = nt.m_end; tn0 = nt.n0; kk = 0;
      tBw = p.B + (int64_t)nt.g * p.b_group_stride;
      tsb = p.sb + (int64_t)nt.g * p.sb_group_stride;
    }
    const int64_t k0 = kk * 128;
    {
      const uint8_t* base;
      if constexpr (XK) {   // rows past the tile's m_end read as zero
        base = p.A + tm0 * p.lda + k0;
        d.x = make_rsrc_k(base, NX ? clamp_bytes((tme - tm0) * p.lda) : x_av0, (uint32_t)k0, live);
      } else {
        base = p.A + k0 * p.lda + tm0;
        d.x = make_rsrc(base, dma_bytes((K - k0) * p.lda - tm0, live));
      }
    }
    {
      const uint8_t* base;
      if constexpr (WK) {
        base = tBw + tn0 * p.ldb + k0;
        d.w = make_rsrc_k(base, NX ? clamp_bytes((p.N - tn0) * p.ldb) : w_av0, (uint32_t)k0, live);
      } else {
        base = tBw + k0 * p.ldb + tn0;
        d.w = make_rsrc(base, dma_bytes((K - k0) * p.ldb - tn0, live));
      }
    }
    if constexpr (STAGED) {
      // (scale arrays are below 4 GiB: the bytes from the tile's first scale word, less the
      // K block's offset, in 32 bits; see make_rsrc_k)
      const int64_t rowa = (tm0 >> p.sa_rshift) * p.sa_rs;
      const uint32_t sa_av = NX ? clamp_bytes(p.sa_bytes - 4 * rowa) : sa_av0;
      d.sa = make_rsrc_k(p.sa + kk * p.sa_ks + rowa, sa_av, (uint32_t)(4 * kk * p.sa_ks), live);
      const int64_t rowb = (ROWS ? tn0 : (tn0 >> 7)) * p.sb_rs;
      const uint32_t sb_av = NX ? clamp_bytes(sb_bytes - 4 * rowb) : sb_av0;
      d.sb = make_rsrc_k(tsb + kk * p.sb_ks + rowb, sb_av, (uint32_t)(4 * kk * p.sb_ks), live);
    }
    return d;
  };
  auto dma_part = [&](const BlockDma& d, int q) {
    if (q < C::kXLoads) {
      dma16(d.x, xoff[q], __builtin_amdgcn_readfirstlane(d.sbase + (wu * C::kXLoads + q) * 1024));
    } else if (q < C::kXLoads + C::kWLoads) {
      const int qw = q - C::kXLoads;
      dma16(d.w, woff[qw],
            __builtin_amdgcn_readfirstlane(d.sbase + C::kXBytes + (wu * C::kWLoads + qw) * 1024));
    } else if (kOneScale && q == C::kXLoads + C::kWLoads) {
      // Scales of the K block: one activation word per tile row (waves [0, kSaWaves)) and the
      // weight words (the weight-scale loaders); every wave issues one such instruction, so
      // the block needs no branch: the remaining waves read outside the descriptor into the
      // dummy slot.
      const uint32_t sbdst = d.sbase + C::kXBytes + C::kWBytes + BM * 4 +
                             (ROWS ? (wu - C::kSbRowWave0) * 256 : 0);
      dma4(sa_loader ? d.sa : d.sb, sa_loader ? saoff : (sb_loader ? sboff : 0xFFFFFFFFu),
           __builtin_amdgcn_readfirstlane(sa_loader ? d.sbase + C::kXBytes + C::kWBytes + wu * 256
                                                    : (sb_loader ? sbdst : lds0 + C::kDummy)));
    } else if (q == C::kXLoads + C::kWLoads) {
      // (two scale instructions per wave: activation words, then weight words)
      dma4(d.sa, sa_loader ? saoff : 0xFFFFFFFFu,
           __builtin_amdgcn_readfirstlane(sa_loader ? d.sbase + C::kXBytes + C::kWBytes + wu * 256
                                                    : lds0 + C::kDummy));
    } else {
      const uint32_t dst = d.sbase + C::kXBytes + C::kWBytes + BM * 4 +
                           (ROWS ? (wu - C::kSbRowWave0) * 256 : 0);
      dma4(d.sb, sb_loader ? sboff : 0xFFFFFFFFu,
           __builtin_amdgcn_readfirstlane(sb_loader ? dst : lds0 + C::kDummy));
    }
  };
  auto issue = [&](int kb, auto nx_tag) {
    const BlockDma d = block_dma(kb, nx_tag);
#pragma unroll
    for (int q = 0; q < kPerStage; ++q) dma_part(d, q);
  };

  v4f acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Pipeline.  Stages hold K blocks kb .. kb + kStages - 1.  The wait and barrier that publish
  // block kb + 1 sit between the last two m pieces of block kb: while a wave waits there, the
  // MFMA pipe still holds the MFMAs of piece NJ - 2, and the MFMAs of piece NJ - 1 run while
  // the fragments of block kb + 1 are read (each weight fragment is re-read into its register
  // right after the MFMA that last uses it).
  // Every wave issues kPerStage DMA instructions per block, in block order, also for blocks
  // past the last (their descriptors are empty: they read zeros into a slot no block reads), so
  // vmcnt says which blocks have landed.
  auto wait_next = [&]() {
    // the next block must have landed; with 3 stages the one after it may still be in flight
    if constexpr (C::kStages == 3) wait_vm<kPerStage>();
    else wait_vm<0>();
  };
  auto stage_ptr = [&](int kb) { return smem + ((uint32_t)(kb + st0) % C::kStages) * C::kStage; };
  auto prepare = [&](int kb) {
    // ragged K: the last block's bytes past K are zeroed before anyone reads them
    if (kb == nkb - 1 && krem < 128 && (XK || WK)) {
      uint8_t* st = stage_ptr(kb);
      if constexpr (XK) zero_k_tail<BM, C::kThreads>(st, krem);
      if constexpr (WK) zero_k_tail<BN, C::kThreads>(st + C::kXBytes, krem);
      if constexpr (MX) {
        // scale bytes of the 32-wide chunks past K (row padding, any value -- an E8M0 NaN
        // would turn the zeroed products into NaN) become 2^0
        const int keep = (krem + 31) >> 5;
        const uint32_t mask = keep >= 4 ? 0xFFFFFFFFu : ((1u << (8 * keep)) - 1u);
        uint32_t* sw = reinterpret_cast<uint32_t*>(st + C::kXBytes + C::kWBytes);
        for (int id = threadIdx.x; id < BM + BN; id += C::kThreads)
          sw[id] = (sw[id] & mask) | (0x7F7F7F7Fu & ~mask);
      }
      __syncthreads();
    }
  };
  // Fragment address bases of the wave's pieces (per tile; frag_at_tile adds a stage's address
  // once per block), and the byte offset of the lane's first activation scale in a stage.
  FragBase<XK> xb = frag_base<XK>(li, g, wm * C::kWTM);
  FragBase<WK> wb = frag_base<WK>(li, g, wn * C::kWTN);
  if constexpr (MX) {
    static_assert(XK && WK, "microscaling: K-major operands (fprop)");
    xb = frag_base_k_mx(li, g, wm * C::kWTM);
    wb = frag_base_k_mx(li, g, wn * C::kWTN);
  }
  // (microscaling: the byte of the lane's k chunk g in the row's word)
  const uint32_t sc_lane = (uint32_t)(C::kXBytes + C::kWBytes + 4 * (wm * C::kWTM + li)) + (MX ? g : 0);
  auto lds_scale = [](uint32_t a) { return MX ? lds_u8_bits(a) : lds_f32(a); };
  auto scales_of = [&](const uint8_t* st) {
    return reinterpret_cast<const float*>(st + C::kXBytes + C::kWBytes);
  };
  // The lane's activation-scale address in a stage (opaque, like the fragment bases): piece r's
  // scale is at + 64 r.
  auto scale_base = [&](const uint8_t* st) {
    uint32_t a = lds_addr(st) + sc_lane;
    asm volatile("" : "+v"(a));
    return a;
  };
  // First m piece of a block: its fragment, and the activation scale c of its rows (the fold's
  // factor is c * sbv; the multiply is left to the end of the piece that precedes the piece's
  // use, so that no wave waits on the scale's LDS read right after issuing it); the block's
  // weight scale sbv (one per wave).
  auto first_x = [&](const uint8_t* st, v8i& xf, float& c, float& sbv) {
    const float* sat = scales_of(st);
    xf = frag_piece<XK>(frag_at_tile<XK>(xb, lds_addr(st)), 0);
    if constexpr ((FOLD || HW) && !ROWS) sbv = sat[BM + (wn * C::kWTN) / 128];
    if constexpr (FOLD || HW) c = lds_scale(scale_base(st));
  };
  // 1x128 weight scales of a block: fold, those of this lane's 4 output columns; MFMA, that of
  // its A-operand row.
  auto fold_row_scales = [&](const uint8_t* st, v4f (&sbr)[NI]) {
    if constexpr (ROWS && FOLD) {
      const float* sat = scales_of(st);
#pragma unroll
      for (int i = 0; i < NI; ++i)
        sbr[i] = *reinterpret_cast<const v4f*>(sat + BM + wn * C::kWTN + 16 * i + 4 * g);
    }
  };
  auto mfma_row_scales = [&](const uint8_t* st, int (&wbr)[NI]) {
    if constexpr (ROWS && HW) {
      const float* sat = scales_of(st);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if constexpr (MX)
          wbr[i] = (int)__float_as_uint(
              lds_u8_bits(lds_addr(sat + BM + wn * C::kWTN + 16 * i + li) + (uint32_t)g));
        else
          wbr[i] = e8m0_of(sat[BM + wn * C::kWTN + 16 * i + li]);
      }
    }
  };
  // The weight-side bases of a stage: piece i by frag_piece(wbase, i).
  auto w_bases = [&](const uint8_t* st) {
    return frag_at_tile<WK>(wb, lds_addr(st) + C::kXBytes);
  };

  const bool prefetched = PF && cy.prefetched;   // block 0 was issued by the previous tile
  if (!prefetched)
    for (int s = 0; s + 1 < C::kStages; ++s) issue(s, std::false_type{});
  v8i wf[NI], xf;
  float ccur = 0.0f, sbv = 1.0f, cprev = 0.0f;
  v4f sbr[NI], P[NI];
  int wbr[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) P[i] = v4f{0.f, 0.f, 0.f, 0.f};   // pending products (fold)
  if (nkb > 0) {
    // block 0 issued during the previous tile: only that tile's later stores may be pending
    if (prefetched) wait_vm_atmost<NI * NJ, (C::kStagedEpi ? 2 * NJ : NI * NJ)>(cy.stores);
    else wait_next();
    barrier();
    prepare(0);
    const uint8_t* st = stage_ptr(0);
    first_x(st, xf, ccur, sbv);
    if constexpr (FOLD && !ROWS) ccur *= sbv;
    const FragBase<WK> ws = w_bases(st);
#pragma unroll
    for (int i = 0; i < NI; ++i) wf[i] = frag_piece<WK>(ws, i);
    fold_row_scales(st, sbr);
    mfma_row_scales(st, wbr);
    if constexpr (kBurst) {
      issue(C::kStages - 1, std::false_type{});
    } else {
      const BlockDma d = block_dma(C::kStages - 1, std::false_type{});   // its first NI instructions
#pragma unroll
      for (int q = 0; q < NI && q < kPerStage; ++q) dma_part(d, q);
    }
  }

  // One K block.  TURN: block kb + 1 follows; PREP: it is the last block (whose bytes past a
  // ragged K are zeroed).  The variants keep every branch out of the common block, so that the
  // compiler keeps each fold next to its MFMAs.
  auto run_block = [&](int kb, auto turn_tag, auto prep_tag) {
    constexpr bool TURN = decltype(turn_tag)::value;
    constexpr bool PREP = decltype(prep_tag)::value;
    if constexpr (PF && PREP) {
      if (pf_live) nt = next_tile();   // (first needed by this block's hand-over)
    }
    const uint8_t* st = stage_ptr(kb);
    const uint8_t* stn = stage_ptr(kb + 1);
    const int wbyte = (HW && !ROWS) ? e8m0_of(sbv) : 0;   // weight scale of the block
    const FragBase<XK> xs = frag_at_tile<XK>(xb, lds_addr(st));
    const uint32_t scs = scale_base(st);
    FragBase<WK> wsn;
    // DMA of block kb + kStages - 1 (into the slot of block kb - 1): its first NI instructions
    // were issued at the previous hand-over, the rest go here (in the last block only when it
    // is the next tile's first block, PF).  DMA of block kb + kStages: started at this block's
    // hand-over.
    constexpr bool CONT = (TURN || PF) && !kBurst;
    BlockDma dcont, dturn;
    // (in the last block, PF: the next tile's first block)
    if constexpr (CONT) dcont = block_dma(kb + C::kStages - 1, std::bool_constant<!TURN>{});
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      v8i xnext;
      float cnext = 0.0f;
      if (j + 1 < NJ) {
        xnext = frag_piece<XK>(xs, j + 1);
        if constexpr (FOLD || HW) cnext = lds_scale(scs + 64u * (uint32_t)(j + 1));   // (fold: times sbv at the end)
      }
      const bool turn = TURN && j == NJ - 1;   // block kb + 1 is published before this piece
      if (turn) {
        __builtin_amdgcn_sched_barrier(0);
        wait_lds();   // this wave's reads of stage kb have completed
        wait_next();
        barrier();
        if constexpr (PREP && !FOLD) {
          // (the accumulations so far are complete here: otherwise the compiler may sink the
          // MFMAs of this block past the ragged-K branch of prepare, keeping their fragments
          // live -- and spilled -- across it)
#pragma unroll
          for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int jj = 0; jj + 1 < NJ; ++jj) asm volatile("" : "+v"(acc[i][jj]));
        }
        if constexpr (PREP) prepare(kb + 1);
        if constexpr (!kBurst) dturn = block_dma(kb + C::kStages, std::bool_constant<PF && PREP>{});
        first_x(stn, xnext, cnext, sbv);
        wsn = w_bases(stn);
        __builtin_amdgcn_sched_barrier(0);
      }
      // activation scale of this lane's row (microscaling: and of its k chunk)
      const int xbyte = !HW ? 0 : MX ? (int)__float_as_uint(ccur) : e8m0_of(ccur);
      // The piece's MFMAs and folds issue at raised wave priority: when both waves of a SIMD
      // are ready, the one feeding the matrix core goes first (measured 1.5% faster than equal
      // priorities, 1.1% faster than raising it only after the hand-over).
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if constexpr (FOLD) {
          // Unit i: the MFMA of (piece j, n piece i) and the fold of the previous piece's n
          // piece i, whose MFMA was issued NI MFMAs earlier and has completed.  The scheduling
          // barrier keeps the compiler from pulling the fold of an MFMA right behind that MFMA
          // (which would stall the wave on every MFMA result).
          const v4f pn = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wf[i], xf, v4f{0.f, 0.f, 0.f, 0.f}, FB, FA, 0, 0, 0, 0);
          // (the empty asm pins the fold here: the compiler would otherwise sink it towards
          // the accumulator's next use, keeping every pending product alive)
          if (j > 0) {
            if constexpr (ROWS) acc[i][j - 1] += P[i] * (sbr[i] * cprev);   // sb[n..n+3] * sa[m]
            else acc[i][j - 1] += P[i] * cprev;
            asm volatile("" : "+v"(acc[i][j - 1]));
          } else {
            // the last piece of the previous block (zero products before the first block),
            // with that block's weight scales (1x128: replaced after this piece's MFMAs)
            if constexpr (ROWS) acc[i][NJ - 1] += P[i] * (sbr[i] * cprev);
            else acc[i][NJ - 1] += P[i] * cprev;
            asm volatile("" : "+v"(acc[i][NJ - 1]));
          }
          P[i] = pn;
        } else if constexpr (HW) {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wf[i], xf, acc[i][j], FB, FA, 0, ROWS ? wbr[i] : wbyte, 0, xbyte);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[i], xf, acc[i][j], FB,
                                                                       FA, 0, 0, 0, 0);
        }
        if (turn) {
          wf[i] = frag_piece<WK>(wsn, i);
          if (!kBurst && i < kPerStage) dma_part(dturn, i);
        } else if constexpr (CONT) {
          const int q = NI + j * NI + i;
          if (q < kPerStage) dma_part(dcont, q);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      if (turn) {
        mfma_row_scales(stn, wbr);
        if constexpr (kBurst) issue(kb + C::kStages, std::bool_constant<PF && PREP>{});
        __builtin_amdgcn_sched_barrier(0);
      }
      if (j == 0) {
        fold_row_scales(st, sbr);   // first needed by the folds of this piece, in the next
        __builtin_amdgcn_sched_barrier(0);
      }
      cprev = ccur;
      if (j + 1 < NJ || TURN) {
        xf = xnext;
        // (fold with 128x128 weight scales: sbv is the next piece's block's, also after a turn)
        ccur = (FOLD && !ROWS) ? cnext * sbv : cnext;
      }
    }
  };
  for (int kb = 0; kb + 2 < nkb; ++kb) run_block(kb, std::true_type{}, std::false_type{});
  if (nkb >= 2) run_block(nkb - 2, std::true_type{}, std::true_type{});
  if (nkb >= 1) run_block(nkb - 1, std::false_type{}, std::false_type{});
  if (!pf_live) wait_vm<0>();   // DMAs of blocks past the last
  if constexpr (FOLD) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if constexpr (ROWS) acc[i][NJ - 1] += P[i] * (sbr[i] * cprev);
      else acc[i][NJ - 1] += P[i] * cprev;
    }
  }

  float post = 1.0f;
  if constexpr (SM == kScaleTensor) post = nkb > 0 ? p.sa[0] * sbw[0] : 0.0f;

  // Epilogue: lane holds C[m][n .. n+3] of each piece.
  if (p.C) {
    // (the wave's columns inside the output, and how many of its rows: tests once per tile)
    const bool cols_in = n0 + wn * C::kWTN + C::kWTN <= p.N;
    const int rows_in = (int)std::min<int64_t>(m_end - (m0 + wm * C::kWTM), C::kWTM);
    uint8_t* const region = smem + C::kEpi + w * C::kEpiWaveBytes;
    if (C::kStagedEpi && p.c_vec16 && cols_in && rows_in == C::kWTM) {
      store_wave_staged<C, SM, false>(p, t, wm, wn, lane, acc, post, region, rows_in);
    } else if (CUT_ROWS && C::kStagedEpi && p.c_vec16 && cols_in) {
      if (rows_in > 0) store_wave_staged<C, SM, true>(p, t, wm, wn, lane, acc, post, region, rows_in);
    } else if (C::kStagedEpi && p.c_vec16) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        v4f v[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          v[i] = acc[i][j];
          if constexpr (SM == kScaleTensor) v[i] = v[i] * post;
          if (nkb == 0) v[i] = v4f{0.f, 0.f, 0.f, 0.f};
        }
        store_rows_staged<C>(p, t, wm, wn, lane, j, v, region);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          v4f v = acc[i][j];
          if constexpr (SM == kScaleTensor) v = v * post;
          if (nkb == 0) v = v4f{0.f, 0.f, 0.f, 0.f};
          store_piece<C>(p, t, wm, wn, li, g, i, j, v);
        }
    }
  }
  if constexpr (QO != 0) quantize_out<C, SM, QO>(p, smem, acc, post, nkb, m0, m_end, n0);
  if constexpr (PF) {
    // Store instructions the wave issued above, at least: one per (n piece, m piece) whose first
    // column and row lie inside the output (a lane of that piece stores).
    int iv = 0, jv = 0, hv = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      jv += (m0 + wm * C::kWTM + 16 * j < m_end) ? 1 : 0;
      hv += (m0 + wm * C::kWTM + 16 * j < m_end) ? 1 : 0;
      hv += (m0 + wm * C::kWTM + 16 * j + 8 < m_end) ? 1 : 0;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) iv += (n0 + wn * C::kWTN + 16 * i < p.N) ? 1 : 0;
    // (staged epilogue: at least one store instruction per 8-row half of an m piece whose first
    // row is inside, when the wave's first column is)
    cy.stores = p.C ? ((C::kStagedEpi && p.c_vec16) ? (iv > 0 ? hv : 0) : iv * jv) : 0;
    cy.prefetched = pf_live ? 1 : 0;
    cy.stage0 = (int)((uint32_t)(st0 + nkb) % C::kStages);
  }
}


// Map a linear workgroup id to a tile so that each of the 8 XCDs (ids are dealt round robin)
// gets a contiguous range of tiles, ordered in groups of GROUP_M tile-rows for L2 reuse.
template <int GROUP_M = kGroupM>
__device__ __forceinline__ void tile_of(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int q = total / 8, r = total % 8;
  const int xcd = id % 8, local = id / 8;
  const int pid = xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
  const int width = GROUP_M * tiles_n;
  const int grp = pid / width;
  const int first = grp * GROUP_M;
  const int gsz = min(tiles_m - first, GROUP_M);
  const int in = pid % width;
  tm = first + in % gsz;
  tn = in / gsz;
}

template <class C, int LAYOUT, int FA, int FB, int SM, int QO = 0>
__global__ __launch_bounds__(C::kThreads, 1) void gemm_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(128))) uint8_t smem[];
  int tm, tn;
  tile_of(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * C::BM;
  const Tile t{0, m0, (int)std::min<int64_t>((int64_t)m0 + C::BM, p.M), tn * C::BN};
  Carry cy{0, 0, 0};
  Tile nt = t;
  gemm_tile<C, LAYOUT, FA, FB, SM, QO>(p, smem, t, nt, [&]() { return t; }, false, cy);
}

// The kernel parameters, read again from the argument segment (scalar loads) where a
// persistent kernel starts a tile, so that values derived from them are not kept live across
// the whole tile loop.
#if defined(__HIP_DEVICE_COMPILE__)
#define FP8BS_REREAD_PARAMS(q, p)                                                      \
  typedef const __attribute__((address_space(4))) GemmParams* ParamPtr;               \
  ParamPtr pp_ = (ParamPtr)__builtin_amdgcn_kernarg_segment_ptr();                    \
  asm volatile("" : "+s"(pp_));                                                       \
  const GemmParams q = *pp_
#else
#define FP8BS_REREAD_PARAMS(q, p) const GemmParams& q = p   /* (host pass: never run) */
#endif

// Dense GEMM on a persistent grid (one workgroup per CU; 256x256 tiles, two LDS stages): each
// workgroup walks tiles id, id + grid, ... in the XCD-local order of tile_of and loads the next
// tile's first K block during the current tile's last block, so that block's load overlaps
// the epilogue's stores.
template <class C, int LAYOUT, int FA, int FB, int SM>
__global__ __launch_bounds__(C::kThreads, 1) void gemm_persistent_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(128))) uint8_t smem[];
  static_assert(C::kStages == 2, "persistent dense GEMM: two-stage tiles");
  const int total = p.tiles_m * p.tiles_n;
  int id = blockIdx.x;
  if (id >= total) return;
  auto tile_at = [&](int i) {
    int tm, tn;
    tile_of(i, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = __builtin_amdgcn_readfirstlane(tm) * C::BM;
    return Tile{0, m0, (int)std::min<int64_t>((int64_t)m0 + C::BM, p.M),
                __builtin_amdgcn_readfirstlane(tn) * C::BN};
  };
  Tile cur = tile_at(id);
  Carry cy{0, 0, 0};
  while (true) {
    const int nid = id + (int)gridDim.x;
    const bool has_next = nid < total;
    Tile nxt = cur;
    FP8BS_REREAD_PARAMS(q, p);
    gemm_tile<C, LAYOUT, FA, FB, SM, 0, true, true>(q, smem, cur, nxt,
                                                    [&]() { return tile_at(nid); }, has_next, cy);
    if (!has_next) break;
    if (!cy.prefetched) {
      __syncthreads();   // the next tile refills the LDS stages
      nxt = tile_at(nid);   // (not formed during the tile: fewer than two K blocks)
    }
    cur = nxt;
    id = nid;
  }
}

// Grouped: a persistent grid walks the concatenation of every group's m tiles (times the n
// tiles).  Each workgroup first builds, in LDS, the group bounds -- each offset clamped to
// [0, M] and raised to the largest offset before it, so that groups never overlap and a
// decreasing offset empties the groups it would have reopened -- and the prefix count of m
// tiles per group, then maps each of its tiles to (group, m tile, n tile) by binary search.
// With two LDS stages the next tile's first K block is loaded while the current tile finishes
// (see gemm_tile).
constexpr int kMaxGroups = 1024;

// Inclusive scan of v over the workgroup's threads in index order (op: max or +), continued
// from carry; also returns the total through carry.  Every thread of the workgroup calls it.
template <int THREADS, bool MAX>
__device__ __forceinline__ int block_scan(int v, int& carry, int* s_wave) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off);
    if (lane >= off) v = MAX ? max(v, o) : v + o;
  }
  if (lane == 63) s_wave[threadIdx.x >> 6] = v;
  __syncthreads();
  int before = carry;
  for (int w = 0; w < (int)(threadIdx.x >> 6); ++w)
    before = MAX ? max(before, s_wave[w]) : before + s_wave[w];
  int total = carry;
  for (int w = 0; w < THREADS / 64; ++w) total = MAX ? max(total, s_wave[w]) : total + s_wave[w];
  carry = total;
  __syncthreads();
  return MAX ? max(before, v) : before + v;
}

template <class C, int FA, int FB, int SM>
__global__ __launch_bounds__(C::kThreads, 1) void grouped_gemm_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(128))) uint8_t smem[];
  __shared__ int s_prefix[kMaxGroups + 1];
  __shared__ int s_lo[kMaxGroups + 1];   // group bounds, clamped and non-decreasing (M < 2^31)
  __shared__ int s_wave_sum[C::kWaves];
  constexpr int BM = C::BM;
  constexpr bool PF = C::kStages == 2;
  const int G = p.num_groups;
  int run_max = 0;
  for (int base = 0; base <= G; base += C::kThreads) {
    const int gi = base + threadIdx.x;
    const int v = gi <= G ? (int)std::min<int64_t>(std::max<int64_t>(p.offsets[gi], 0), p.M) : 0;
    const int m = block_scan<C::kThreads, true>(v, run_max, s_wave_sum);
    if (gi <= G) s_lo[gi] = m;
  }
  __syncthreads();
  // m tiles per group, prefix-summed
  int carry = 0;
  for (int base = 0; base < G; base += C::kThreads) {
    const int gi = base + threadIdx.x;
    const int tiles = gi < G ? (s_lo[gi + 1] - s_lo[gi] + BM - 1) / BM : 0;
    const int v = block_scan<C::kThreads, false>(tiles, carry, s_wave_sum);
    if (gi < G) s_prefix[gi + 1] = v;
  }
  if (threadIdx.x == 0) s_prefix[0] = 0;
  __syncthreads();
  const int m_tiles = s_prefix[G];
  const int tiles_n = p.tiles_n;
  const int total = m_tiles * tiles_n;
  // Workgroup id + k * gridDim stays on the XCD of the workgroup (the grid is a multiple of 8),
  // and tile_of gives each XCD a contiguous range of the concatenated tiles in groups of m
  // tiles, so the 32 workgroups of an XCD share A rows and expert weight tiles in its L2.
  auto tile_at = [&](int id) {
    int mt, tn;
    tile_of<kGroupMGrouped>(id, m_tiles, tiles_n, mt, tn);
    // the last group with s_prefix[g] <= mt (the prefix does not decrease): the number of
    // g in [1, G) with s_prefix[g] <= mt, counted 64 groups at a time by the wave's lanes (one
    // LDS round trip per 64 groups instead of one per step of a binary search)
    int cnt = 0;
    for (int base = 1; base < G; base += 64) {
      const int gq = base + (int)(threadIdx.x & 63);
      cnt += __popcll(__ballot(gq < G && s_prefix[gq] <= mt));
    }
    // (the same in every lane: kept in scalar registers)
    const int gi = __builtin_amdgcn_readfirstlane(cnt);
    const int glo = __builtin_amdgcn_readfirstlane(s_lo[gi]);
    const int ghi = __builtin_amdgcn_readfirstlane(s_lo[gi + 1]);
    const int m0 = glo + __builtin_amdgcn_readfirstlane(mt - s_prefix[gi]) * BM;
    return Tile{gi, m0, std::min(m0 + BM, ghi), __builtin_amdgcn_readfirstlane(tn) * C::BN};
  };
  int id = blockIdx.x;
  if (id >= total) return;
  Tile cur = tile_at(id);
  Carry cy{0, 0, 0};
  while (true) {
    const int nid = id + (int)gridDim.x;
    const bool has_next = nid < total;
    Tile nxt = cur;
    FP8BS_REREAD_PARAMS(q, p);
    gemm_tile<C, FP8BS_FPROP, FA, FB, SM, 0, PF, true, true>(q, smem, cur, nxt,
                                                       [&]() { return tile_at(nid); }, has_next,
                                                       cy);
    if (!has_next) break;
    if (!cy.prefetched) {
      __syncthreads();   // the next tile refills the LDS stages
      nxt = tile_at(nid);   // (not formed during the tile: fewer than two K blocks, or no prefetch)
    }
    cur = nxt;
    id = nid;
  }
}

// Launch one GEMM kernel.  Kernels that use more than 64 KiB of dynamic LDS need the limit
// raised once per device; that is done on the first launch of each kernel instantiation on a
// device (a bit per device, set after the call succeeded), so later launches only enqueue.
constexpr int kMaxDevices = 64;

// Compute units of the current device, read once per device (the persistent grouped grid has
// one workgroup per CU).  0 when the device cannot be queried.
inline int device_cus() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 0;
  cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

template <auto KERNEL>
int launch_gemm(int blocks, int threads, int lds, hipStream_t st, const GemmParams& p) {
  static std::atomic<uint64_t> lds_ready{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8BS_ERR_LAUNCH;
  const uint64_t bit = uint64_t(1) << dev;
  if (!(lds_ready.load(std::memory_order_acquire) & bit)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(KERNEL),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
      return FP8BS_ERR_LAUNCH;
    lds_ready.fetch_or(bit, std::memory_order_acq_rel);
  }
  void* args[] = {const_cast<GemmParams*>(&p)};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(KERNEL), dim3(blocks),
                                 dim3(threads), args, lds, st);
  return e == hipSuccess ? FP8BS_OK : FP8BS_ERR_LAUNCH;
}

// Tile configurations.
using CfgA = Cfg<256, 128, 2, 2>;   // 4 waves, 128 x 64 per wave, 3 stages
using CfgB = Cfg<256, 128, 4, 2>;   // 8 waves, 64 x 64 per wave, 3 stages
using CfgC = Cfg<256, 256, 2, 4>;   // 8 waves, 128 x 64 per wave, 2 stages
using CfgD = Cfg<128, 128, 2, 2>;   // 4 waves, 64 x 64 per wave (small M, grouped)

// Two-stage tiles without fused output quantization run on the persistent grid (one
// workgroup per CU, deferred epilogue); the others one workgroup per tile.
template <class C, int LAYOUT, int FA, int FB, int SM, int QO = 0>
int launch_dense(GemmParams p, hipStream_t st) {
  p.tiles_m = (int)ceil_div(p.M, C::BM);
  p.tiles_n = (int)ceil_div(p.N, C::BN);
  if ((int64_t)p.tiles_m * p.tiles_n > 0x7FFFFFFF) return FP8BS_ERR_SHAPE;
  const int tiles = p.tiles_m * p.tiles_n;
  if constexpr (C::kStages == 2 && QO == 0 && kPersistentDense) {
    const int cus = device_cus();
    if (cus <= 0) return FP8BS_ERR_LAUNCH;
    return launch_gemm<gemm_persistent_kernel<C, LAYOUT, FA, FB, SM>>(std::min(tiles, cus),
                                                                      C::kThreads, C::kLds, st, p);
  } else {
    return launch_gemm<gemm_kernel<C, LAYOUT, FA, FB, SM, QO>>(tiles, C::kThreads, C::kLds, st, p);
  }
}

// Tile configuration of a dense GEMM: FP8BS_TILE_AUTO takes the largest tile that still gives
// every CU at least one workgroup (two waves per SIMD hide LDS and MFMA latency best); any
// other value of fp8bs_tile forces that configuration (the *_tiled entry points).
char pick_variant(int64_t M, int64_t N, int tile) {
  switch (tile) {
    case FP8BS_TILE_256x128_W4: return 'A';
    case FP8BS_TILE_256x128_W8: return 'B';
    case FP8BS_TILE_256x256_W8: return 'C';
    case FP8BS_TILE_128x128_W4: return 'D';
    default: break;
  }
  if (ceil_div(M, 256) * ceil_div(N, 256) >= 256) return 'C';
  if (ceil_div(M, 256) * ceil_div(N, 128) >= 256) return 'B';
  return 'D';
}

inline bool tile_ok(int tile) { return tile >= FP8BS_TILE_AUTO && tile <= FP8BS_TILE_128x128_W4; }

template <int LAYOUT, int FA, int FB, int SM, int QO = 0>
int dispatch_variant(const GemmParams& p, int tile, hipStream_t st) {
  switch (pick_variant(p.M, p.N, tile)) {
    case 'B': return launch_dense<CfgB, LAYOUT, FA, FB, SM, QO>(p, st);
    case 'C': return launch_dense<CfgC, LAYOUT, FA, FB, SM, QO>(p, st);
    case 'D': return launch_dense<CfgD, LAYOUT, FA, FB, SM, QO>(p, st);
    default: return launch_dense<CfgA, LAYOUT, FA, FB, SM, QO>(p, st);
  }
}

template <int LAYOUT, int SM>
int dispatch_formats(int fa, int fb, const GemmParams& p, int tile, hipStream_t st) {
  if (fa == FP8BS_E4M3 && fb == FP8BS_E4M3) return dispatch_variant<LAYOUT, FP8BS_E4M3, FP8BS_E4M3, SM>(p, tile, st);
  if (fa == FP8BS_E5M2 && fb == FP8BS_E4M3) return dispatch_variant<LAYOUT, FP8BS_E5M2, FP8BS_E4M3, SM>(p, tile, st);
  if (fa == FP8BS_E4M3 && fb == FP8BS_E5M2) return dispatch_variant<LAYOUT, FP8BS_E4M3, FP8BS_E5M2, SM>(p, tile, st);
  return dispatch_variant<LAYOUT, FP8BS_E5M2, FP8BS_E5M2, SM>(p, tile, st);
}

template <int SM>
int dispatch_dense(int layout, int fa, int fb, const GemmParams& p, int tile, hipStream_t st) {
  if constexpr (SM == kScaleFoldRows || SM == kScaleHwRows) {
    // 1x128 weight scales need a K-major weight operand: fprop only (checked by the caller)
    return dispatch_formats<FP8BS_FPROP, SM>(fa, fb, p, tile, st);
  }
  switch (layout) {
    case FP8BS_FPROP: return dispatch_formats<FP8BS_FPROP, SM>(fa, fb, p, tile, st);
    case FP8BS_DGRAD: return dispatch_formats<FP8BS_DGRAD, SM>(fa, fb, p, tile, st);
    default: return dispatch_formats<FP8BS_WGRAD, SM>(fa, fb, p, tile, st);
  }
}

// Scale indexing for one operand.  rows: the operand's output dimension (m or n);
// kmajor: the operand is stored [rows, K] (else [K, rows]).
struct ScaleIndex {
  int64_t ks, rs, bytes;
  int rshift;   // scale row of operand row r: r >> rshift
};

bool scale_index(int gran, bool kmajor, bool weight_side, int64_t rows, int64_t K,
                 ScaleIndex& s) {
  const int64_t kblocks = ceil_div(K, 128), rblocks = ceil_div(rows, 128);
  if (gran == FP8BS_PER_TENSOR) {
    s = {0, 0, 4, 0};
    return true;
  }
  if (gran == FP8BS_BLOCK_1x128) {
    if (!kmajor) return false;                  // 1x128 blocks run along K: K-major operands only
    (void)weight_side;
    s = {rows, 1, kblocks * rows * 4, 0};       // float[K/128][rows]
    return true;
  }
  if (gran == FP8BS_BLOCK_128x128) {
    if (kmajor) s = {1, kblocks, rblocks * kblocks * 4, 7};   // float[rows/128][K/128]
    else s = {rblocks, 1, kblocks * rblocks * 4, 7};          // float[K/128][rows/128]
    return true;
  }
  return false;
}

// Grouped GEMM tile configuration: FP8BS_TILE_AUTO takes 256x256 (fastest on the MoE shapes
// despite the padding of ragged 256-row tiles); FP8BS_TILE_256x128_W8 and
// FP8BS_TILE_128x128_W4 force the others.
inline bool grouped_tile_ok(int tile) {
  return tile == FP8BS_TILE_AUTO || tile == FP8BS_TILE_256x128_W8 ||
         tile == FP8BS_TILE_256x256_W8 || tile == FP8BS_TILE_128x128_W4;
}

template <class C, int SM>
int launch_grouped(int fa, int fb, int cus, GemmParams p, hipStream_t st) {
  p.tiles_n = (int)ceil_div(p.N, C::BN);
  p.tiles_m = (int)(ceil_div(p.M, C::BM) + p.num_groups);   // upper bound on m tiles
  if ((int64_t)p.tiles_m * p.tiles_n > 0x7FFFFFFF) return FP8BS_ERR_SHAPE;
  const int blocks = (int)std::min<int64_t>((int64_t)p.tiles_m * p.tiles_n, std::max(cus, 1));
  constexpr int E4 = FP8BS_E4M3, E5 = FP8BS_E5M2;
  if (fa == E4 && fb == E4) return launch_gemm<grouped_gemm_kernel<C, E4, E4, SM>>(blocks, C::kThreads, C::kLds, st, p);
  if (fa == E5 && fb == E4) return launch_gemm<grouped_gemm_kernel<C, E5, E4, SM>>(blocks, C::kThreads, C::kLds, st, p);
  if (fa == E4 && fb == E5) return launch_gemm<grouped_gemm_kernel<C, E4, E5, SM>>(blocks, C::kThreads, C::kLds, st, p);
  return launch_gemm<grouped_gemm_kernel<C, E5, E5, SM>>(blocks, C::kThreads, C::kLds, st, p);
}

template <int SM>
int dispatch_grouped(int fa, int fb, int cus, const GemmParams& p, int tile, hipStream_t st) {
  switch (tile) {
    case FP8BS_TILE_256x128_W8: return launch_grouped<CfgB, SM>(fa, fb, cus, p, st);
    case FP8BS_TILE_128x128_W4: return launch_grouped<CfgD, SM>(fa, fb, cus, p, st);
    default: return launch_grouped<CfgC, SM>(fa, fb, cus, p, st);
  }
}


// ------------------------------------------------------------------ argument checks (host)
// Validates the dense GEMM arguments and fills p.  tensor_only: both operands carry per-tensor
// scales.  b_rows: the weight side carries 1x128 scales.  empty: nothing to compute (M == 0 or
// N == 0); the status is then FP8BS_OK.
inline int dense_params(int layout, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                        int fa, int ga, const float* scale_inv_a, const void* B, int64_t ldb,
                        int fb, int gb, const float* scale_inv_b, void* C_bf16, int64_t ldc,
                        GemmParams& p, bool& tensor_only, bool& empty, bool& b_rows,
                        bool c_optional = false) {
  empty = false;
  if (layout < FP8BS_FPROP || layout > FP8BS_WGRAD || !fmt_ok(fa) || !fmt_ok(fb) || ga < 0 ||
      ga > 2 || gb < 0 || gb > 2)
    return FP8BS_ERR_ARG;
  if (M < 0 || N < 0 || K < 0) return FP8BS_ERR_SHAPE;
  if (M == 0 || N == 0) {
    empty = true;
    return FP8BS_OK;
  }
  if ((!C_bf16 && !c_optional) || (K > 0 && (!A || !B || !scale_inv_a || !scale_inv_b)))
    return FP8BS_ERR_NULL;
  const bool xk = layout != FP8BS_WGRAD, wk = layout == FP8BS_FPROP;
  const int64_t a_width = xk ? K : M, b_width = wk ? K : N;
  if ((C_bf16 && ldc < N) || (K > 0 && (lda < a_width || ldb < b_width))) return FP8BS_ERR_SHAPE;
  // 32-bit buffer offsets inside a tile: 256 rows of the pitch must stay below 2^31.
  if (lda >= (int64_t(1) << 23) || ldb >= (int64_t(1) << 23)) return FP8BS_ERR_SHAPE;
  if (M > (int64_t(1) << 31) - 256 || N > (int64_t(1) << 31) - 256) return FP8BS_ERR_SHAPE;
  if (K > 0 && (!aligned16(A) || !aligned16(B) || lda % 16 || ldb % 16)) return FP8BS_ERR_ALIGN;
  if (C_bf16 && (!aligned4(C_bf16) || ldc % 2)) return FP8BS_ERR_ALIGN;
  ScaleIndex sa{}, sb{};
  if (!scale_index(ga, xk, false, M, K, sa) || !scale_index(gb, wk, true, N, K, sb))
    return FP8BS_ERR_UNSUPPORTED;
  // scale arrays below 4 GiB (the kernels size their scale DMA in 32 bits)
  if (sa.bytes >= (int64_t(1) << 32) || sb.bytes >= (int64_t(1) << 32)) return FP8BS_ERR_SHAPE;
  p = GemmParams{};
  p.M = M; p.N = N; p.K = K;
  p.A = static_cast<const uint8_t*>(A); p.lda = lda;
  p.B = static_cast<const uint8_t*>(B); p.ldb = ldb;
  p.sa = scale_inv_a; p.sa_ks = sa.ks; p.sa_rs = sa.rs; p.sa_bytes = sa.bytes; p.sa_rshift = sa.rshift;
  p.sb = scale_inv_b; p.sb_ks = sb.ks; p.sb_rs = sb.rs; p.sb_bytes = sb.bytes;
  p.C = static_cast<uint16_t*>(C_bf16); p.ldc = ldc;
  p.c_vec = (reinterpret_cast<uintptr_t>(C_bf16) % 8 == 0) && (ldc % 4 == 0);
  p.c_vec16 = (reinterpret_cast<uintptr_t>(C_bf16) % 16 == 0) && (ldc % 8 == 0);
  tensor_only = ga == FP8BS_PER_TENSOR && gb == FP8BS_PER_TENSOR;
  b_rows = gb == FP8BS_BLOCK_1x128;   // only accepted for a K-major weight operand (fprop)
  return FP8BS_OK;
}

// Validates the grouped GEMM arguments and fills p (empty: nothing to compute, status OK).
inline int grouped_params(int32_t num_groups, const int64_t* group_offsets, int64_t total_M,
                          int64_t N, int64_t K, const void* A, int64_t lda, int fa,
                          const float* scale_inv_a, const void* B, int64_t ldb, int fb,
                          const float* scale_inv_b, void* C_bf16, int64_t ldc, GemmParams& p,
                          bool& empty) {
  empty = false;
  if (!fmt_ok(fa) || !fmt_ok(fb) || num_groups < 0 || num_groups > kMaxGroups)
    return FP8BS_ERR_ARG;
  if (total_M < 0 || N < 0 || K < 0) return FP8BS_ERR_SHAPE;
  if (total_M == 0 || N == 0 || num_groups == 0) {
    empty = true;
    return FP8BS_OK;
  }
  if (K == 0) return FP8BS_ERR_SHAPE;
  if (!group_offsets || !A || !B || !scale_inv_a || !scale_inv_b || !C_bf16) return FP8BS_ERR_NULL;
  if (lda < K || ldb < K || ldc < N) return FP8BS_ERR_SHAPE;
  if (lda >= (int64_t(1) << 23) || ldb >= (int64_t(1) << 23)) return FP8BS_ERR_SHAPE;
  if (total_M > (int64_t(1) << 31) - 256 || N > (int64_t(1) << 31) - 256) return FP8BS_ERR_SHAPE;
  if (!aligned16(A) || !aligned16(B) || lda % 16 || ldb % 16) return FP8BS_ERR_ALIGN;
  if (!aligned4(C_bf16) || ldc % 2 || (reinterpret_cast<uintptr_t>(group_offsets) & 7))
    return FP8BS_ERR_ALIGN;
  p = GemmParams{};
  p.M = total_M; p.N = N; p.K = K;
  p.A = static_cast<const uint8_t*>(A); p.lda = lda;
  p.B = static_cast<const uint8_t*>(B); p.ldb = ldb;
  p.sa = scale_inv_a; p.sa_ks = total_M; p.sa_rs = 1; p.sa_rshift = 0;
  p.sa_bytes = ceil_div(K, 128) * total_M * 4;
  p.sb = scale_inv_b; p.sb_ks = 1; p.sb_rs = ceil_div(K, 128);
  p.C = static_cast<uint16_t*>(C_bf16); p.ldc = ldc;
  p.c_vec = (reinterpret_cast<uintptr_t>(C_bf16) % 8 == 0) && (ldc % 4 == 0);
  p.c_vec16 = (reinterpret_cast<uintptr_t>(C_bf16) % 16 == 0) && (ldc % 8 == 0);
  p.offsets = group_offsets;
  p.num_groups = num_groups;
  p.b_group_stride = N * ldb;
  p.sb_group_stride = ceil_div(N, 128) * ceil_div(K, 128);
  p.sb_bytes = p.sb_group_stride * 4;   // one group's weight scales
  // scale arrays below 4 GiB (the kernels size their scale DMA in 32 bits)
  if (p.sa_bytes >= (int64_t(1) << 32) || p.sb_bytes >= (int64_t(1) << 32)) return FP8BS_ERR_SHAPE;
  return FP8BS_OK;
}

}  // namespace

// The dense kernels of one layout (and scale family) are instantiated in a translation unit of
// their own, so that the library's sources compile in parallel: gemm_fprop.hip (fp32 block,
// 1x128-both and per-tensor scales), gemm_fprop_pow2.hip (E8M0 scales), gemm_mx.hip
// (microscaling), gemm_dgrad.hip,
// gemm_wgrad.hip, gemm_grouped.hip.  sm is one of the kScale* modes above; hidden symbols, not
// part of the C ABI.
#define FP8BS_HIDDEN __attribute__((visibility("hidden")))
FP8BS_HIDDEN int gemm_fprop_fp32(int sm, int fa, int fb, const GemmParams& p, int tile, hipStream_t st);
FP8BS_HIDDEN int gemm_fprop_pow2(int sm, int fa, int fb, const GemmParams& p, int tile, hipStream_t st);
FP8BS_HIDDEN int gemm_fprop_mx(int fa, int fb, const GemmParams& p, int tile, hipStream_t st);
FP8BS_HIDDEN int gemm_grouped_mx(int fa, int fb, int cus, const GemmParams& p, int tile,
                                 hipStream_t st);
FP8BS_HIDDEN int gemm_dgrad(int sm, int fa, int fb, const GemmParams& p, int tile, hipStream_t st);
FP8BS_HIDDEN int gemm_wgrad(int sm, int fa, int fb, const GemmParams& p, int tile, hipStream_t st);
FP8BS_HIDDEN int gemm_grouped(bool pow2, int fa, int fb, int cus, const GemmParams& p, int tile,
                              hipStream_t st);

}  // namespace fp8bs
