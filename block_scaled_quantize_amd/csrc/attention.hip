// FP8 KV cache for gfx950: the cache writer and grouped-query decode attention over the cache.
//
// Method: "NVIDIA NeMo RL logra una aceleración del 48% con entrenamiento de precisión FP8 de
// extremo a extremo", section "Ganancias de rendimiento en el mundo real": FP8 is extended to
// the KV cache and to attention.  The pages fix no cache format; the one used here is the
// activation recipe of section "El avance técnico" applied to cached keys and values: E4M3 (or
// E5M2) codes with one fp32 scale per 128-element head vector, quantized by the blockwise 1x128
// rule.  Attention reads the codes (half the bytes of a bf16 cache), dequantizes in registers
// and computes in fp32.
//
// Cache layout: codes [B][T][KVH][128] (the KVH head vectors of a token adjacent, 128 bytes
// each), dequantization factors float [B][T][KVH].
//
// Writer: 8 lanes per head vector (16 bf16 per lane, two 16-byte loads), the 1x128 rule of the
// blockwise quantizer (amax over the 8 lanes by DPP, the same scale, encode and NaN handling).
//
// Decode attention (HBM-bound: every cached byte is read once per step): one workgroup of 4
// waves per (sequence, KV head) -- or per (sequence, KV head, chunk of tokens) in the split
// form, whose partial results a second kernel merges -- with the query-key and the
// probability-value products on the matrix cores (attn_decode_mma_kernel, below), the softmax
// online in base 2, and the four waves' partial results merged through LDS at the end.
#include <math.h>

#include "common.h"

namespace fp8bs {
namespace {

// ---------------------------------------------------------------- cache writer
constexpr int kAppendThreads = 256;   // 32 head vectors per workgroup

template <int FMT, bool POW2>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(
    int64_t B, int64_t KVH, int64_t T, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, const int32_t* __restrict__ positions,
    uint8_t* __restrict__ k_codes, float* __restrict__ k_si, uint8_t* __restrict__ v_codes,
    float* __restrict__ v_si) {
  const int64_t vectors = 2 * KVH;   // K heads then V heads of one sequence
  const int64_t b = blockIdx.y;
  const int64_t gi = (int64_t)blockIdx.x * (kAppendThreads / 8) + (threadIdx.x >> 3);
  const int l8 = threadIdx.x & 7;
  if (gi >= vectors) return;
  const int64_t pos = positions[b];
  if (pos < 0 || pos >= T) return;
  const bool is_v = gi >= KVH;
  const int64_t kvh = is_v ? gi - KVH : gi;
  const uint16_t* src = (is_v ? v_new : k_new) + (b * KVH + kvh) * 128 + l8 * 16;
  const uint4 a = *reinterpret_cast<const uint4*>(src);
  const uint4 c = *reinterpret_cast<const uint4*>(src + 8);
  const uint32_t d[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
  const uint32_t amax = group8_max(amax16_bits(d));   // the 8 lanes of this head vector
  const float s = scale_from_amax_bits<FMT, POW2>(amax);
  const uint4 q = amax < 0x7F80u ? encode16<FMT, true>(d, s)
                                 : patch_nan16(encode16<FMT, false>(d, s), d);
  const int64_t row = (b * T + pos) * KVH + kvh;
  *reinterpret_cast<uint4*>((is_v ? v_codes : k_codes) + row * 128 + l8 * 16) = q;
  if (l8 == 0) (is_v ? v_si : k_si)[row] = 1.0f / s;
}

// ---------------------------------------------------------------- decode attention
constexpr int kAttnWaves = 4;   // waves per workgroup (one workgroup per sequence and KV head)

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

// Buffer resource over nbytes (at most 4 GiB - 1) from base: raw 32-bit data, offsets at or
// past nbytes read as zero.
__device__ __forceinline__ uint4 attn_rsrc(const void* base, uint64_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  uint4 r;
  r.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  r.z = __builtin_amdgcn_readfirstlane(nbytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)nbytes);
  r.w = 0x00020000u;
  return r;
}
typedef unsigned int attn_u32x4 __attribute__((ext_vector_type(4)));
// 16 bytes per lane from buffer offset voff to LDS address lds + 16 * lane.
__device__ __forceinline__ void attn_dma16(uint4 rsrc, uint32_t voff, uint32_t lds) {
  const attn_u32x4 r = {rsrc.x, rsrc.y, rsrc.z, rsrc.w};
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(r), "s"(lds) : "memory", "m0");
}

// Eight FP8 codes (bytes of w.x then w.y) as bf16 (exact).
template <int FMT>
__device__ __forceinline__ bf16x8 decode8_bf16(v2i w) {
  bf16x2 a, b, c, d;
  if constexpr (FMT == FP8BS_E4M3) {
    a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false);
    b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true);
    c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false);
    d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true);
  } else {
    a = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w.x, 1.0f, false);
    b = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w.x, 1.0f, true);
    c = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w.y, 1.0f, false);
    d = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w.y, 1.0f, true);
  }
  return bf16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Decode attention with both products on the matrix cores (G = 1, 2, 4 or 8 query heads per KV
// head: the heads are MFMA rows, 4 per k group of lanes).
// A wave takes 32 consecutive tokens per batch.  Scores: one v_mfma_f32_16x16x32_bf16 per 16
// tokens and 32 elements, A = keys (row = token; the lanes of k group g feed elements
// 32 g .. 32 g + 31 to the four MFMAs, so each loads 32 contiguous bytes of its token's row, decoded
// exactly to bf16), B = queries (column = head, zero past G, the same element order); lane l holds
// the scores of head l % 16 for tokens 4 (l / 16) + r of each 16-token half.  Those 8 scores
// per lane are already the A operand of the value sums (row = head, k slot j = token
// pi(j) = 4 (l / 16) + j for j < 4, 16 + 4 (l / 16) + j - 4 otherwise), so the probabilities x
// value factors never leave the registers; they are split into bf16 hi + lo terms (their sum
// within 2^-17 of the fp32 weight; bf16 x bf16 products are exact in fp32).  Values: the rows
// go to a per-wave LDS buffer by buffer_load ... lds and come back transposed
// (ds_read_b64_tr_b8: 8 tokens pi(j) of one element per lane), decoded exactly to bf16; two
// MFMAs per 16 elements.  The softmax is
// online in base 2 with a wave-uniform running maximum per head, reduced once per batch.  The
// batch's 32 key and 32 value factors are loaded one per lane and handed out through LDS (memory
// instructions, not bytes, set the pace here: 9 loads per lane and batch).
// SPLIT: the workgroup takes tokens [s * chunk, (s + 1) * chunk) of its sequence (workgroup id =
// (sequence x KV head) x S + s) and writes its partial result -- per head the maximum logit, the
// sum of weights and the weighted value sums -- to part[((b KVH + kv) S + s) G + g][130] for
// attn_combine_kernel; otherwise it takes the whole sequence and writes the output.
template <int FMT, int G, bool SPLIT = false>
__global__ __launch_bounds__(64 * kAttnWaves) void attn_decode_mma_kernel(
    int64_t H, int64_t KVH, int64_t T, const uint16_t* __restrict__ q,
    const uint8_t* __restrict__ k_codes, const float* __restrict__ k_si,
    const uint8_t* __restrict__ v_codes, const float* __restrict__ v_si,
    const int32_t* __restrict__ seq_lens, float score_scale, uint16_t* __restrict__ out,
    int64_t chunk = 0, int S = 1, float* __restrict__ part = nullptr) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "heads as MFMA columns / rows");
  constexpr int W = kAttnWaves;
  constexpr int KT = 32;   // tokens per batch
  __shared__ float s_acc[W][G][128];
  __shared__ float s_m[W][G], s_l[W][G];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[W][KT * 128];
  __shared__ __attribute__((aligned(16))) float s_f[W][2 * KT];   // the batch's K, V factors

  // Workgroup ids are dealt to the 8 XCDs round robin; the whole-sequence form renumbers them so
  // that each XCD takes a contiguous range (sequence-major): the KV heads of a sequence then share
  // one XCD's L2, where the token-major factor lines they all read are fetched once instead of
  // once per head (3% faster on 64 sequences; the split form measured slower with it).
  int64_t id = blockIdx.x;
  if constexpr (!SPLIT) {
    const int64_t n = gridDim.x, q8 = n / 8, r8 = n % 8;
    const int64_t xcd = blockIdx.x % 8, local = blockIdx.x / 8;
    id = xcd < r8 ? xcd * (q8 + 1) + local : r8 * (q8 + 1) + (xcd - r8) * q8 + local;
  }
  const int64_t bh = SPLIT ? id / S : id;   // sequence x KV head
  const int sp = SPLIT ? (int)(id % S) : 0;
  const int64_t b = bh / KVH, kvh = bh % KVH;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, qg = lane >> 4;   // MFMA row / column, and k group
  int64_t len = seq_lens[b];
  len = len < 0 ? 0 : (len > T ? T : len);
  // this workgroup's tokens [tbeg, len)
  const int64_t tbeg = SPLIT ? (int64_t)sp * chunk : 0;
  if constexpr (SPLIT) len = len < tbeg + chunk ? len : tbeg + chunk;

  // B operand of the scores: head col (zero past G); MFMA c takes elements 32 qg + 8 c .. + 7
  // in the lanes of k group qg (the keys use the same assignment: a contraction is free to pair
  // its terms in any order), so each lane's key pieces are 32 contiguous bytes
  bf16x8 qf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    qf[c] = bf16x8{};
    if (col < G) {
      const uint4 v = *reinterpret_cast<const uint4*>(
          q + ((b * H + kvh * G + col) * 128 + 32 * qg + 8 * c));
      qf[c] = __builtin_bit_cast(bf16x8, v);
    }
  }

  float m[G];
#pragma unroll
  for (int g = 0; g < G; ++g) m[g] = -INFINITY;
  float lsum = 0.0f;   // head col, this lane's tokens
  v4f pacc[8];         // k group qg (lanes 16 qg .. + 15): heads 4 qg .. 4 qg + 3 of element 16 cb + col
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) pacc[cb] = v4f{0.f, 0.f, 0.f, 0.f};
  const int jj = col >> 1, hh = col & 1;   // the token row this lane points at in the value reads
  const int prow = jj < 4 ? 4 * qg + jj : 16 + 4 * qg + (jj - 4);

  auto row_of = [&](int64_t t) { return (b * T + (t < len ? t : len - 1)) * KVH + kvh; };
  // value rows of this (sequence, KV head) for the LDS DMA: token t at t * KVH * 128 from the
  // first row; the bound ends after the last valid token, so rows past it read as zeros
  const uint4 vrsrc = attn_rsrc(v_codes + (b * T * KVH + kvh) * 128,
                                len > 0 ? (uint64_t)((len - 1) * KVH * 128 + 128) : 0);
  const uint32_t vlds = (uint32_t)reinterpret_cast<uintptr_t>(&s_v[w][0]);
  for (int64_t t0 = tbeg + (int64_t)w * KT; t0 < len; t0 += W * KT) {
    // value rows straight into this wave's LDS rows (token 8u + lane / 8, bytes (lane % 8) 16)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      attn_dma16(vrsrc, (uint32_t)((t0 + 8 * u + (lane >> 3)) * KVH * 128 + (lane & 7) * 16),
                 __builtin_amdgcn_readfirstlane(vlds + u * 1024));
    // then the batch's other loads: key pieces (token 16 ch + col, bytes 32 qg .. + 31) and one
    // factor per lane (lanes 0..31 the keys' of tokens 0..31, lanes 32..63 the values')
    uint4 kraw[2][2];
    const float fac = (lane < 32 ? k_si : v_si)[row_of(t0 + (lane & 31))];
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      const int64_t kr = row_of(t0 + 16 * ch + col) * 128 + 32 * qg;
      kraw[ch][0] = *reinterpret_cast<const uint4*>(k_codes + kr);
      kraw[ch][1] = *reinterpret_cast<const uint4*>(k_codes + kr + 16);
    }
    // the factors of the lane's score rows (tokens 16 ch + 4 qg + r) through LDS
    s_f[w][lane] = fac;
    float ksr[2][4], vsr[2][4];
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      const float4 kf = *reinterpret_cast<const float4*>(&s_f[w][16 * ch + 4 * qg]);
      const float4 vf4 = *reinterpret_cast<const float4*>(&s_f[w][KT + 16 * ch + 4 * qg]);
      ksr[ch][0] = kf.x; ksr[ch][1] = kf.y; ksr[ch][2] = kf.z; ksr[ch][3] = kf.w;
      vsr[ch][0] = vf4.x; vsr[ch][1] = vf4.y; vsr[ch][2] = vf4.z; vsr[ch][3] = vf4.w;
    }
    // scores of the two 16-token halves
    v4f sc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        const uint4& kp = kraw[ch][c >> 1];
        const v2i codes = (c & 1) ? v2i{(int)kp.z, (int)kp.w} : v2i{(int)kp.x, (int)kp.y};
        sc[ch] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode8_bf16<FMT>(codes), qf[c], sc[ch],
                                                         0, 0, 0);
      }
    float s[8];
    float mx = -INFINITY;
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = col < G && t0 + 16 * ch + 4 * qg + r < len;
        s[4 * ch + r] = ok ? sc[ch][r] * (ksr[ch][r] * score_scale) : -INFINITY;   // base 2
        mx = fmaxf(mx, s[4 * ch + r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // lane g holds head g's batch maximum: wave-uniform values, a scalar branch each, taken
    // only when the running maximum grows
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mg = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), g));
      if (mg > m[g]) {
        const float alpha = __builtin_amdgcn_exp2f(m[g] - mg);   // 0 when m = -inf
        if (col == g) lsum *= alpha;
        const float ap = qg == g / 4 ? alpha : 1.0f;   // head g's value sums: k group g / 4
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) pacc[cb][g % 4] *= ap;
        m[g] = mg;
      }
    }
    float mc = 0.0f;
#pragma unroll
    for (int g = 0; g < G; ++g) mc = col == g ? m[g] : mc;
    // probabilities x value factors: the A operand of the value sums, as bf16 hi + lo
    bf16x8 pa, pl;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = s[j] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s[j] - mc);
      lsum += p;
      const float pw = p * vsr[j >> 2][j & 3];
      pa[j] = (__bf16)pw;
      pl[j] = (__bf16)(pw - (float)pa[j]);
    }
    // the value rows' DMA has landed (issued before every load the scores waited for, and vector
    // memory operations complete in order; this wait makes it explicit)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint8_t* vrow = &s_v[w][prow * 128 + 8 * hh];
    bf16x8 vb[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const v2i codes = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) v2i*)(vrow + 16 * cb));
      vb[cb] = decode8_bf16<FMT>(codes);
      pacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb[cb], pacc[cb], 0, 0, 0);
    }
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
      pacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb[cb], pacc[cb], 0, 0, 0);
  }

  // denominators over the 4 k groups; k group qg holds the value sums of heads 4 qg + r, lanes
  // 0..G-1 the heads' denominators and maxima
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int g = 4 * qg + r;
    if (g < G) {
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) s_acc[w][g][16 * cb + col] = pacc[cb][r];
    }
  }
  if (lane < G) {
    float ml = 0.0f;
#pragma unroll
    for (int g = 0; g < G; ++g) ml = lane == g ? m[g] : ml;
    s_m[w][lane] = ml;
    s_l[w][lane] = lsum;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * 128; idx += 64 * W) {
    const int g = idx >> 7, d = idx & 127;
    float mxw = -INFINITY;
#pragma unroll
    for (int v = 0; v < W; ++v) mxw = fmaxf(mxw, s_m[v][g]);
    float num = 0.0f, den = 0.0f;
    if (mxw != -INFINITY) {
#pragma unroll
      for (int v = 0; v < W; ++v) {
        const float f = __builtin_amdgcn_exp2f(s_m[v][g] - mxw);   // 0 for a wave without tokens
        num = fmaf(f, s_acc[v][g][d], num);
        den = fmaf(f, s_l[v][g], den);
      }
    }
    if constexpr (SPLIT) {
      float* pp = part + ((bh * S + sp) * G + g) * 130;
      pp[2 + d] = num;
      if (d == 0) {
        pp[0] = mxw;   // -inf (and zero sums) for a workgroup without tokens
        pp[1] = den;
      }
    } else {
      const float o = den > 0.0f ? num / den : 0.0f;   // no cached token: zeros
      typedef __bf16 bf1;
      const bf1 ob = (bf1)o;
      out[(b * H + kvh * G + g) * 128 + d] = __builtin_bit_cast(uint16_t, ob);
    }
  }
}

// Merge of the S partial results of each (sequence, KV head): the same rescaling by the base-2
// maximum as the merge of a workgroup's waves.  One workgroup per (sequence, KV head), one thread
// per (head, element).
template <int G>
__global__ __launch_bounds__(128 * G) void attn_combine_kernel(int64_t H, int64_t KVH, int S,
                                                               const float* __restrict__ part,
                                                               uint16_t* __restrict__ out) {
  const int64_t bh = blockIdx.x, b = bh / KVH, kvh = bh % KVH;
  const int g = threadIdx.x >> 7, d = threadIdx.x & 127;
  const float* base = part + (bh * S * G + g) * 130;
  constexpr int kStride = G * 130;   // between the partials of consecutive splits
  float mx = -INFINITY;
  for (int sp = 0; sp < S; ++sp) mx = fmaxf(mx, base[sp * kStride]);
  float num = 0.0f, den = 0.0f;
  if (mx != -INFINITY) {
    for (int sp = 0; sp < S; ++sp) {
      const float f = __builtin_amdgcn_exp2f(base[sp * kStride] - mx);   // 0 for an empty split
      num = fmaf(f, base[sp * kStride + 2 + d], num);
      den = fmaf(f, base[sp * kStride + 1], den);
    }
  }
  const float o = den > 0.0f ? num / den : 0.0f;
  typedef __bf16 bf1;
  const bf1 ob = (bf1)o;
  out[(b * H + kvh * G + g) * 128 + d] = __builtin_bit_cast(uint16_t, ob);
}

template <int FMT>
int dispatch_attn(int G, dim3 grid, hipStream_t st, int64_t H, int64_t KVH, int64_t T,
                  const uint16_t* q, const uint8_t* kc, const float* ks, const uint8_t* vc,
                  const float* vs, const int32_t* lens, float c, uint16_t* out) {
  const dim3 block(64 * kAttnWaves);
  switch (G) {
    case 1: return launch(attn_decode_mma_kernel<FMT, 1>, grid, block, st, H, KVH, T, q, kc, ks, vc, vs, lens, c, out, (int64_t)0, 1, (float*)nullptr);
    case 2: return launch(attn_decode_mma_kernel<FMT, 2>, grid, block, st, H, KVH, T, q, kc, ks, vc, vs, lens, c, out, (int64_t)0, 1, (float*)nullptr);
    case 4: return launch(attn_decode_mma_kernel<FMT, 4>, grid, block, st, H, KVH, T, q, kc, ks, vc, vs, lens, c, out, (int64_t)0, 1, (float*)nullptr);
    case 8: return launch(attn_decode_mma_kernel<FMT, 8>, grid, block, st, H, KVH, T, q, kc, ks, vc, vs, lens, c, out, (int64_t)0, 1, (float*)nullptr);
    default: return FP8BS_ERR_UNSUPPORTED;
  }
}

// Split decode: S = ceil(T / chunk) workgroups per (sequence, KV head), then the merge.
template <int FMT, int G>
int launch_split(int64_t B, int64_t H, int64_t KVH, int64_t T, int64_t chunk, int S,
                 hipStream_t st, const uint16_t* q, const uint8_t* kc, const float* ks,
                 const uint8_t* vc, const float* vs, const int32_t* lens, float c, float* part,
                 uint16_t* out) {
  if (S > 0) {
    const int r = launch(attn_decode_mma_kernel<FMT, G, true>, dim3((unsigned)(B * KVH * S)),
                         dim3(64 * kAttnWaves), st, H, KVH, T, q, kc, ks, vc, vs, lens, c, out,
                         chunk, S, part);
    if (r != FP8BS_OK) return r;
  }
  return launch(attn_combine_kernel<G>, dim3((unsigned)(B * KVH)), dim3(128 * G), st, H, KVH, S,
                (const float*)part, out);
}

template <int FMT>
int dispatch_split(int G, int64_t B, int64_t H, int64_t KVH, int64_t T, int64_t chunk, int S,
                   hipStream_t st, const uint16_t* q, const uint8_t* kc, const float* ks,
                   const uint8_t* vc, const float* vs, const int32_t* lens, float c, float* part,
                   uint16_t* out) {
  switch (G) {
    case 1: return launch_split<FMT, 1>(B, H, KVH, T, chunk, S, st, q, kc, ks, vc, vs, lens, c, part, out);
    case 2: return launch_split<FMT, 2>(B, H, KVH, T, chunk, S, st, q, kc, ks, vc, vs, lens, c, part, out);
    case 4: return launch_split<FMT, 4>(B, H, KVH, T, chunk, S, st, q, kc, ks, vc, vs, lens, c, part, out);
    case 8: return launch_split<FMT, 8>(B, H, KVH, T, chunk, S, st, q, kc, ks, vc, vs, lens, c, part, out);
    default: return FP8BS_ERR_UNSUPPORTED;
  }
}

// The matrix-core decode addresses a (sequence, KV head)'s value rows with 32-bit offsets.
bool mma_offsets_ok(int64_t T, int64_t KVH) { return (T + 32) * KVH * 128 <= 0xFFFFFFFFll; }

bool cache_sizes_ok(int64_t B, int64_t T, int64_t KVH) {
  // B * T * KVH * 128 bytes must be addressable with 64-bit offsets
  if (B < 0 || T < 0 || KVH < 0) return false;
  if (B == 0 || T == 0 || KVH == 0) return true;
  const int64_t lim = INT64_MAX / 256;
  return T <= lim / B && KVH <= lim / (B * T);
}

}  // namespace
}  // namespace fp8bs

using namespace fp8bs;

extern "C" int fp8_kv_cache_append(int64_t B, int64_t KVH, int64_t T, const void* k_new_bf16,
                                   const void* v_new_bf16, const int32_t* positions, int fmt,
                                   int mode, void* k_codes, float* k_scale_inv, void* v_codes,
                                   float* v_scale_inv, void* stream) {
  if (!fmt_ok(fmt) || (mode != FP8BS_SCALE_FP32 && mode != FP8BS_SCALE_POW2)) return FP8BS_ERR_ARG;
  if (!cache_sizes_ok(B, T, KVH)) return FP8BS_ERR_SHAPE;
  if (B == 0 || KVH == 0 || T == 0) return FP8BS_OK;
  if (B > 65535 || ceil_div(2 * KVH, kAppendThreads / 8) > 0x7FFFFFFF) return FP8BS_ERR_SHAPE;
  if (!k_new_bf16 || !v_new_bf16 || !positions || !k_codes || !k_scale_inv || !v_codes ||
      !v_scale_inv)
    return FP8BS_ERR_NULL;
  if (!aligned16(k_new_bf16) || !aligned16(v_new_bf16) || !aligned16(k_codes) ||
      !aligned16(v_codes) || !aligned4(k_scale_inv) || !aligned4(v_scale_inv) ||
      !aligned4(positions))
    return FP8BS_ERR_ALIGN;
  const dim3 grid((unsigned)ceil_div(2 * KVH, kAppendThreads / 8), (unsigned)B);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint16_t* kn = static_cast<const uint16_t*>(k_new_bf16);
  const uint16_t* vn = static_cast<const uint16_t*>(v_new_bf16);
  uint8_t* kc = static_cast<uint8_t*>(k_codes);
  uint8_t* vc = static_cast<uint8_t*>(v_codes);
  const dim3 block(kAppendThreads);
  const bool pow2 = mode == FP8BS_SCALE_POW2;
  if (fmt == FP8BS_E4M3)
    return pow2 ? launch(kv_append_kernel<FP8BS_E4M3, true>, grid, block, st, B, KVH, T, kn, vn, positions, kc, k_scale_inv, vc, v_scale_inv)
                : launch(kv_append_kernel<FP8BS_E4M3, false>, grid, block, st, B, KVH, T, kn, vn, positions, kc, k_scale_inv, vc, v_scale_inv);
  return pow2 ? launch(kv_append_kernel<FP8BS_E5M2, true>, grid, block, st, B, KVH, T, kn, vn, positions, kc, k_scale_inv, vc, v_scale_inv)
              : launch(kv_append_kernel<FP8BS_E5M2, false>, grid, block, st, B, KVH, T, kn, vn, positions, kc, k_scale_inv, vc, v_scale_inv);
}

extern "C" int fp8_attention_decode(int64_t B, int64_t H, int64_t KVH, int64_t T,
                                    const void* q_bf16, const void* k_codes,
                                    const float* k_scale_inv, const void* v_codes,
                                    const float* v_scale_inv, const int32_t* seq_lens,
                                    float sm_scale, int fmt, void* out_bf16, void* stream) {
  if (!fmt_ok(fmt)) return FP8BS_ERR_ARG;
  if (H < 0 || !cache_sizes_ok(B, T, KVH)) return FP8BS_ERR_SHAPE;
  if (B == 0 || H == 0) return FP8BS_OK;
  if (KVH == 0 || H % KVH != 0) return FP8BS_ERR_SHAPE;
  const int64_t G = H / KVH;
  if (G != 1 && G != 2 && G != 4 && G != 8) return FP8BS_ERR_UNSUPPORTED;
  if (!mma_offsets_ok(T, KVH)) return FP8BS_ERR_UNSUPPORTED;
  if (B * KVH > 0x7FFFFFFF || B > INT64_MAX / 256 / H) return FP8BS_ERR_SHAPE;
  if (!isfinite(sm_scale)) return FP8BS_ERR_ARG;
  if (!q_bf16 || !seq_lens || !out_bf16 ||
      (T > 0 && (!k_codes || !k_scale_inv || !v_codes || !v_scale_inv)))
    return FP8BS_ERR_NULL;
  if (!aligned16(q_bf16) || (T > 0 && (!aligned16(k_codes) || !aligned16(v_codes) ||
                                       !aligned4(k_scale_inv) || !aligned4(v_scale_inv))) ||
      !aligned4(seq_lens) || !aligned4(out_bf16))
    return FP8BS_ERR_ALIGN;
  const float c = sm_scale * 1.4426950408889634f;   // scores in base 2 (exp2 in the kernel)
  const dim3 grid((unsigned)(B * KVH));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint16_t* q = static_cast<const uint16_t*>(q_bf16);
  const uint8_t* kc = static_cast<const uint8_t*>(k_codes);
  const uint8_t* vc = static_cast<const uint8_t*>(v_codes);
  uint16_t* out = static_cast<uint16_t*>(out_bf16);
  if (fmt == FP8BS_E4M3)
    return dispatch_attn<FP8BS_E4M3>((int)G, grid, st, H, KVH, T, q, kc, k_scale_inv, vc,
                                     v_scale_inv, seq_lens, c, out);
  return dispatch_attn<FP8BS_E5M2>((int)G, grid, st, H, KVH, T, q, kc, k_scale_inv, vc,
                                   v_scale_inv, seq_lens, c, out);
}

extern "C" size_t fp8_attention_decode_workspace_size(int64_t B, int64_t H, int64_t KVH,
                                                      int64_t T, int64_t chunk) {
  if (B <= 0 || H <= 0 || KVH <= 0 || T <= 0 || chunk <= 0 || H % KVH != 0) return 0;
  if (!cache_sizes_ok(B, T, KVH)) return 0;
  const int64_t S = ceil_div(T, chunk), G = H / KVH;
  if (B * KVH > INT64_MAX / 4 / 130 / G / S) return 0;
  return (size_t)(B * KVH * S * G * 130 * 4);
}

extern "C" int fp8_attention_decode_split(int64_t B, int64_t H, int64_t KVH, int64_t T,
                                          const void* q_bf16, const void* k_codes,
                                          const float* k_scale_inv, const void* v_codes,
                                          const float* v_scale_inv, const int32_t* seq_lens,
                                          float sm_scale, int fmt, int64_t chunk,
                                          void* workspace, size_t workspace_bytes,
                                          void* out_bf16, void* stream) {
  if (!fmt_ok(fmt)) return FP8BS_ERR_ARG;
  if (H < 0 || !cache_sizes_ok(B, T, KVH)) return FP8BS_ERR_SHAPE;
  if (chunk <= 0 || chunk % 32 != 0) return FP8BS_ERR_SHAPE;
  if (B == 0 || H == 0) return FP8BS_OK;
  if (KVH == 0 || H % KVH != 0) return FP8BS_ERR_SHAPE;
  const int64_t G = H / KVH;
  if (G != 1 && G != 2 && G != 4 && G != 8) return FP8BS_ERR_UNSUPPORTED;
  if (!mma_offsets_ok(T, KVH)) return FP8BS_ERR_UNSUPPORTED;
  const int64_t S = ceil_div(T, chunk);
  if (B * KVH > 0x7FFFFFFF || S > 0x7FFFFFFF / (B * KVH) || B > INT64_MAX / 256 / H)
    return FP8BS_ERR_SHAPE;
  if (!isfinite(sm_scale)) return FP8BS_ERR_ARG;
  const size_t need = T > 0 ? fp8_attention_decode_workspace_size(B, H, KVH, T, chunk) : 0;
  if (T > 0 && need == 0) return FP8BS_ERR_SHAPE;
  if (!q_bf16 || !seq_lens || !out_bf16 ||
      (T > 0 && (!k_codes || !k_scale_inv || !v_codes || !v_scale_inv || !workspace)))
    return FP8BS_ERR_NULL;
  if (workspace_bytes < need) return FP8BS_ERR_SHAPE;
  if (!aligned16(q_bf16) || (T > 0 && (!aligned16(k_codes) || !aligned16(v_codes) ||
                                       !aligned4(k_scale_inv) || !aligned4(v_scale_inv) ||
                                       !aligned4(workspace))) ||
      !aligned4(seq_lens) || !aligned4(out_bf16))
    return FP8BS_ERR_ALIGN;
  const float c = sm_scale * 1.4426950408889634f;   // scores in base 2 (exp2 in the kernel)
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint16_t* q = static_cast<const uint16_t*>(q_bf16);
  const uint8_t* kc = static_cast<const uint8_t*>(k_codes);
  const uint8_t* vc = static_cast<const uint8_t*>(v_codes);
  float* part = static_cast<float*>(workspace);
  uint16_t* out = static_cast<uint16_t*>(out_bf16);
  if (fmt == FP8BS_E4M3)
    return dispatch_split<FP8BS_E4M3>((int)G, B, H, KVH, T, chunk, (int)S, st, q, kc, k_scale_inv,
                                      vc, v_scale_inv, seq_lens, c, part, out);
  return dispatch_split<FP8BS_E5M2>((int)G, B, H, KVH, T, chunk, (int)S, st, q, kc, k_scale_inv,
                                    vc, v_scale_inv, seq_lens, c, part, out);
}
