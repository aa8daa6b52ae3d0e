// Sustained FP8 matrix-core rate on register operands: every wave of a 512-thread workgroup (two
// per SIMD, as in the GEMM tiles) repeats independent E4M3 x E4M3 MFMAs on operands loaded once
// from a small code array, with no memory traffic inside the loop.  The rate this reaches with a
// workload's own code distribution is the practical ceiling of that workload's GEMMs: the matrix
// core's power draw depends on the operand bits, and the shader clock drops below its peak when
// the codes are dense random values.  Not part of the C ABI of the library (built into
// libfp8bs_bench.so).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;

// Operands: 8 sets of 64 lanes x 32 bytes (4 A-side, 4 B-side), read once per wave.  Each loop
// step issues 32 MFMAs of 16x16x128 (or 16 of 32x32x64: the same multiply-adds) cycling over
// the four B sets, so that consecutive MFMAs see different bits.
template <int SHAPE>
__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(const v8i* __restrict__ codes,
                                                            float* __restrict__ out, int steps) {
  const int l = threadIdx.x & 63;
  v8i a[4], b[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    a[q] = codes[q * 64 + l];
    b[q] = codes[(4 + q) * 64 + l];
  }
  float s = 0.f;
  if constexpr (SHAPE == 0) {
    v4f acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < steps; ++it) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int q = 0; q < 8; ++q)
          acc[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[q & 3], b[(q + r) & 3], acc[q],
                                                                   0, 0, 0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) s += acc[q][0] + acc[q][1] + acc[q][2] + acc[q][3];
  } else {
    v16f acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[q][e] = 0.f;
    for (int it = 0; it < steps; ++it) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[q & 3], b[(q + r) & 3], acc[q],
                                                                  0, 0, 0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[q][e];
  }
  out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

// shape 0: V_MFMA 16x16x128 FP8, 1: 32x32x64 FP8.  codes: 16384 bytes (E4M3 codes), 16-byte
// aligned; out: blocks * 512 floats.  Each workgroup also takes lds_bytes of (unused) LDS, so that
// one workgroup per CU can be forced.  Multiply-adds per launch: blocks * 8 waves * steps *
// 32 * 16 * 16 * 128.  Returns 0, or -1 for invalid arguments / a failed launch.
extern "C" int fp8bs_bench_mfma(const void* codes, float* out, int shape, int steps, int blocks,
                                int lds_bytes, void* stream) {
  if (!codes || !out || (reinterpret_cast<uintptr_t>(codes) & 15) || steps <= 0 || blocks <= 0 ||
      lds_bytes < 0 || lds_bytes > 160 * 1024 || (shape != 0 && shape != 1))
    return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const v8i* c = static_cast<const v8i*>(codes);
  if (shape == 0) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&mfma_loop_kernel<0>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes) != hipSuccess)
      return -1;
    mfma_loop_kernel<0><<<blocks, kThreads, lds_bytes, st>>>(c, out, steps);
  } else {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&mfma_loop_kernel<1>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes) != hipSuccess)
      return -1;
    mfma_loop_kernel<1><<<blocks, kThreads, lds_bytes, st>>>(c, out, steps);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
