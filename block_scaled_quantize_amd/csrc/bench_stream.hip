// Streaming kernels with the quantizers' HBM traffic (2 bytes read and 1 byte written per
// element, no arithmetic beyond taking one byte of each input), used by the benchmark to measure
// the rate this GPU streams that mix at -- the practical ceiling the HBM-bound quantizers are
// compared with.  Not part of the C ABI of the library (built as libfp8bs_bench.so).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

// The high byte of each of the 16 bf16 values in 8 dwords.
__device__ __forceinline__ uint4 high_bytes(uint4 a, uint4 b) {
  auto pack = [](uint32_t lo, uint32_t hi) {
    return __builtin_amdgcn_perm(hi, lo, 0x07050301u);   // bytes 1, 3 of lo, then of hi
  };
  return make_uint4(pack(a.x, a.y), pack(a.z, a.w), pack(b.x, b.y), pack(b.z, b.w));
}

// One-shot grid: each lane moves one 16-element chunk (the 1x128 quantizer's shape: 8 lanes per
// 128-element row block, 32 row blocks per workgroup).
__global__ __launch_bounds__(kThreads) void stream_oneshot_kernel(const uint4* __restrict__ x,
                                                                  int64_t chunks,
                                                                  uint4* __restrict__ y) {
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c >= chunks) return;
  const uint4 a = x[2 * c], b = x[2 * c + 1];
  y[c] = high_bytes(a, b);
}

// One-shot grid with PER chunks per lane, the loads of all chunks issued before any store.
template <int PER>
__global__ __launch_bounds__(kThreads) void stream_multi_kernel(const uint4* __restrict__ x,
                                                                int64_t chunks,
                                                                uint4* __restrict__ y) {
  const int64_t c0 = (int64_t)blockIdx.x * kThreads * PER + threadIdx.x;
  uint4 a[PER], b[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t c = c0 + (int64_t)i * kThreads;
    if (c < chunks) {
      a[i] = x[2 * c];
      b[i] = x[2 * c + 1];
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t c = c0 + (int64_t)i * kThreads;
    if (c < chunks) y[c] = high_bytes(a[i], b[i]);
  }
}

// One-shot grid with non-temporal loads (NTL) and / or stores (NTS).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <bool NTL, bool NTS>
__global__ __launch_bounds__(kThreads) void stream_nt_kernel(const uint4* __restrict__ x,
                                                             int64_t chunks,
                                                             uint4* __restrict__ y) {
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c >= chunks) return;
  uint4 a, b;
  if constexpr (NTL) {
    const u32x4 va = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + 2 * c));
    const u32x4 vb = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + 2 * c + 1));
    a = make_uint4(va.x, va.y, va.z, va.w);
    b = make_uint4(vb.x, vb.y, vb.z, vb.w);
  } else {
    a = x[2 * c];
    b = x[2 * c + 1];
  }
  const uint4 v = high_bytes(a, b);
  if constexpr (NTS) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(y + c));
  } else {
    y[c] = v;
  }
}

// The short-row quantizer's geometry on rows of 4096 elements: a workgroup takes 32 rows x 128
// columns, 8 lanes per 256-byte row segment (rows 8 KiB apart).
__global__ __launch_bounds__(kThreads) void stream_tile_kernel(const uint4* __restrict__ x,
                                                               int64_t chunks,
                                                               uint4* __restrict__ y) {
  constexpr int64_t kRowChunks = 4096 / 16;
  const int t = threadIdx.x;
  const int64_t rb = blockIdx.x / 32, cb = blockIdx.x % 32;
  const int64_t c = (rb * 32 + (t >> 3)) * kRowChunks + cb * 8 + (t & 7);
  if (c >= chunks) return;
  y[c] = high_bytes(x[2 * c], x[2 * c + 1]);
}

// Persistent grid (a fixed number of workgroups per CU) striding over the chunks.
__global__ __launch_bounds__(kThreads) void stream_stride_kernel(const uint4* __restrict__ x,
                                                                 int64_t chunks,
                                                                 uint4* __restrict__ y) {
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < chunks;
       c += (int64_t)gridDim.x * kThreads)
    y[c] = high_bytes(x[2 * c], x[2 * c + 1]);
}

}  // namespace

// variant 0: one-shot, 1 chunk per lane; 1: one-shot, 2 chunks; 2: one-shot, 4 chunks;
// 3: 2048 workgroups striding; 4: 4096 workgroups striding; 5, 6, 7: one-shot with
// non-temporal loads, stores, both; 8: 32-row tiles of rows of 4096 elements (n a multiple of
// 32 * 4096).  n must be a multiple of 16 and both pointers 16-byte aligned.  Returns 0, or -1
// for invalid arguments / a failed launch.
extern "C" int fp8bs_bench_stream(const void* x_bf16, int64_t n, void* y, int variant,
                                  void* stream) {
  if (!x_bf16 || !y || n <= 0 || n % 16 || (reinterpret_cast<uintptr_t>(x_bf16) & 15) ||
      (reinterpret_cast<uintptr_t>(y) & 15))
    return -1;
  const int64_t chunks = n / 16;
  const uint4* xi = static_cast<const uint4*>(x_bf16);
  uint4* yo = static_cast<uint4*>(y);
  hipStream_t st = static_cast<hipStream_t>(stream);
  auto grid_for = [&](int per) { return dim3((unsigned)((chunks + kThreads * per - 1) / (kThreads * per))); };
  switch (variant) {
    case 0: stream_oneshot_kernel<<<grid_for(1), kThreads, 0, st>>>(xi, chunks, yo); break;
    case 1: stream_multi_kernel<2><<<grid_for(2), kThreads, 0, st>>>(xi, chunks, yo); break;
    case 2: stream_multi_kernel<4><<<grid_for(4), kThreads, 0, st>>>(xi, chunks, yo); break;
    case 3: stream_stride_kernel<<<2048, kThreads, 0, st>>>(xi, chunks, yo); break;
    case 4: stream_stride_kernel<<<4096, kThreads, 0, st>>>(xi, chunks, yo); break;
    case 5: stream_nt_kernel<true, false><<<grid_for(1), kThreads, 0, st>>>(xi, chunks, yo); break;
    case 6: stream_nt_kernel<false, true><<<grid_for(1), kThreads, 0, st>>>(xi, chunks, yo); break;
    case 7: stream_nt_kernel<true, true><<<grid_for(1), kThreads, 0, st>>>(xi, chunks, yo); break;
    case 8:
      if (n % (32 * 4096)) return -1;
      stream_tile_kernel<<<dim3((unsigned)(n / 4096)), kThreads, 0, st>>>(xi, chunks, yo);
      break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
