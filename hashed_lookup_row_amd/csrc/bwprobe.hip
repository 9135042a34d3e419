// Streaming kernels that measure what this GPU's HBM gives plain traffic: a
// read-only sweep, a write-only sweep and a copy, each with ordinary or
// non-temporal accesses.  They are the measured ceiling the row kernels of
// libhlr are compared with; they compute nothing of the embedding cache and
// are built into their own library (libhlr_bwprobe.so), loaded only by the
// benchmark's ceiling mode.
//
// Every kernel moves 16-byte units.  Block b of a one-shot launch covers
// units [b*256*U, (b+1)*256*U): thread t takes units t, t+256, ... so each
// wave access is 1 KiB contiguous, and all U loads of a thread are issued
// before the first is used.  A read sweep folds what it loads into one word
// per thread (XOR of the bits), stored so the loads cannot be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kU = 8;

typedef float f4v __attribute__((ext_vector_type(4)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u4v ld(const u4v *p) {
  if (NT) return __builtin_nontemporal_load(p);
  return *p;
}

template <bool NT>
__device__ __forceinline__ void st(u4v *p, u4v v) {
  if (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

template <bool NT>
__global__ void __launch_bounds__(kThreads) read_kernel(const u4v *__restrict__ src, int64_t n4,
                                                        uint32_t *__restrict__ sink) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (kThreads * kU) + threadIdx.x;
  u4v v[kU];
#pragma unroll
  for (int k = 0; k < kU; ++k) {
    const int64_t i = base + k * kThreads;
    v[k] = ld<NT>(src + (i < n4 ? i : 0));
  }
  uint32_t x = 0;
#pragma unroll
  for (int k = 0; k < kU; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  sink[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = x;
}

template <bool NT>
__global__ void __launch_bounds__(kThreads) write_kernel(u4v *__restrict__ dst, int64_t n4, uint32_t val) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (kThreads * kU) + threadIdx.x;
  const u4v v = {val, val ^ 1u, val ^ 2u, val ^ 3u};
#pragma unroll
  for (int k = 0; k < kU; ++k) {
    const int64_t i = base + k * kThreads;
    if (i < n4) st<NT>(dst + i, v);
  }
}

template <bool NT>
__global__ void __launch_bounds__(kThreads) copy_kernel(const u4v *__restrict__ src, u4v *__restrict__ dst,
                                                        int64_t n4) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (kThreads * kU) + threadIdx.x;
  u4v v[kU];
#pragma unroll
  for (int k = 0; k < kU; ++k) {
    const int64_t i = base + k * kThreads;
    v[k] = ld<NT>(src + (i < n4 ? i : 0));
  }
#pragma unroll
  for (int k = 0; k < kU; ++k) {
    const int64_t i = base + k * kThreads;
    if (i < n4) st<NT>(dst + i, v[k]);
  }
}

}  // namespace

// kind: 0 read, 1 write, 2 copy; nt: non-temporal accesses.  bytes % 16 == 0,
// src/dst 16-byte aligned; sink holds one uint32 per thread of the read grid
// (hlr_bwprobe_sink_words(bytes)).  Returns 0, or 1 on a bad argument, 2 on a
// launch error.
extern "C" int64_t hlr_bwprobe_sink_words(int64_t bytes) {
  const int64_t n4 = bytes / 16;
  const int64_t grid = (n4 + kThreads * kU - 1) / (kThreads * kU);
  return grid * kThreads;
}

extern "C" int hlr_bwprobe(int kind, int nt, const void *src, void *dst, int64_t bytes, uint32_t *sink,
                           hipStream_t stream) {
  if (bytes <= 0 || bytes % 16 != 0) return 1;
  if ((kind == 0 || kind == 2) && (!src || reinterpret_cast<uintptr_t>(src) % 16)) return 1;
  if ((kind == 1 || kind == 2) && (!dst || reinterpret_cast<uintptr_t>(dst) % 16)) return 1;
  if (kind == 0 && !sink) return 1;
  const int64_t n4 = bytes / 16;
  const int64_t g = (n4 + kThreads * kU - 1) / (kThreads * kU);
  if (g > 0x7fffffff) return 1;
  const int grid = static_cast<int>(g);
  const u4v *s = static_cast<const u4v *>(src);
  u4v *d = static_cast<u4v *>(dst);
  switch (kind * 2 + (nt ? 1 : 0)) {
    case 0: read_kernel<false><<<grid, kThreads, 0, stream>>>(s, n4, sink); break;
    case 1: read_kernel<true><<<grid, kThreads, 0, stream>>>(s, n4, sink); break;
    case 2: write_kernel<false><<<grid, kThreads, 0, stream>>>(d, n4, 0x3f800000u); break;
    case 3: write_kernel<true><<<grid, kThreads, 0, stream>>>(d, n4, 0x3f800000u); break;
    case 4: copy_kernel<false><<<grid, kThreads, 0, stream>>>(s, d, n4); break;
    case 5: copy_kernel<true><<<grid, kThreads, 0, stream>>>(s, d, n4); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
