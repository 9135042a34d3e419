// Shared device and host helpers of libhlr (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "hlr.h"

#pragma clang fp contract(off)

namespace hlr {

constexpr int kWave = 64;

// SplitMix64 finaliser (variant-13 shift/multiply constants): the bucket hash of
// the MPZCH identity tensor and of the hashed tables.
__host__ __device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ int readlane_i32(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

__device__ __forceinline__ int64_t readlane_i64(int64_t v, int lane) {
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint64_t>(v) & 0xffffffffu), lane);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint64_t>(v) >> 32), lane);
  return static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                              static_cast<uint32_t>(lo));
}

// Wave-aggregated add of a per-lane predicate count to a device counter.
__device__ __forceinline__ void wave_count(unsigned long long *ctr, bool pred) {
  const uint64_t m = ballot(pred);
  if (m != 0 && lane_id() == __builtin_ctzll(__ballot(true))) atomicAdd(ctr, (unsigned long long)__popcll(m));
}

__device__ __forceinline__ int64_t atomic_cas_i64(int64_t *p, int64_t expect, int64_t val) {
  return static_cast<int64_t>(atomicCAS(reinterpret_cast<unsigned long long *>(p),
                                        static_cast<unsigned long long>(expect),
                                        static_cast<unsigned long long>(val)));
}

__device__ __forceinline__ float4 f4_sub(float4 a, float4 b) {
  return make_float4(a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w);
}

typedef float f4v __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte store.
__device__ __forceinline__ void store_nt(float4 *p, float4 v) {
  const f4v x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<f4v *>(p));
}

// ---------------------------------------------------------------- host side
inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline uint64_t next_pow2(uint64_t x) {
  uint64_t p = 1;
  while (p < x) p <<= 1;
  return p;
}

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Carves sub-buffers out of a caller workspace (256-byte aligned pieces).
struct Carver {
  char *base;
  size_t off = 0;
  explicit Carver(void *b) : base(static_cast<char *>(b)) {}
  template <typename T>
  T *take(size_t count) {
    T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
    off += round_up(count * sizeof(T), 256);
    return p;
  }
};

inline hlr_status launch_status() {
  return hipGetLastError() == hipSuccess ? HLR_OK : HLR_HIP_ERROR;
}

constexpr int64_t kMaxN = (int64_t(1) << 31) - 1;

inline int grid_for(int64_t work, int per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

}  // namespace hlr

namespace {
// Fill kernel (used instead of hipMemsetAsync so the stream may be captured in a graph).
template <typename T>
__global__ void __launch_bounds__(256) hlr_fill_kernel(T *p, int64_t n, T v) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += 256ll * gridDim.x) p[i] = v;
}

template <typename T>
inline void hlr_fill(T *p, int64_t n, T v, hipStream_t s) {
  if (n <= 0) return;
  int g = hlr::grid_for(n, 256 * 4);
  if (g > 4096) g = 4096;
  hlr_fill_kernel<T><<<g, 256, 0, s>>>(p, n, v);
}
}  // namespace
