// Row gather (the model reads the cached row M[i]: "Memory Layer: Train the
// In-Model Cache for Recommendation Models", sec. 2; a miss reads the zero
// vector) and the hashing-trick row map of hashed tables ("DLRMv4: MLPerf
// recommendation training goes sequential", feature expansion paragraph).
//
// The gather is a pure HBM copy: out[i] = table[rows[i]].  Work is a flat list
// of 16-byte units (position, column); consecutive lanes take consecutive
// columns of one row, so every wave load is a 1 KiB contiguous piece of a
// row.  Each lane keeps UNROLL independent loads in flight before it stores;
// output rows are streamed with non-temporal stores so the table's hot rows
// stay in L2/MALL.  No LDS staging: the data has no reuse inside a block.
#include "hlr_common.hpp"
#include "step_parts.hpp"

namespace {
using namespace hlr;

constexpr int kThreads = 256;
// Loads in flight per lane.  Two: the gather alone is as fast with two as
// with four (81-83 us for 131,072 rows of 2 KiB), and the hashed-tables step,
// whose gathers run beside the next group's plan kernels, is faster
// (1.756-1.767 ms against 1.795-1.810 with four and 1.808-1.811 with one).
constexpr int kUnroll = 2;

// fresh (nullable): positions with fresh[i] == 0 read the zero vector too (a
// row inserted by this batch's lookup whose storage has not been cleared).
template <int V4>
__global__ void __launch_bounds__(kThreads)
    gather_kernel(const float4 *__restrict__ table, int64_t num_rows, const int64_t *__restrict__ rows,
                  const int8_t *__restrict__ fresh, int64_t n, float4 *__restrict__ out, int64_t v4_rt) {
  const int64_t v4 = V4 > 0 ? V4 : v4_rt;
  const int64_t total = n * v4;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (kThreads * kUnroll) + threadIdx.x;
  float4 val[kUnroll];
  int64_t src[kUnroll];
#pragma unroll
  for (int k = 0; k < kUnroll; ++k) {
    const int64_t u = base + k * kThreads;
    src[k] = -1;
    if (u < total) {
      const int64_t i = u / v4;
      const int64_t r = rows[i];
      if (r >= 0 && r < num_rows && (fresh == nullptr || fresh[i] != 0)) src[k] = r * v4 + (u - i * v4);
    }
  }
#pragma unroll
  for (int k = 0; k < kUnroll; ++k) val[k] = src[k] >= 0 ? table[src[k]] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < kUnroll; ++k) {
    const int64_t u = base + k * kThreads;
    if (u < total) store_nt(out + u, val[k]);
  }
}

__global__ void __launch_bounds__(kThreads)
    hashed_rows_kernel(const int64_t *__restrict__ ids, int64_t n, uint64_t num_rows, int64_t *__restrict__ rows) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i < n) rows[i] = static_cast<int64_t>(mix64(static_cast<uint64_t>(ids[i])) % num_rows);
}

}  // namespace

namespace {

hlr_status gather_launch(const float *table, int64_t num_rows, int64_t dim, const int64_t *rows, const int8_t *fresh,
                         int64_t n, float *out, hipStream_t stream) {
  if (n < 0 || n > kMaxN || num_rows < 0) return HLR_INVALID_ARG;
  if (dim <= 0 || dim % 4 != 0) return HLR_UNSUPPORTED_DIM;
  if (n == 0) return HLR_OK;
  if (!rows || !out || (num_rows > 0 && !table)) return HLR_INVALID_ARG;
  if ((table && !aligned(table, 16)) || !aligned(out, 16) || !aligned(rows, 8)) return HLR_MISALIGNED;
  const int64_t v4 = dim / 4;
  const int grid = grid_for(n * v4, kThreads * kUnroll);
  const float4 *t4 = reinterpret_cast<const float4 *>(table);
  float4 *o4 = reinterpret_cast<float4 *>(out);
  switch (v4) {
    case 16: gather_kernel<16><<<grid, kThreads, 0, stream>>>(t4, num_rows, rows, fresh, n, o4, v4); break;
    case 32: gather_kernel<32><<<grid, kThreads, 0, stream>>>(t4, num_rows, rows, fresh, n, o4, v4); break;
    case 64: gather_kernel<64><<<grid, kThreads, 0, stream>>>(t4, num_rows, rows, fresh, n, o4, v4); break;
    case 128: gather_kernel<128><<<grid, kThreads, 0, stream>>>(t4, num_rows, rows, fresh, n, o4, v4); break;
    default: gather_kernel<0><<<grid, kThreads, 0, stream>>>(t4, num_rows, rows, fresh, n, o4, v4); break;
  }
  return launch_status();
}

}  // namespace

extern "C" hlr_status gather_rows(const float *table, int64_t num_rows, int64_t dim, const int64_t *rows, int64_t n,
                                  float *out, hipStream_t stream) {
  return gather_launch(table, num_rows, dim, rows, nullptr, n, out, stream);
}

hlr_status hlr::gather_rows_fresh(const float *table, int64_t num_rows, int64_t dim, const int64_t *rows,
                                  const int8_t *hit, int64_t n, float *out, hipStream_t stream) {
  if (n > 0 && !hit) return HLR_INVALID_ARG;
  return gather_launch(table, num_rows, dim, rows, hit, n, out, stream);
}

extern "C" hlr_status hashed_rows(const int64_t *ids, int64_t n, int64_t num_rows, int64_t *out_rows,
                                  hipStream_t stream) {
  if (n < 0 || n > kMaxN || num_rows < 1) return HLR_INVALID_ARG;
  if (n == 0) return HLR_OK;
  if (!ids || !out_rows) return HLR_INVALID_ARG;
  if (!aligned(ids, 8) || !aligned(out_rows, 8)) return HLR_MISALIGNED;
  hashed_rows_kernel<<<grid_for(n, kThreads), kThreads, 0, stream>>>(ids, n, static_cast<uint64_t>(num_rows),
                                                                     out_rows);
  return launch_status();
}
