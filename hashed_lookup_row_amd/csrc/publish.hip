// Bookkeeping for publishing written rows (Raw Embedding Streaming in
// "Memory Layer: Train the In-Model Cache for Recommendation Models", sec. 2:
// rows written by training are deduplicated, quantised and pushed to serving
// at intervals).  Between two publishes the rows written by every batch are
// collected once each in a list, through a per-row flag.
//   mark_rows:  appends each row not yet flagged to the list (wave-aggregated
//               counter updates: one global atomic per wave, not per row)
//   clear_marks: unflags the listed rows and empties the list
#include "hlr_common.hpp"

namespace {
using namespace hlr;

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads)
    mark_kernel(const int64_t *__restrict__ rows, int64_t n, const int64_t *__restrict__ count, int64_t num_rows,
                uint32_t *flags, int64_t *list, unsigned long long *list_count) {
  int64_t m = n;
  if (count) {
    const int64_t c = *count;
    m = c < 0 ? 0 : (c < n ? c : n);
  }
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  bool fresh = false;
  int64_t r = -1;
  if (i < m) {
    r = rows[i];
    if (r >= 0 && r < num_rows) fresh = atomicOr(&flags[r], 1u) == 0u;
  }
  const uint64_t bal = ballot(fresh);
  if (bal == 0) return;
  const int leader = __builtin_ctzll(bal);
  unsigned long long base = 0;
  if (lane_id() == leader) base = atomicAdd(list_count, static_cast<unsigned long long>(__popcll(bal)));
  base = __shfl(base, leader);
  if (fresh) list[base + static_cast<unsigned long long>(__popcll(bal & lanemask_lt()))] = r;
}

__global__ void __launch_bounds__(kThreads)
    clear_kernel(const int64_t *__restrict__ list, const int64_t *__restrict__ list_count, int64_t cap,
                 uint32_t *flags) {
  int64_t m = *list_count;
  m = m < cap ? m : cap;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < m; i += stride) {
    const int64_t r = list[i];
    if (r >= 0 && r < cap) flags[r] = 0u;
  }
}

}  // namespace

extern "C" hlr_status mark_rows(const int64_t *rows, int64_t n, const int64_t *count, int64_t num_rows,
                                uint32_t *flags, int64_t *list, int64_t *list_count, hipStream_t stream) {
  if (n < 0 || n > kMaxN || num_rows < 0) return HLR_INVALID_ARG;
  if (n == 0 || num_rows == 0) return HLR_OK;
  if (!rows || !flags || !list || !list_count) return HLR_INVALID_ARG;
  if (!aligned(rows, 8) || !aligned(flags, 4) || !aligned(list, 8) || !aligned(list_count, 8) ||
      (count && !aligned(count, 8)))
    return HLR_MISALIGNED;
  mark_kernel<<<grid_for(n, kThreads), kThreads, 0, stream>>>(rows, n, count, num_rows, flags, list,
                                                              reinterpret_cast<unsigned long long *>(list_count));
  return launch_status();
}

extern "C" hlr_status clear_marks(const int64_t *list, int64_t *list_count, int64_t num_rows, uint32_t *flags,
                                  hipStream_t stream) {
  if (num_rows < 0) return HLR_INVALID_ARG;
  if (!list_count || (num_rows > 0 && (!list || !flags))) return HLR_INVALID_ARG;
  if ((list && !aligned(list, 8)) || !aligned(list_count, 8) || (flags && !aligned(flags, 4))) return HLR_MISALIGNED;
  if (num_rows > 0) {
    int g = grid_for(num_rows, kThreads * 8);
    if (g > 1024) g = 1024;
    clear_kernel<<<g, kThreads, 0, stream>>>(list, list_count, num_rows, flags);
  }
  hlr_fill(list_count, 1, int64_t(0), stream);
  return launch_status();
}
