// Row updates from a batch.
//
// LAST_WINS — the Writeback of "Memory Layer: Train the In-Model Cache for
// Recommendation Models", sec. 2: the gradient g = M[i] - e_i is applied by
// exact SGD at learning rate 1 so the row becomes e_i; duplicate IDs of the
// batch are deduplicated first so each row receives one exact write.  The
// last occurrence of a row wins.
//   lw_init   clear a transient hash table keyed by row (2n slots)
//   lw_last   a block folds its positions in LDS (row -> last position),
//             then one global atomicMax per distinct row of the block; new
//             global slots go to a compact list
//   lw_apply  one wave per distinct row: reads M and e at the last
//             occurrence, writes fl(M - fl(M - e)) with 16-byte accesses
//
// SGD_SUM — per-row SGD with duplicate gradients summed and applied once (the
// same sparse-table update pattern at a learning rate other than 1, as in the
// hashed tables of "DLRMv4: MLPerf recommendation training goes sequential").
// Positions are grouped by row with a stable radix sort (radix.hpp); one wave
// owns a row: it sums the row's gradients in batch order in runs of 256
// occurrences (run totals added in batch order) and writes
// fl(M - fl(lr * s)).
#include "radix.hpp"

namespace {
using namespace hlr;

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

struct LWWork {
  int64_t *hkey;    // row held by the slot (-1 = free)
  int32_t *hlast;   // last position of that row
  int32_t *list;    // slots in use, compacted (first *count entries)
  uint32_t *count;  // [1]
  uint32_t cap;
};

size_t lw_layout(int64_t n, LWWork *w, void *base) {
  Carver c(base);
  const uint64_t cap = next_pow2(static_cast<uint64_t>(n > 32 ? 2 * n : 64));
  w->hkey = c.take<int64_t>(cap);
  w->hlast = c.take<int32_t>(cap);
  w->list = c.take<int32_t>(cap);
  w->count = c.take<uint32_t>(1);
  w->cap = static_cast<uint32_t>(cap);
  return c.off;
}

__global__ void __launch_bounds__(kThreads) lw_init(LWWork w) {
  const uint32_t stride = kThreads * gridDim.x;
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < w.cap; i += stride) {
    w.hkey[i] = -1;
    w.hlast[i] = -1;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *w.count = 0u;
}

// Last occurrence of every row.  A block first folds its 512 positions in an
// LDS hash table (row -> largest position, LDS atomics), then publishes one
// global atomicMax per distinct row of the block: a hot Zipf row costs one
// global atomic per block, not one per position.  Each thread issues the CAS
// of all its LDS entries before waiting on any, so the global round trips
// overlap.  Newly claimed global slots are appended to a compact list (one
// global atomicAdd per block).
constexpr int kLwItems = 2;
constexpr int kLwTile = kThreads * kLwItems;  // positions per block
constexpr int kLwLds = 2 * kLwTile;           // LDS hash entries
constexpr int kLwPer = kLwLds / kThreads;     // LDS entries scanned per thread

__global__ void __launch_bounds__(kThreads)
    lw_last(const int64_t *__restrict__ rows, int64_t n, int64_t num_rows, LWWork w) {
  __shared__ unsigned long long lkey[kLwLds];
  __shared__ int32_t lpos[kLwLds];
  __shared__ int32_t lnew_slots[kLwLds];
  __shared__ uint32_t lnew, lbase;
  for (int e = threadIdx.x; e < kLwLds; e += kThreads) {
    lkey[e] = ~0ull;
    lpos[e] = -1;
  }
  if (threadIdx.x == 0) lnew = 0u;
  __syncthreads();
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kLwTile;
#pragma unroll
  for (int k = 0; k < kLwItems; ++k) {
    const int64_t i = base + k * kThreads + threadIdx.x;
    if (i >= n) continue;
    const int64_t r = rows[i];
    if (r < 0 || r >= num_rows) continue;
    uint32_t e = static_cast<uint32_t>(mix64(static_cast<uint64_t>(r)) >> 40) & (kLwLds - 1);
    for (;;) {
      const unsigned long long prev = atomicCAS(&lkey[e], ~0ull, static_cast<unsigned long long>(r));
      if (prev == ~0ull || prev == static_cast<unsigned long long>(r)) break;
      e = (e + 1) & (kLwLds - 1);
    }
    atomicMax(&lpos[e], static_cast<int32_t>(i));
  }
  __syncthreads();
  const uint32_t mask = w.cap - 1;
  int64_t key[kLwPer];
  int32_t pos[kLwPer];
  uint32_t gs[kLwPer];
  int64_t prev[kLwPer];
#pragma unroll
  for (int j = 0; j < kLwPer; ++j) {
    const int e = threadIdx.x + j * kThreads;
    const unsigned long long k = lkey[e];
    key[j] = k == ~0ull ? -1 : static_cast<int64_t>(k);
    pos[j] = lpos[e];
    gs[j] = static_cast<uint32_t>(mix64(static_cast<uint64_t>(key[j])) >> 32) & mask;
  }
  // all first-probe CAS in flight together
#pragma unroll
  for (int j = 0; j < kLwPer; ++j) prev[j] = key[j] >= 0 ? atomic_cas_i64(&w.hkey[gs[j]], -1, key[j]) : key[j];
#pragma unroll
  for (int j = 0; j < kLwPer; ++j) {
    if (key[j] < 0) continue;
    bool created = prev[j] == -1;
    while (!created && prev[j] != key[j]) {  // collision: linear probing
      gs[j] = (gs[j] + 1) & mask;
      prev[j] = atomic_cas_i64(&w.hkey[gs[j]], -1, key[j]);
      created = prev[j] == -1;
    }
    atomicMax(&w.hlast[gs[j]], pos[j]);
    if (created) lnew_slots[atomicAdd(&lnew, 1u)] = static_cast<int32_t>(gs[j]);
  }
  __syncthreads();
  if (threadIdx.x == 0) lbase = lnew ? atomicAdd(w.count, lnew) : 0u;
  __syncthreads();
  for (uint32_t j = threadIdx.x; j < lnew; j += kThreads) w.list[lbase + j] = lnew_slots[j];
}

// One wave per winner row (two rows in flight per wave): g = fl(M - e), M' = fl(M - g).
template <int NC>
__global__ void __launch_bounds__(kThreads)
    lw_apply(float4 *table, const float4 *__restrict__ src, LWWork w, int64_t v4) {
  constexpr int RPW = 2;
  const uint32_t count = *w.count;
  const int lane = lane_id();
  const uint32_t waves = gridDim.x * (kThreads / kWave);
  for (uint32_t j0 = ((blockIdx.x * kThreads + threadIdx.x) / kWave) * RPW; j0 < count; j0 += waves * RPW) {
    int64_t mrow[RPW], erow[RPW];
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      mrow[q] = -1;
      if (j0 + q < count) {
        const int32_t s = w.list[j0 + q];
        mrow[q] = w.hkey[s] * v4;
        erow[q] = static_cast<int64_t>(w.hlast[s]) * v4;
      }
    }
    float4 m[RPW][NC], e[RPW][NC];
#pragma unroll
    for (int q = 0; q < RPW; ++q)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int64_t col = lane + c * kWave;
        if (mrow[q] >= 0 && col < v4) {
          m[q][c] = table[mrow[q] + col];
          e[q][c] = src[erow[q] + col];
        }
      }
#pragma unroll
    for (int q = 0; q < RPW; ++q)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int64_t col = lane + c * kWave;
        if (mrow[q] >= 0 && col < v4) {
          const float4 g = f4_sub(m[q][c], e[q][c]);  // g = fl(M - e)
          table[mrow[q] + col] = f4_sub(m[q][c], g);  // M' = fl(M - g)
        }
      }
  }
}

// One wave per row segment; lanes own 16-byte column units (NC per lane).
template <int NC>
__global__ void __launch_bounds__(kThreads)
    sgd_apply(float4 *table, const float4 *__restrict__ g, const uint32_t *__restrict__ skey,
              const uint32_t *__restrict__ spos, const int32_t *__restrict__ seg_start,
              const int32_t *__restrict__ seg_end, const int64_t *__restrict__ nseg, float lr, int64_t v4) {
  const int64_t nsegs = *nseg;
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (kThreads / kWave);
  const int lane = lane_id();
  for (int64_t k = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / kWave; k < nsegs; k += waves) {
    const int32_t s = seg_start[k], e = seg_end[k];
    const int64_t r = skey[s];
    float4 tot[NC], run[NC];
    for (int32_t rs = s; rs < e; rs += HLR_SGD_SUM_RUN) {
      const int32_t re = rs + HLR_SGD_SUM_RUN < e ? rs + HLR_SGD_SUM_RUN : e;
      {
        const int64_t p = spos[rs];
#pragma unroll
        for (int q = 0; q < NC; ++q) {
          const int64_t c = lane + q * kWave;
          run[q] = c < v4 ? g[p * v4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      int32_t j = rs + 1;
      for (; j + 4 <= re; j += 4) {
        float4 x[4][NC];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t p = spos[j + u];
#pragma unroll
          for (int q = 0; q < NC; ++q) {
            const int64_t c = lane + q * kWave;
            x[u][q] = c < v4 ? g[p * v4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int q = 0; q < NC; ++q) run[q] = make_float4(run[q].x + x[u][q].x, run[q].y + x[u][q].y,
                                                            run[q].z + x[u][q].z, run[q].w + x[u][q].w);
      }
      for (; j < re; ++j) {
        const int64_t p = spos[j];
#pragma unroll
        for (int q = 0; q < NC; ++q) {
          const int64_t c = lane + q * kWave;
          const float4 x = c < v4 ? g[p * v4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
          run[q] = make_float4(run[q].x + x.x, run[q].y + x.y, run[q].z + x.z, run[q].w + x.w);
        }
      }
#pragma unroll
      for (int q = 0; q < NC; ++q)
        tot[q] = rs == s ? run[q]
                         : make_float4(tot[q].x + run[q].x, tot[q].y + run[q].y, tot[q].z + run[q].z,
                                       tot[q].w + run[q].w);
    }
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      const int64_t c = lane + q * kWave;
      if (c < v4) {
        const float4 wv = table[r * v4 + c];
        const float4 st = make_float4(lr * tot[q].x, lr * tot[q].y, lr * tot[q].z, lr * tot[q].w);
        table[r * v4 + c] = f4_sub(wv, st);
      }
    }
  }
}

template <int NC>
void sgd_launch(float4 *t4, const float4 *g4, SegWork<uint32_t> &w, int cur, float lr, int64_t v4, hipStream_t s) {
  int grid = grid_for(w.n, 4 * 8);  // ~8 segments per wave at most, 4 waves per block
  if (grid > 2048) grid = 2048;
  sgd_apply<NC><<<grid, kThreads, 0, s>>>(t4, g4, w.k[cur], w.v[cur], w.seg_start, w.seg_end, w.nseg, lr, v4);
}

}  // namespace

extern "C" size_t writeback_rows_workspace_size(int64_t num_rows, int64_t dim, int64_t n, int32_t mode) {
  (void)num_rows;
  (void)dim;
  if (n < 0) return 0;
  if (mode == HLR_WB_LAST_WINS) {
    LWWork w;
    return lw_layout(n, &w, nullptr);
  }
  SegWork<uint32_t> w;
  return segwork_layout<uint32_t>(n, &w, nullptr);
}

extern "C" hlr_status writeback_rows(float *table, int64_t num_rows, int64_t dim, const int64_t *rows,
                                     const float *src, int64_t n, int32_t mode, float lr, void *ws, size_t ws_bytes,
                                     hipStream_t stream) {
  if (n < 0 || n > kMaxN || num_rows < 0 || num_rows >= 0x7fffffff) return HLR_INVALID_ARG;
  if (mode != HLR_WB_LAST_WINS && mode != HLR_WB_SGD_SUM) return HLR_INVALID_ARG;
  if (mode == HLR_WB_LAST_WINS && lr != 1.0f) return HLR_INVALID_ARG;
  if (dim <= 0 || dim % 4 != 0) return HLR_UNSUPPORTED_DIM;
  if (n == 0 || num_rows == 0) return HLR_OK;
  if (!table || !rows || !src) return HLR_INVALID_ARG;
  if (!aligned(table, 16) || !aligned(src, 16) || !aligned(rows, 8)) return HLR_MISALIGNED;
  const size_t need = writeback_rows_workspace_size(num_rows, dim, n, mode);
  if (!ws || ws_bytes < need) return HLR_WORKSPACE_TOO_SMALL;
  if (!aligned(ws, 256)) return HLR_MISALIGNED;
  const int64_t v4 = dim / 4;
  float4 *t4 = reinterpret_cast<float4 *>(table);
  const float4 *s4 = reinterpret_cast<const float4 *>(src);
  if (mode == HLR_WB_LAST_WINS) {
    LWWork w;
    lw_layout(n, &w, ws);
    int gi = grid_for(w.cap, kThreads);
    if (gi > 4096) gi = 4096;
    lw_init<<<gi, kThreads, 0, stream>>>(w);
    lw_last<<<grid_for(n, kLwTile), kThreads, 0, stream>>>(rows, n, num_rows, w);
    int ga = grid_for(n, 8);
    if (ga > 2048) ga = 2048;
    const int64_t nc = (v4 + kWave - 1) / kWave;
    if (nc == 1) lw_apply<1><<<ga, kThreads, 0, stream>>>(t4, s4, w, v4);
    else if (nc == 2) lw_apply<2><<<ga, kThreads, 0, stream>>>(t4, s4, w, v4);
    else if (nc <= 4) lw_apply<4><<<ga, kThreads, 0, stream>>>(t4, s4, w, v4);
    else return HLR_UNSUPPORTED_DIM;
    return launch_status();
  }
  SegWork<uint32_t> w;
  segwork_layout<uint32_t>(n, &w, ws);
  const int cur = group_by_row(w, rows, nullptr, num_rows, stream);
  const int64_t nc = (v4 + kWave - 1) / kWave;
  if (nc == 1) sgd_launch<1>(t4, s4, w, cur, lr, v4, stream);
  else if (nc == 2) sgd_launch<2>(t4, s4, w, cur, lr, v4, stream);
  else if (nc <= 4) sgd_launch<4>(t4, s4, w, cur, lr, v4, stream);
  else return HLR_UNSUPPORTED_DIM;  // dim > 1024
  return launch_status();
}
