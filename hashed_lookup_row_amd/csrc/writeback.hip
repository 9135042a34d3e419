// Row updates from a batch.
//
// LAST_WINS — the Writeback of "Memory Layer: Train the In-Model Cache for
// Recommendation Models", sec. 2: the gradient g = M[i] - e_i is applied by
// exact SGD at learning rate 1 so the row becomes e_i; duplicate IDs of the
// batch are deduplicated first so each row receives one exact write.  The
// last occurrence of a row wins.
//   lw_init   clear a transient hash table keyed by row (2n slots)
//   lw_last   per wave, lanes holding the same row are grouped (ballot peel)
//             and only the group's highest lane does the atomicMax of its
//             position, so a hot Zipf row costs one atomic per wave
//   lw_apply  flat 16-byte units (position, column): the winner position of
//             each row reads M and e, writes fl(M - fl(M - e))
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
  int64_t *hkey;   // row held by the slot (-1 = free)
  int32_t *hlast;  // last position of that row
  int32_t *pent;   // per position: its slot, -1 = row skipped
  uint32_t cap;
};

size_t lw_layout(int64_t n, LWWork *w, void *base) {
  Carver c(base);
  const uint64_t cap = next_pow2(static_cast<uint64_t>(n > 32 ? 2 * n : 64));
  w->hkey = c.take<int64_t>(cap);
  w->hlast = c.take<int32_t>(cap);
  w->pent = c.take<int32_t>(static_cast<size_t>(n > 0 ? n : 1));
  w->cap = static_cast<uint32_t>(cap);
  return c.off;
}

__global__ void __launch_bounds__(kThreads) lw_init(LWWork w) {
  const uint32_t stride = kThreads * gridDim.x;
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < w.cap; i += stride) {
    w.hkey[i] = -1;
    w.hlast[i] = -1;
  }
}

__device__ __forceinline__ int32_t lw_slot(LWWork w, int64_t r) {
  const uint32_t mask = w.cap - 1;
  uint32_t s = static_cast<uint32_t>(mix64(static_cast<uint64_t>(r)) >> 32) & mask;
  for (;;) {
    const int64_t k = __hip_atomic_load(&w.hkey[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (k == r) return static_cast<int32_t>(s);
    if (k == -1) {
      const int64_t prev = atomic_cas_i64(&w.hkey[s], -1, r);
      if (prev == -1 || prev == r) return static_cast<int32_t>(s);
    }
    s = (s + 1) & mask;
  }
}

__global__ void __launch_bounds__(kThreads)
    lw_last(const int64_t *__restrict__ rows, int64_t n, int64_t num_rows, LWWork w) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const bool valid = i < n;
  const int64_t r = valid ? rows[i] : -1;
  const bool ok = valid && r >= 0 && r < num_rows;
  if (valid && !ok) w.pent[i] = -1;
  const int64_t i0 = i - lane_id();
  uint64_t todo = ballot(ok);
  while (todo) {
    const int leader = __builtin_ctzll(todo);
    const int64_t rl = readlane_i64(r, leader);
    const uint64_t grp = ballot(ok && r == rl);
    const int last = 63 - __builtin_clzll(grp);
    int32_t s = 0;
    if (lane_id() == leader) {
      s = lw_slot(w, rl);
      atomicMax(&w.hlast[s], static_cast<int32_t>(i0 + last));
    }
    s = readlane_i32(s, leader);
    if ((grp >> lane_id()) & 1ull) w.pent[i] = s;
    todo &= ~grp;
  }
}

template <int V4>
__global__ void __launch_bounds__(kThreads)
    lw_apply(float4 *table, const float4 *__restrict__ src, const int64_t *__restrict__ rows, int64_t n,
             LWWork w, int64_t v4_rt) {
  const int64_t v4 = V4 > 0 ? V4 : v4_rt;
  const int64_t total = n * v4;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (kThreads * kUnroll) + threadIdx.x;
  int64_t dst[kUnroll], from[kUnroll];
#pragma unroll
  for (int k = 0; k < kUnroll; ++k) {
    const int64_t u = base + k * kThreads;
    dst[k] = -1;
    if (u < total) {
      const int64_t i = u / v4;
      const int32_t s = w.pent[i];
      if (s >= 0 && w.hlast[s] == static_cast<int32_t>(i)) {
        const int64_t c = u - i * v4;
        dst[k] = rows[i] * v4 + c;
        from[k] = u;
      }
    }
  }
  float4 m[kUnroll], e[kUnroll];
#pragma unroll
  for (int k = 0; k < kUnroll; ++k) {
    if (dst[k] >= 0) {
      m[k] = table[dst[k]];
      e[k] = src[from[k]];
    }
  }
#pragma unroll
  for (int k = 0; k < kUnroll; ++k) {
    if (dst[k] >= 0) {
      const float4 g = f4_sub(m[k], e[k]);  // g = fl(M - e)
      table[dst[k]] = f4_sub(m[k], g);      // M' = fl(M - g)
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
    int gi = grid_for(w.cap, kThreads * 4);
    if (gi > 2048) gi = 2048;
    lw_init<<<gi, kThreads, 0, stream>>>(w);
    lw_last<<<grid_for(n, kThreads), kThreads, 0, stream>>>(rows, n, num_rows, w);
    const int ga = grid_for(n * v4, kThreads * kUnroll);
    switch (v4) {
      case 16: lw_apply<16><<<ga, kThreads, 0, stream>>>(t4, s4, rows, n, w, v4); break;
      case 32: lw_apply<32><<<ga, kThreads, 0, stream>>>(t4, s4, rows, n, w, v4); break;
      case 128: lw_apply<128><<<ga, kThreads, 0, stream>>>(t4, s4, rows, n, w, v4); break;
      default: lw_apply<0><<<ga, kThreads, 0, stream>>>(t4, s4, rows, n, w, v4); break;
    }
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
