// EMA row updates ("CS3: Efficient Online Capability Synergy for Two-Tower
// Recommendation", sec. 2): CTS keeps c <- a*c + (1-a)*v for positive
// interactions only (mask = labels), CMS keeps s <- b*s + (1-b)*h for every
// interaction (mask = NULL).  Duplicates of a row are applied in batch order.
//
// Plan: positions that take part are grouped by row with a stable radix sort
// (radix.hpp), so each row's positions come out in batch order.  A row's
// positions are applied in order (T = fl(fl(a*T) + fl(b*v))): short rows by
// one wave each (ema_light), long rows by blocks that stream the value rows
// through LDS, one chunk per block, the chunks of a row running in parallel
// from speculative warmed-up states (ema_heavy) that ema_combine verifies bit
// for bit.  The result equals the sequential loop bit for bit.
#include <cmath>

#include "radix.hpp"

namespace {
using namespace hlr;

constexpr int kThreads = 256;

__device__ __forceinline__ float4 ema_step(float4 t, float4 v, float a, float b) {
  return make_float4(a * t.x + b * v.x, a * t.y + b * v.y, a * t.z + b * v.z, a * t.w + b * v.w);
}

constexpr int kPrefetch = 16;

// state <- step(state, vals[spos[j]]) for j in [j0, j1), in order, next loads in flight.
template <int NC>
__device__ __forceinline__ void ema_run(const float4 *__restrict__ vals, const uint32_t *__restrict__ spos,
                                        int32_t j0, int32_t j1, int64_t v4, int lane, float a, float b,
                                        float4 (&t)[NC]) {
  int32_t j = j0;
  for (; j + kPrefetch <= j1; j += kPrefetch) {
    float4 x[kPrefetch][NC];
#pragma unroll
    for (int u = 0; u < kPrefetch; ++u) {
      const int64_t p = spos[j + u];
#pragma unroll
      for (int q = 0; q < NC; ++q) {
        const int64_t c = lane + q * kWave;
        x[u][q] = c < v4 ? vals[p * v4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int u = 0; u < kPrefetch; ++u)
#pragma unroll
      for (int q = 0; q < NC; ++q) t[q] = ema_step(t[q], x[u][q], a, b);
  }
  for (; j < j1; ++j) {
    const int64_t p = spos[j];
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      const int64_t c = lane + q * kWave;
      const float4 x = c < v4 ? vals[p * v4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
      t[q] = ema_step(t[q], x, a, b);
    }
  }
}

// Light rows (fewer than kHeavyMin occurrences): one wave per row, exact.
// Longer rows are registered (in chunks of L) for the block kernels.
template <int NC>
__global__ void __launch_bounds__(kThreads)
    ema_light(float4 *table, const float4 *__restrict__ vals, const uint32_t *__restrict__ skey,
              const uint32_t *__restrict__ spos, const int32_t *__restrict__ seg_start,
              const int32_t *__restrict__ seg_end, const int64_t *__restrict__ nseg_p, float a, float b, int64_t v4,
              int L, uint32_t *counters, int2 *hlist, int32_t *clist) {
  const int64_t nseg = *nseg_p;
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (kThreads / kWave);
  const int lane = lane_id();
  for (int64_t k = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / kWave; k < nseg; k += waves) {
    const int32_t s = seg_start[k], e = seg_end[k];
    if (e - s >= kHeavyMin) {
      if (lane == 0) push_heavy(static_cast<int32_t>(k), e - s, L, counters, hlist, clist);
      continue;
    }
    const int64_t r = skey[s];
    float4 st[NC];
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      const int64_t c = lane + q * kWave;
      st[q] = c < v4 ? table[r * v4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    ema_run<NC>(vals, spos, s, e, v4, lane, a, b, st);
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      const int64_t c = lane + q * kWave;
      if (c < v4) table[r * v4 + c] = st[q];
    }
  }
}

// Heavy rows: one block per chunk of <= L occurrences, the value rows streamed
// through LDS (block_stream).  A row with one chunk is applied exactly from its
// stored value.  For a longer row, chunk 0 runs exactly; chunk m > 0 starts W
// occurrences early from a zero state (the recurrence contracts by a per step,
// so after W steps the state no longer depends on where it started) and
// records sigma (the state entering its first occurrence) and tau (the state
// after its last) for ema_combine.
template <int EPT>
__global__ void __launch_bounds__(kThreads)
    ema_heavy(float *table, const float *__restrict__ vals, const uint32_t *__restrict__ skey,
              const uint32_t *__restrict__ spos, const int32_t *__restrict__ seg_start,
              const int32_t *__restrict__ seg_end, const uint32_t *__restrict__ counters,
              const int2 *__restrict__ hlist, float a, float b, int64_t D, int L, int W, float *partial) {
  __shared__ float lds[2 * kStageFloats];
  const uint32_t count = counters[0];
  const int64_t v4 = D / 4;
  const float4 *x4 = reinterpret_cast<const float4 *>(vals);
  const int tid = threadIdx.x;
  auto row_of = [&](int32_t j) { return x4 + static_cast<int64_t>(spos[j]) * v4; };
  for (uint32_t i = blockIdx.x; i < count; i += gridDim.x) {
    const int2 km = hlist[i];
    const int32_t s = seg_start[km.x], e = seg_end[km.x];
    const int64_t r = skey[s];
    const int32_t j0 = s + km.y * L;
    const int32_t j1 = j0 + L < e ? j0 + L : e;
    const bool exact_start = km.y == 0 || j0 - W <= s;
    const int32_t from = exact_start ? s : j0 - W;
    float st[EPT], sig[EPT];
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int64_t el = tid + 256 * q;
      st[q] = (exact_start && el < D) ? table[r * D + el] : 0.f;
      sig[q] = st[q];
    }
    if (e - s <= L) {  // the whole row in one chunk
      block_stream<EPT>(row_of, s, e, D, lds, [&](int32_t, int q, float v) { st[q] = a * st[q] + b * v; });
#pragma unroll
      for (int q = 0; q < EPT; ++q) {
        const int64_t el = tid + 256 * q;
        if (el < D) table[r * D + el] = st[q];
      }
      continue;
    }
    block_stream<EPT>(row_of, from, j1, D, lds, [&](int32_t j, int q, float v) {
      if (j == j0) sig[q] = st[q];
      st[q] = a * st[q] + b * v;
    });
    const int64_t slot = run_slot(j0, km.y, L);
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int64_t el = tid + 256 * q;
      if (el < D) {
        partial[(2 * slot) * D + el] = sig[q];
        partial[(2 * slot + 1) * D + el] = st[q];
      }
    }
  }
}

// Rows with several chunks: walk the chunks in order.  If sigma_m equals the
// exact state entering chunk m bit for bit, tau_m is exact; otherwise chunk m is
// recomputed from the exact state.  The result equals the sequential loop bit
// for bit in every case; speculation only decides how much ran in parallel.
template <int EPT>
__global__ void __launch_bounds__(kThreads)
    ema_combine(float *table, const float *__restrict__ vals, const uint32_t *__restrict__ skey,
                const uint32_t *__restrict__ spos, const int32_t *__restrict__ seg_start,
                const int32_t *__restrict__ seg_end, const uint32_t *__restrict__ counters,
                const int32_t *__restrict__ clist, float a, float b, int64_t D, int L,
                const float *__restrict__ partial) {
  __shared__ float lds[2 * kStageFloats];
  const uint32_t count = counters[1];
  const int64_t v4 = D / 4;
  const float4 *x4 = reinterpret_cast<const float4 *>(vals);
  const int tid = threadIdx.x;
  auto row_of = [&](int32_t j) { return x4 + static_cast<int64_t>(spos[j]) * v4; };
  for (uint32_t i = blockIdx.x; i < count; i += gridDim.x) {
    const int32_t k = clist[i];
    const int32_t s = seg_start[k], e = seg_end[k];
    const int32_t nch = (e - s + L - 1) / L;
    float cur[EPT];
    const int64_t s0 = run_slot(s, 0, L);
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int64_t el = tid + 256 * q;
      cur[q] = el < D ? partial[(2 * s0 + 1) * D + el] : 0.f;
    }
    for (int32_t m = 1; m < nch; ++m) {
      const int32_t c0 = s + m * L;
      const int32_t c1 = c0 + L < e ? c0 + L : e;
      const int64_t sl = run_slot(c0, m, L);
      float tau[EPT];
      bool ok = true;
#pragma unroll
      for (int q = 0; q < EPT; ++q) {
        const int64_t el = tid + 256 * q;
        tau[q] = cur[q];
        if (el < D) {
          const float sg = partial[(2 * sl) * D + el];
          tau[q] = partial[(2 * sl + 1) * D + el];
          ok = ok && __float_as_uint(sg) == __float_as_uint(cur[q]);
        }
      }
      if (!__syncthreads_or(!ok)) {
#pragma unroll
        for (int q = 0; q < EPT; ++q) cur[q] = tau[q];
        continue;
      }
      // a speculative start differs somewhere: recompute this chunk from the exact state
      block_stream<EPT>(row_of, c0, c1, D, lds, [&](int32_t, int q, float v) { cur[q] = a * cur[q] + b * v; });
    }
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int64_t el = tid + 256 * q;
      if (el < D) table[skey[s] * D + el] = cur[q];
    }
  }
}

// Chunking: warm-up W = ceil(32 / -ln a) steps shrinks a start error by e^-32
// (below fp32 resolution) before a speculative chunk starts; L >= W keeps the
// extra work below 2x.  Without contraction (a outside (0, 1)) rows run whole.
inline void ema_plan(float a, int64_t n, int *L, int *W) {
  constexpr int kMinChunk = 1024;
  if (a > 0.f && a < 1.f) {
    const double w = std::ceil(32.0 / -std::log(static_cast<double>(a)));
    *W = static_cast<int>(w < 1048576.0 ? w : 1048576.0);
    *L = *W > kMinChunk ? *W : kMinChunk;
  } else {
    *W = 0;
    *L = static_cast<int>(n > kMinChunk ? (n < 0x7fffffff ? n : 0x7fffffff) : kMinChunk);
  }
}

inline size_t ema_partial_elems(int64_t n, int64_t dim) {
  // sized for the smallest chunk length (1024): (2 * ceil(n / 1024) + 2) slots x (sigma, tau)
  return static_cast<size_t>(2 * ((n + 1023) / 1024) + 2) * 2 * static_cast<size_t>(dim / 4);
}

template <int NC, int EPT>
void ema_launch(float *table, const float *vals, SegWork<uint32_t> &w, int cur, float a, float b, int64_t dim,
                float *partial, hipStream_t s) {
  int L, W;
  ema_plan(a, w.n, &L, &W);
  const int64_t v4 = dim / 4;
  int grid = grid_for(w.n, 4 * 4);
  if (grid > 4096) grid = 4096;
  ema_light<NC><<<grid, kThreads, 0, s>>>(reinterpret_cast<float4 *>(table), reinterpret_cast<const float4 *>(vals),
                                          w.k[cur], w.v[cur], w.seg_start, w.seg_end, w.nseg, a, b, v4, L, w.ticket,
                                          w.hlist, w.clist);
  ema_heavy<EPT><<<kHeavyBlocks, kThreads, 0, s>>>(table, vals, w.k[cur], w.v[cur], w.seg_start, w.seg_end,
                                                    w.ticket, w.hlist, a, b, dim, L, W, partial);
  ema_combine<EPT><<<kHeavyBlocks, kThreads, 0, s>>>(table, vals, w.k[cur], w.v[cur], w.seg_start, w.seg_end,
                                                      w.ticket, w.clist, a, b, dim, L, partial);
}

}  // namespace

extern "C" size_t ema_update_rows_workspace_size(int64_t num_rows, int64_t dim, int64_t n) {
  (void)num_rows;
  (void)dim;
  if (n < 0) return 0;
  SegWork<uint32_t> w;
  Carver c(nullptr);
  c.off = segwork_layout<uint32_t>(n, &w, nullptr);
  c.take<float4>(ema_partial_elems(n, dim > 0 ? dim : 4));
  return c.off;
}

extern "C" hlr_status ema_update_rows(float *table, int64_t num_rows, int64_t dim, const int64_t *rows,
                                      const float *vals, const uint8_t *mask, int64_t n, float a, float b, void *ws,
                                      size_t ws_bytes, hipStream_t stream) {
  if (n < 0 || n > kMaxN || num_rows < 0 || num_rows >= 0x7fffffff) return HLR_INVALID_ARG;
  if (dim <= 0 || dim % 4 != 0 || dim > 1024) return HLR_UNSUPPORTED_DIM;
  if (n == 0 || num_rows == 0) return HLR_OK;
  if (!table || !rows || !vals) return HLR_INVALID_ARG;
  if (!aligned(table, 16) || !aligned(vals, 16) || !aligned(rows, 8)) return HLR_MISALIGNED;
  const size_t need = ema_update_rows_workspace_size(num_rows, dim, n);
  if (!ws || ws_bytes < need) return HLR_WORKSPACE_TOO_SMALL;
  if (!aligned(ws, 256)) return HLR_MISALIGNED;
  SegWork<uint32_t> w;
  Carver c(ws);
  c.off = segwork_layout<uint32_t>(n, &w, ws);
  float *partial = reinterpret_cast<float *>(c.take<float4>(ema_partial_elems(n, dim)));
  const int cur = group_by_row(w, rows, mask, num_rows, stream);
  const int64_t nc = (dim / 4 + kWave - 1) / kWave;
  if (nc == 1) ema_launch<1, 1>(table, vals, w, cur, a, b, dim, partial, stream);
  else if (nc == 2) ema_launch<2, 2>(table, vals, w, cur, a, b, dim, partial, stream);
  else ema_launch<4, 4>(table, vals, w, cur, a, b, dim, partial, stream);
  return launch_status();
}
