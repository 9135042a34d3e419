// EMA row updates ("CS3: Efficient Online Capability Synergy for Two-Tower
// Recommendation", sec. 2): CTS keeps c <- a*c + (1-a)*v for positive
// interactions only (mask = labels), CMS keeps s <- b*s + (1-b)*h for every
// interaction (mask = NULL).  Duplicates of a row are applied in batch order.
//
// Plan: positions that take part are grouped by row with a stable radix sort
// (radix.hpp), so each row's positions come out in batch order.  One wave owns
// a row: lanes own 16-byte column units, the row is read once, the positions'
// vectors are applied in order (T = fl(fl(a*T) + fl(b*v))) with the next
// vectors' loads issued ahead, and the row is written once.  The result equals
// the sequential loop bit for bit.
#include "radix.hpp"

namespace {
using namespace hlr;

constexpr int kThreads = 256;

__device__ __forceinline__ float4 ema_step(float4 t, float4 v, float a, float b) {
  return make_float4(a * t.x + b * v.x, a * t.y + b * v.y, a * t.z + b * v.z, a * t.w + b * v.w);
}

template <int NC>
__global__ void __launch_bounds__(kThreads)
    ema_apply(float4 *table, const float4 *__restrict__ vals, const uint32_t *__restrict__ skey,
              const uint32_t *__restrict__ spos, const int32_t *__restrict__ seg_start,
              const int32_t *__restrict__ seg_end, const int64_t *__restrict__ nseg, float a, float b, int64_t v4) {
  const int64_t nsegs = *nseg;
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (kThreads / kWave);
  const int lane = lane_id();
  for (int64_t k = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / kWave; k < nsegs; k += waves) {
    const int32_t s = seg_start[k], e = seg_end[k];
    const int64_t r = skey[s];
    float4 t[NC];
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      const int64_t c = lane + q * kWave;
      t[q] = c < v4 ? table[r * v4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    int32_t j = s;
    for (; j + 4 <= e; j += 4) {
      float4 x[4][NC];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t p = spos[j + u];
#pragma unroll
        for (int q = 0; q < NC; ++q) {
          const int64_t c = lane + q * kWave;
          x[u][q] = c < v4 ? vals[p * v4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < NC; ++q) t[q] = ema_step(t[q], x[u][q], a, b);
    }
    for (; j < e; ++j) {
      const int64_t p = spos[j];
#pragma unroll
      for (int q = 0; q < NC; ++q) {
        const int64_t c = lane + q * kWave;
        const float4 x = c < v4 ? vals[p * v4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
        t[q] = ema_step(t[q], x, a, b);
      }
    }
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      const int64_t c = lane + q * kWave;
      if (c < v4) table[r * v4 + c] = t[q];
    }
  }
}

template <int NC>
void ema_launch(float4 *t4, const float4 *v4p, SegWork<uint32_t> &w, int cur, float a, float b, int64_t v4,
                hipStream_t s) {
  int grid = grid_for(w.n, 4 * 8);
  if (grid > 2048) grid = 2048;
  ema_apply<NC><<<grid, kThreads, 0, s>>>(t4, v4p, w.k[cur], w.v[cur], w.seg_start, w.seg_end, w.nseg, a, b, v4);
}

}  // namespace

extern "C" size_t ema_update_rows_workspace_size(int64_t num_rows, int64_t dim, int64_t n) {
  (void)num_rows;
  (void)dim;
  if (n < 0) return 0;
  SegWork<uint32_t> w;
  return segwork_layout<uint32_t>(n, &w, nullptr);
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
  segwork_layout<uint32_t>(n, &w, ws);
  const int cur = group_by_row(w, rows, mask, num_rows, stream);
  const int64_t v4 = dim / 4;
  float4 *t4 = reinterpret_cast<float4 *>(table);
  const float4 *x4 = reinterpret_cast<const float4 *>(vals);
  const int64_t nc = (v4 + kWave - 1) / kWave;
  if (nc == 1) ema_launch<1>(t4, x4, w, cur, a, b, v4, stream);
  else if (nc == 2) ema_launch<2>(t4, x4, w, cur, a, b, v4, stream);
  else ema_launch<4>(t4, x4, w, cur, a, b, v4, stream);
  return launch_status();
}
