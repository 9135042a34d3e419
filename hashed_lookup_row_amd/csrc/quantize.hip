// int8 row quantisation for publishing touched rows to serving (Raw Embedding
// Streaming in "Memory Layer: Train the In-Model Cache for Recommendation
// Models", sec. 2; serving reads int8 rows, sec. 5).
//
// Per row, asymmetric min-max in fp32, each operation rounded on its own:
//   scale = fl(fl(max - min) / 255)  (1 when max == min)
//   bias  = fl(min + fl(128 * scale))
//   q_d   = clamp(rne(fl(fl(x_d - bias) / scale)), -128, 127)
// One wave per row: lanes own 16-byte column units, min and max are reduced
// across the wave with xor shuffles (order-independent for finite values), and
// each lane stores the four codes of a unit as one 32-bit word.
#include "hlr_common.hpp"

namespace {
using namespace hlr;

constexpr int kThreads = 256;

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ uint32_t code(float x, float bias, float scale) {
  const float centred = x - bias;
  float v = __builtin_rintf(centred / scale);
  v = fminf(fmaxf(v, -128.f), 127.f);
  return static_cast<uint32_t>(static_cast<int32_t>(v)) & 0xffu;
}

template <int NC>
__global__ void __launch_bounds__(kThreads)
    quant_kernel(const float4 *__restrict__ table, int64_t num_rows, int64_t v4, const int64_t *__restrict__ rows,
                 int64_t n, const int64_t *__restrict__ count, int scatter, uint32_t *__restrict__ q,
                 float *__restrict__ out_scale, float *__restrict__ out_bias) {
  int64_t m = n;
  if (count) {
    const int64_t c = *count;
    m = c < 0 ? 0 : (c < n ? c : n);
  }
  const int lane = lane_id();
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (kThreads / kWave);
  for (int64_t i = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / kWave; i < m; i += waves) {
    const int64_t r = rows[i];
    if (r < 0 || r >= num_rows) {
      if (!scatter) {
        for (int64_t c = lane; c < v4; c += kWave) q[i * v4 + c] = 0u;
        if (lane == 0) {
          out_scale[i] = 0.f;
          out_bias[i] = 0.f;
        }
      }
      continue;
    }
    float4 x[NC];
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int64_t c = lane + k * kWave;
      x[k] = table[r * v4 + (c < v4 ? c : 0)];  // lanes past the row end repeat unit 0 (no effect on min/max)
    }
    float lo = x[0].x, hi = x[0].x;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      lo = fminf(fminf(fminf(lo, x[k].x), fminf(x[k].y, x[k].z)), x[k].w);
      hi = fmaxf(fmaxf(fmaxf(hi, x[k].x), fmaxf(x[k].y, x[k].z)), x[k].w);
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    const float range = hi - lo;
    const float scale = range == 0.f ? 1.f : range / 255.f;
    const float bias = lo + 128.f * scale;
    const int64_t o = scatter ? r : i;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int64_t c = lane + k * kWave;
      if (c < v4)
        q[o * v4 + c] = code(x[k].x, bias, scale) | (code(x[k].y, bias, scale) << 8) |
                        (code(x[k].z, bias, scale) << 16) | (code(x[k].w, bias, scale) << 24);
    }
    if (lane == 0) {
      out_scale[o] = scale;
      out_bias[o] = bias;
    }
  }
}

}  // namespace

extern "C" hlr_status quantize_rows_int8(const float *table, int64_t num_rows, int64_t dim, const int64_t *rows,
                                         int64_t n, const int64_t *count, int32_t scatter, int8_t *out_q,
                                         float *out_scale, float *out_bias, hipStream_t stream) {
  if (n < 0 || n > kMaxN || num_rows < 0 || (scatter != 0 && scatter != 1)) return HLR_INVALID_ARG;
  if (dim <= 0 || dim % 4 != 0 || dim > 1024) return HLR_UNSUPPORTED_DIM;
  if (n == 0) return HLR_OK;
  if (!rows || !out_q || !out_scale || !out_bias || (num_rows > 0 && !table)) return HLR_INVALID_ARG;
  if ((table && !aligned(table, 16)) || !aligned(rows, 8) || !aligned(out_q, 4) || !aligned(out_scale, 4) ||
      !aligned(out_bias, 4) || (count && !aligned(count, 8)))
    return HLR_MISALIGNED;
  const int64_t v4 = dim / 4;
  int grid = grid_for(n, kThreads / kWave);
  if (grid > 4096) grid = 4096;
  const float4 *t4 = reinterpret_cast<const float4 *>(table);
  uint32_t *q4 = reinterpret_cast<uint32_t *>(out_q);
  const int64_t nc = (v4 + kWave - 1) / kWave;
  if (nc == 1)
    quant_kernel<1><<<grid, kThreads, 0, stream>>>(t4, num_rows, v4, rows, n, count, scatter, q4, out_scale, out_bias);
  else if (nc == 2)
    quant_kernel<2><<<grid, kThreads, 0, stream>>>(t4, num_rows, v4, rows, n, count, scatter, q4, out_scale, out_bias);
  else
    quant_kernel<4><<<grid, kThreads, 0, stream>>>(t4, num_rows, v4, rows, n, count, scatter, q4, out_scale, out_bias);
  return launch_status();
}
