// The row traffic of one Memory-Layer batch as one pass over its rows
// ("Memory Layer: Train the In-Model Cache for Recommendation Models", sec. 2:
// the model reads the cached row M[i] of every position, then the Writeback
// applies g = M[i] - e_i by exact SGD at learning rate 1, once per distinct
// row, so the row becomes the item-tower vector of its last occurrence).
//
// Done as two kernels (gather, then Writeback), every stored row is read twice
// and a duplicated row is read again by every block that holds one of its
// positions.  Here the lookup's last kernel groups the batch's positions by
// row (mlwork.hpp) and the compute stream makes one pass, ml_fused: one wave
// per group reads the row once (the zero vector for a row the batch inserted:
// it has not been cleared, and a new ID reads zero), writes it to every
// position of the group, and applies M' = fl(M - fl(M - e_last)).  A group
// holding every position of its row applies the Writeback at once.  The
// groups of a row spread over several tiles each add their count to the
// row's done counter once their own reads of the row have returned, and the
// group that completes the count applies the Writeback, so no group reads the
// row after it is rewritten.  The group that applies a row's Writeback returns
// the row's plan entries to zero.  Positions without a row (overflow, invalid ID)
// form groups of their own and read the zero vector.  Groups, and the
// positions inside a group, come in no fixed order; every output is
// nevertheless fixed: each position's gathered row, and each row's Writeback
// from its last occurrence.
#include "mlwork.hpp"
#include "step_parts.hpp"

namespace {
using namespace hlr;

// One wave per group, one group per wave: a plain grid of blocks that retire
// as they finish (a persistent grid holding every wave slot measured slower,
// and kept the next batch's lookup kernels from running beside it).  Lanes
// own 16-byte units lane + 64 c of a row.
template <int NC>
__global__ void __launch_bounds__(ml::kThreads)
    ml_fused(float4 *table, const float4 *__restrict__ src, float4 *__restrict__ out, int64_t v4, ml::Work w) {
  const uint32_t g = __builtin_amdgcn_readfirstlane(blockIdx.x * (ml::kThreads / kWave) + threadIdx.x / kWave);
  const uint32_t tile = g / ml::kTile;  // group j of tile t is descriptor t * kTile + j
  if (tile >= w.tiles || g % ml::kTile >= w.ntile[tile]) return;
  const int lane = lane_id();
  int64_t col[NC];
  bool on[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    col[c] = lane + c * kWave;
    on[c] = col[c] < v4;
    if (!on[c]) col[c] = 0;
  }
  const uint4 d = w.gdesc[g];
  const uint32_t cnt = d.w & ml::kCountMask;
  const bool norow = d.w & ml::kNoRow;
  const uint32_t row = norow ? 0u : d.x;
  // the row (loaded from row 0 and dropped when there is none to read: a load
  // under a condition would be waited for inside it), the row's totals, the
  // first 64 positions
  const bool read = !(d.w & (ml::kNoRow | ml::kFresh));
  const int64_t rb = read ? static_cast<int64_t>(row) * v4 : 0;
  float4 m[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) m[c] = table[rb + col[c]];
  const uint2 hc = norow ? make_uint2(cnt, 1u) : *reinterpret_cast<const uint2 *>(&w.hrow[row]);
  const uint32_t total = hc.x;
  const uint32_t last1 = hc.y;  // last position + 1
  const int32_t pv = w.gpos[d.z + (static_cast<uint32_t>(lane) < cnt ? lane : 0)];
  // whole is the same in every lane (one descriptor, one record): a scalar
  // branch, so a group that does not apply the Writeback now loads no e (an
  // e read from row 0 and dropped cost about 1 us per batch in L2 traffic)
  const bool whole = __builtin_amdgcn_readfirstlane(static_cast<int>(!norow && total == cnt)) != 0;
  float4 e[NC];
  if (whole) {
    const int64_t eb = static_cast<int64_t>(last1 - 1) * v4;
#pragma unroll
    for (int c = 0; c < NC; ++c) e[c] = src[eb + col[c]];
  } else {
#pragma unroll
    for (int c = 0; c < NC; ++c) e[c] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (!read) {
#pragma unroll
    for (int c = 0; c < NC; ++c) m[c] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // the gather: the row to every position of the group
  const uint32_t nk = cnt < kWave ? cnt : kWave;
  for (uint32_t k = 0; k < nk; ++k) {
    const int64_t ob = static_cast<int64_t>(__builtin_amdgcn_readlane(pv, k)) * v4;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      if (on[c]) store_nt(out + ob + col[c], m[c]);
  }
  for (uint32_t k0 = kWave; k0 < cnt; k0 += kWave) {
    const uint32_t left = cnt - k0;
    const int32_t pk = w.gpos[d.z + k0 + (static_cast<uint32_t>(lane) < left ? lane : 0)];
    const uint32_t nk2 = left < kWave ? left : kWave;
    for (uint32_t k = 0; k < nk2; ++k) {
      const int64_t ob = static_cast<int64_t>(__builtin_amdgcn_readlane(pk, k)) * v4;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (on[c]) store_nt(out + ob + col[c], m[c]);
    }
  }
  if (norow) return;
  if (!whole) {
    // This group's reads of the row and of its entries have returned (the
    // stores above used them); count its positions as done.  The group that
    // completes the row applies the Writeback; every other group of the row
    // has read the row's entries by then.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    uint32_t prev = 0;
    if (lane == 0) prev = atomicAdd(&w.hrow[row].z, cnt);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev + cnt != total) return;
    const int64_t lb = static_cast<int64_t>(last1 - 1) * v4;
#pragma unroll
    for (int c = 0; c < NC; ++c) e[c] = src[lb + col[c]];
  }
  if (lane == 0) w.hrow[row] = make_uint4(0u, 0u, 0u, 0u);  // the row's entry back to zero for the next batch
  // fl(M - fl(M - e)), stored non-temporally like the gathered rows (the next
  // batch that reads the row finds it in HBM either way; plain stores measured
  // about 1 us per batch slower).  The row and e are read with plain loads: a
  // row spread over several tiles is re-read by each, and those re-reads come
  // from the last-level cache (non-temporal row loads: 80 against 73 us).
  const int64_t wb = static_cast<int64_t>(row) * v4;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (on[c]) store_nt(table + wb + col[c], f4_sub(m[c], f4_sub(m[c], e[c])));
}

// The rows a batch's row pass wrote, added to a written-row set (RES
// publishing): one thread per descriptor slot; a group with a row sets the
// row's flag, and the lanes that found it clear append the row to the list
// (one list atomic per wave).  A row in several tiles is several groups; its
// flag is set once, so it is listed once.
__global__ void __launch_bounds__(ml::kThreads)
    ml_mark_written(ml::Work w, int64_t num_rows, uint32_t *flags, int64_t *list, unsigned long long *list_count) {
  const int64_t g = static_cast<int64_t>(blockIdx.x) * ml::kThreads + threadIdx.x;
  const int64_t tile = g / ml::kTile;
  bool fresh = false;
  int64_t r = -1;
  if (tile < w.tiles && static_cast<uint32_t>(g % ml::kTile) < w.ntile[tile]) {
    const uint4 d = w.gdesc[g];
    if (!(d.w & ml::kNoRow) && static_cast<int64_t>(d.x) < num_rows) {
      r = d.x;
      fresh = atomicOr(&flags[r], 1u) == 0u;
    }
  }
  const uint64_t bal = ballot(fresh);
  if (bal == 0) return;
  const int leader = __builtin_ctzll(bal);
  unsigned long long base = 0;
  if (lane_id() == leader) base = atomicAdd(list_count, static_cast<unsigned long long>(__popcll(bal)));
  base = __shfl(base, leader);
  if (fresh) list[base + static_cast<unsigned long long>(__popcll(bal & lanemask_lt()))] = r;
}

}  // namespace

extern "C" hlr_status memory_layer_step_mark_written(const void *wb_ws, size_t wb_ws_bytes, int64_t n, int64_t n_max,
                                                     int64_t capacity, uint32_t *flags, int64_t *list,
                                                     int64_t *list_count, hipStream_t stream) {
  if (n < 0 || n > n_max || n_max > kMaxN || capacity <= 0) return HLR_INVALID_ARG;
  if (n == 0) return HLR_OK;
  if (!wb_ws || !flags || !list || !list_count) return HLR_INVALID_ARG;
  if (!aligned(wb_ws, 256) || !aligned(flags, 4) || !aligned(list, 8) || !aligned(list_count, 8))
    return HLR_MISALIGNED;
  ml::Work w;
  if (wb_ws_bytes < ml::layout(n_max, capacity, &w, const_cast<void *>(wb_ws))) return HLR_WORKSPACE_TOO_SMALL;
  w.tiles = (n + ml::kTile - 1) / ml::kTile;  // this batch's tiles
  ml_mark_written<<<grid_for(w.tiles * ml::kTile, ml::kThreads), ml::kThreads, 0, stream>>>(
      w, capacity, flags, list, reinterpret_cast<unsigned long long *>(list_count));
  return launch_status();
}

hlr_status hlr::ml_apply(float *values, int64_t num_rows, int64_t dim, const float *e, int64_t n, int64_t n_max,
                         float *out, void *ws, hipStream_t stream) {
  if (n == 0) return HLR_OK;
  ml::Work w;
  ml::layout(n_max, num_rows, &w, ws);
  w.tiles = (n + ml::kTile - 1) / ml::kTile;  // this batch's tiles
  const int64_t v4 = dim / 4;
  const int64_t nc = (v4 + kWave - 1) / kWave;
  // one wave per descriptor slot (a tile of kTile positions has at most kTile groups)
  const int grid = grid_for(w.tiles * ml::kTile, ml::kThreads / kWave);
  float4 *t4 = reinterpret_cast<float4 *>(values);
  const float4 *e4 = reinterpret_cast<const float4 *>(e);
  float4 *o4 = reinterpret_cast<float4 *>(out);
  if (nc == 1) ml_fused<1><<<grid, ml::kThreads, 0, stream>>>(t4, e4, o4, v4, w);
  else if (nc == 2) ml_fused<2><<<grid, ml::kThreads, 0, stream>>>(t4, e4, o4, v4, w);
  else ml_fused<4><<<grid, ml::kThreads, 0, stream>>>(t4, e4, o4, v4, w);
  return launch_status();
}
