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
// A row's sum is one fp32 running sum per element over its positions in batch
// order.  Positions are grouped by row with a stable radix sort (radix.hpp),
// and the plan lists the rows of kChainMin (512) or more occurrences by
// length.  Rows with fewer occurrences are summed by one wave each (light
// part: 8 positions per round trip, so such a row takes at most about 64 of
// them).  A longer row is one dependent chain per element: every (row,
// 16-element slice) is a block of four waves, one element per 16-lane row,
// walking the row's positions in order with 16 positions per load
// instruction (chain_sum16), so a Zipf-hot row (tens of thousands of
// duplicates) spreads over many CUs while each element's sum keeps its order.
// Both parts run in one launch (sgd_apply_kernel): a few heavy blocks per
// update first, longest rows first, so the long chains start at once; the
// light rows, which carry most of the bytes, stream beside them on the rest
// of the GPU.  The launch takes up to eight independent updates (distinct
// tables) at once.
//
// L2_ALIGN — the alternative to Writeback that the same Memory Layer section
// compares: SGD on ||M[r] - sg(e_i)||^2, i.e. the gradient 2 (M[r] - e_i) per
// occurrence at the row's value before the batch, summed and applied as in
// SGD_SUM (same kernels, the gradient formed on the fly from M and e).
#include "radix.hpp"
#include "step_parts.hpp"

namespace {
using namespace hlr;

constexpr int kThreads = 256;

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

// Distinct rows of a LAST_WINS plan (list order), for callers that publish
// the rows a batch wrote.
__global__ void __launch_bounds__(kThreads)
    lw_rows(LWWork w, int64_t n, int64_t *__restrict__ out_rows, int64_t *__restrict__ out_count) {
  const uint32_t count = *w.count;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i < count && i < n) out_rows[i] = w.hkey[w.list[i]];
  if (i == 0) *out_count = count;
}

// One wave per winner row (two rows in flight per wave): g = fl(M - e), M' = fl(M - g).
// fresh (nullable): a row whose last position has fresh[p] == 0 was inserted by
// this batch's lookup and not cleared; it is taken as zero (M = 0) instead of
// being read.
template <int NC>
__global__ void __launch_bounds__(kThreads)
    lw_apply(float4 *table, const float4 *__restrict__ src, const int8_t *__restrict__ fresh, LWWork w, int64_t v4) {
  constexpr int RPW = 2;
  const uint32_t count = *w.count;
  const int lane = lane_id();
  const uint32_t waves = gridDim.x * (kThreads / kWave);
  for (uint32_t j0 = ((blockIdx.x * kThreads + threadIdx.x) / kWave) * RPW; j0 < count; j0 += waves * RPW) {
    int64_t mrow[RPW], erow[RPW];
    bool zero[RPW];
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      mrow[q] = -1;
      zero[q] = false;
      if (j0 + q < count) {
        const int32_t s = w.list[j0 + q];
        const int32_t p = w.hlast[s];
        mrow[q] = w.hkey[s] * v4;
        erow[q] = static_cast<int64_t>(p) * v4;
        if (fresh) zero[q] = fresh[p] == 0;
      }
    }
    float4 m[RPW][NC], e[RPW][NC];
#pragma unroll
    for (int q = 0; q < RPW; ++q)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int64_t col = lane + c * kWave;
        if (mrow[q] >= 0 && col < v4) {
          e[q][c] = src[erow[q] + col];
          m[q][c] = zero[q] ? make_float4(0.f, 0.f, 0.f, 0.f) : table[mrow[q] + col];
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

// Duplicate-summed SGD: a wave sums a run of a row's gradients in batch order
// (lanes own 16-byte column units), acc = g[spos[j0]], then acc += g[spos[j]].
// L2 = true is the L2-alignment update: the source holds targets e_i and each
// occurrence's gradient is fl(2 * fl(M - e_i)) with M the row before the batch
// (the doubling is exact); everything else is as for SGD_SUM.
template <int NC>
constexpr int light_batch() { return NC == 4 ? 4 : 8; }

__device__ __forceinline__ float4 l2_grad(float4 m, float4 e) {
  const float4 d = f4_sub(m, e);
  return make_float4(2.f * d.x, 2.f * d.y, 2.f * d.z, 2.f * d.w);
}

__device__ __forceinline__ float l2_grad(float m, float e) { return 2.f * (m - e); }

template <int NC, bool L2>
__device__ __forceinline__ void sum_run(const float4 *__restrict__ g, const uint32_t *__restrict__ spos, int32_t j0,
                                        int32_t j1, int64_t v4, int lane, const float4 (&m)[NC], float4 (&acc)[NC]) {
  rows_run<light_batch<NC>(), NC>(g, spos, j0, j1, v4, lane, [&](int32_t j, const float4(&x)[NC]) {
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      const float4 y = L2 ? l2_grad(m[q], x[q]) : x[q];
      acc[q] = j == j0 ? y : make_float4(acc[q].x + y.x, acc[q].y + y.y, acc[q].z + y.z, acc[q].w + y.w);
    }
  });
}

// Light rows (fewer than kChainMin occurrences): one wave per row; the row
// is read once, before its gradients, and written once: fl(M - fl(lr * s)).  Longer rows belong to the heavy part.  A wave walks
// rows k, k + waves, ...; the next row's (start, end, row) is loaded while the
// current row is processed (wave-uniform, so scalar loads).
template <int NC, bool L2>
__device__ __forceinline__ void sgd_light(float4 *table, const float4 *__restrict__ g,
                                          const uint32_t *__restrict__ seg_key, const uint32_t *__restrict__ spos,
                                          const int32_t *__restrict__ seg_start, const int32_t *__restrict__ seg_end,
                                          const int64_t *__restrict__ nseg_p, float lr, int64_t v4, int block,
                                          int nblocks) {
  const int64_t nseg = *nseg_p;
  const int64_t waves = static_cast<int64_t>(nblocks) * (kThreads / kWave);
  const int lane = lane_id();
  int64_t k = __builtin_amdgcn_readfirstlane(static_cast<int>((block * kThreads + threadIdx.x) / kWave));
  if (k >= nseg) return;
  int32_t s = seg_start[k], e = seg_end[k];
  int64_t r = seg_key[k];
  for (;;) {
    const int64_t kn = k + waves;
    const int64_t kc = kn < nseg ? kn : nseg - 1;
    const int32_t sn = seg_start[kc], en = seg_end[kc];
    const int64_t rn = seg_key[kc];
    if (e - s < kChainMin) {
      float4 m[NC], run[NC];
#pragma unroll
      for (int q = 0; q < NC; ++q) {
        const int64_t c = lane + q * kWave;
        m[q] = table[r * v4 + (c < v4 ? c : 0)];
      }
      sum_run<NC, L2>(g, spos, s, e, v4, lane, m, run);
#pragma unroll
      for (int q = 0; q < NC; ++q) {
        const int64_t c = lane + q * kWave;
        const float4 st = make_float4(lr * run[q].x, lr * run[q].y, lr * run[q].z, lr * run[q].w);
        if (c < v4) table[r * v4 + c] = f4_sub(m[q], st);  // fl(M - fl(lr * s))
      }
    }
    if (kn >= nseg) break;
    k = kn;
    s = sn;
    e = en;
    r = rn;
  }
}

// Heavy rows: one block of four waves per (row, 16-element slice); wave w
// takes elements 16 * slice + 4w + r in its rows r = 0..3, each one chain over
// all the row's positions in batch order (chain_sum16), then lane 0 of the row
// writes fl(M - fl(lr * s)).  24 load instructions (384 positions) a batch:
// one hot row of 24,576 occurrences at dim 512 alone took 19.8 ns per position
// with 48 and 14.8 with 24 (12-16: no faster), and the hashed-tables apply
// 531-553 us against 561-574 (with the light rows beside them the heavy part is
// bound by its random 64-byte reads, not by the chain: with the light rows
// skipped it still takes about 510 us).  Blocks take items in the plan's order, longest
// rows first.  L2: every gradient is taken at the row before the batch, which
// no block writes before its own chain has read it (one block per element).
constexpr int kHeavyBatch = 24;  // load instructions per batch of the heavy walk

template <bool L2, bool Off32>
__device__ __forceinline__ void sgd_heavy(float *table, const float *__restrict__ g,
                                          const uint32_t *__restrict__ skey, const uint32_t *__restrict__ spos,
                                          const int32_t *__restrict__ seg_start, const int32_t *__restrict__ seg_end,
                                          uint32_t *counters, const int32_t *__restrict__ slist,
                                          int64_t n, float lr, int64_t D, int nblocks) {
  const int64_t S = (D + 15) / 16;
  uint32_t cnt[kLenBuckets];
  int64_t items = 0;
#pragma unroll
  for (int b = 0; b < kLenBuckets; ++b) {
    cnt[b] = counters[4 + b];
    items += static_cast<int64_t>(cnt[b]) * S;
  }
  const int wv = static_cast<int>(threadIdx.x) / kWave;
  const int r = lane_id() / 16;
  __shared__ __align__(16) float lds[kThreads / kWave][kChainSlots * 64];
  __shared__ uint32_t sh_it;
  // Items (segment, slice), longest segments first, go to the blocks as they
  // come free (counters[2]), so a block that drew a short chain takes the
  // next one while the longest runs: the apply ends with the longest chain,
  // not with the block that drew the most work.
  for (;;) {
    if (threadIdx.x == 0) sh_it = atomicAdd(&counters[2], 1u);
    __syncthreads();
    const int64_t it = sh_it;
    __syncthreads();
    if (it >= items) break;
    int32_t k;
    int64_t slice;
    heavy_item(cnt, slist, n, S, it, &k, &slice);
    const int64_t el = slice * 16 + 4 * wv + r;
    const int32_t s = seg_start[k], end = seg_end[k];
    const int64_t at = static_cast<int64_t>(skey[s]) * D + (el < D ? el : 0);
    const float mv = table[at];
    const float acc =
        chain_sum16<kHeavyBatch, Off32>(g, spos, s, end, D, el, lds[wv], [&](float x) { return L2 ? l2_grad(mv, x) : x; });
    if ((lane_id() & 15) == 0 && el < D) {
      const float st = lr * acc;
      table[at] = mv - st;  // fl(M - fl(lr * s))
    }
  }
  // The last heavy block of the update to finish drawing returns both
  // counters to zero (counters[3] counts the blocks done), so the plan can be
  // applied again.
  if (threadIdx.x == 0 && atomicAdd(&counters[3], 1u) == static_cast<uint32_t>(nblocks - 1)) {
    counters[2] = 0u;
    counters[3] = 0u;
  }
}

// One update (table, gradients, plan) of a launch, and the blocks it owns.
struct SgdJob {
  float *table;
  const float *g;
  const uint32_t *seg_key, *skey, *spos;
  const int32_t *seg_start, *seg_end;
  const int64_t *nseg;
  uint32_t *counters;
  const int32_t *slist;
  int64_t n;
  float lr;
  int heavy_begin, heavy_blocks, light_begin, light_blocks;
};

// Independent updates (distinct tables) applied by one launch: the heavy
// blocks of every update first (their runs start at once), then the light
// blocks of every update.  The parts and the updates touch disjoint rows.
constexpr int kMaxSgdJobs = 8;
struct SgdJobs {
  SgdJob job[kMaxSgdJobs];
  int count;
  int64_t D;
};

template <int NC, bool L2, bool Off32>
__global__ void __launch_bounds__(kThreads) sgd_apply_kernel(SgdJobs js) {
  const int blk = static_cast<int>(blockIdx.x);
  for (int i = 0; i < js.count; ++i) {
    const SgdJob &j = js.job[i];
    if (blk >= j.heavy_begin && blk < j.heavy_begin + j.heavy_blocks) {
      sgd_heavy<L2, Off32>(j.table, j.g, j.skey, j.spos, j.seg_start, j.seg_end, j.counters, j.slist, j.n, j.lr,
                           js.D, j.heavy_blocks);
      return;
    }
    if (blk >= j.light_begin && blk < j.light_begin + j.light_blocks) {
      sgd_light<NC, L2>(reinterpret_cast<float4 *>(j.table), reinterpret_cast<const float4 *>(j.g), j.seg_key,
                        j.spos, j.seg_start, j.seg_end, j.nseg, j.lr, js.D / 4, blk - j.light_begin,
                        j.light_blocks);
      return;
    }
  }
}

// The job of one SGD_SUM / L2_ALIGN update: its plan's buffers in ws and its block counts.
SgdJob sgd_job(float *table, const float *g, int64_t n, int64_t dim, float lr, void *ws, int64_t num_rows) {
  SegWork<uint32_t> w;
  segwork_layout<uint32_t>(n, &w, ws);
  const int cur = sorted_buffer(num_rows);
  SgdJob j{};
  j.table = table;
  j.g = g;
  j.seg_key = w.seg_key;
  j.skey = w.k[cur];
  j.spos = w.v[cur];
  j.seg_start = w.seg_start;
  j.seg_end = w.seg_end;
  j.nseg = w.nseg;
  j.counters = w.ticket;
  j.slist = w.slist;
  j.n = n;
  j.lr = lr;
  // heavy blocks hold 4 waves of about 120 registers each; 128 per update
  // leave most of the GPU to the light rows that stream beside them
  const int gl = grid_for(n, 4 * 4), gh = grid_for(n, 1024);
  j.light_blocks = gl < 4096 ? gl : 4096;
  j.heavy_blocks = gh < 128 ? gh : 128;
  return j;
}

// A gradient array whose byte offsets fit the 31-bit range of a buffer resource.
inline bool off32_ok(int64_t n, int64_t dim) { return n * dim * 4 < (int64_t(1) << 31); }

// One launch for up to kMaxSgdJobs updates of one dim and mode: heavy blocks
// of every job, then light blocks of every job.
template <bool L2>
void sgd_launch(SgdJobs &js, hipStream_t s) {
  int next = 0;
  bool off32 = true;
  for (int i = 0; i < js.count; ++i) {
    js.job[i].heavy_begin = next;
    next += js.job[i].heavy_blocks;
    off32 = off32 && off32_ok(js.job[i].n, js.D);
  }
  for (int i = 0; i < js.count; ++i) {
    js.job[i].light_begin = next;
    next += js.job[i].light_blocks;
  }
  if (next == 0) return;
  const int64_t nc = (js.D / 4 + kWave - 1) / kWave;
#define HLR_SGD_LAUNCH(NC, O32) sgd_apply_kernel<NC, L2, O32><<<next, kThreads, 0, s>>>(js)
  if (off32) {
    if (nc == 1) HLR_SGD_LAUNCH(1, true);
    else if (nc == 2) HLR_SGD_LAUNCH(2, true);
    else HLR_SGD_LAUNCH(4, true);
  } else {
    if (nc == 1) HLR_SGD_LAUNCH(1, false);
    else if (nc == 2) HLR_SGD_LAUNCH(2, false);
    else HLR_SGD_LAUNCH(4, false);
  }
#undef HLR_SGD_LAUNCH
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

namespace {

hlr_status wb_args(int64_t num_rows, int64_t n, int32_t mode) {
  if (n < 0 || n > kMaxN || num_rows < 0 || num_rows >= 0x7fffffff) return HLR_INVALID_ARG;
  if (mode != HLR_WB_LAST_WINS && mode != HLR_WB_SGD_SUM && mode != HLR_WB_L2_ALIGN) return HLR_INVALID_ARG;
  return HLR_OK;
}

hlr_status ws_check(void *ws, size_t ws_bytes, size_t need) {
  if (!ws || ws_bytes < need) return HLR_WORKSPACE_TOO_SMALL;
  if (!aligned(ws, 256)) return HLR_MISALIGNED;
  return HLR_OK;
}

// Plan: depends on rows only.  LAST_WINS: the row -> last position table and
// its compact list; SGD_SUM: positions grouped by row (sort + segments).
void wb_plan(int64_t num_rows, const int64_t *rows, int64_t n, int32_t mode, void *ws, hipStream_t stream) {
  if (mode == HLR_WB_LAST_WINS) {
    LWWork w;
    lw_layout(n, &w, ws);
    int gi = grid_for(w.cap, kThreads);
    if (gi > 4096) gi = 4096;
    lw_init<<<gi, kThreads, 0, stream>>>(w);
    lw_last<<<grid_for(n, kLwTile), kThreads, 0, stream>>>(rows, n, num_rows, w);
    return;
  }
  SegWork<uint32_t> w;
  segwork_layout<uint32_t>(n, &w, ws);
  group_by_row(w, rows, nullptr, num_rows, stream);
  list_heavy_segments(w, stream);
}

// Apply: reads the plan left in the workspace by wb_plan.
void wb_apply(float *table, int64_t num_rows, int64_t dim, const float *src, int64_t n, int32_t mode, float lr,
              void *ws, hipStream_t stream, const int8_t *fresh = nullptr) {
  const int64_t v4 = dim / 4;
  const int64_t nc = (v4 + kWave - 1) / kWave;
  if (mode == HLR_WB_LAST_WINS) {
    LWWork w;
    lw_layout(n, &w, ws);
    int ga = grid_for(n, 8);
    if (ga > 2048) ga = 2048;
    float4 *t4 = reinterpret_cast<float4 *>(table);
    const float4 *s4 = reinterpret_cast<const float4 *>(src);
    if (nc == 1) lw_apply<1><<<ga, kThreads, 0, stream>>>(t4, s4, fresh, w, v4);
    else if (nc == 2) lw_apply<2><<<ga, kThreads, 0, stream>>>(t4, s4, fresh, w, v4);
    else lw_apply<4><<<ga, kThreads, 0, stream>>>(t4, s4, fresh, w, v4);
    return;
  }
  SgdJobs js{};
  js.count = 1;
  js.D = dim;
  js.job[0] = sgd_job(table, src, n, dim, lr, ws, num_rows);
  if (mode == HLR_WB_L2_ALIGN) sgd_launch<true>(js, stream);
  else sgd_launch<false>(js, stream);
}

}  // namespace

extern "C" hlr_status writeback_rows(float *table, int64_t num_rows, int64_t dim, const int64_t *rows,
                                     const float *src, int64_t n, int32_t mode, float lr, void *ws, size_t ws_bytes,
                                     hipStream_t stream) {
  hlr_status st = wb_args(num_rows, n, mode);
  if (st != HLR_OK) return st;
  if (mode == HLR_WB_LAST_WINS && lr != 1.0f) return HLR_INVALID_ARG;
  if (dim <= 0 || dim % 4 != 0 || dim > 1024) return HLR_UNSUPPORTED_DIM;
  if (n == 0 || num_rows == 0) return HLR_OK;
  if (!table || !rows || !src) return HLR_INVALID_ARG;
  if (!aligned(table, 16) || !aligned(src, 16) || !aligned(rows, 8)) return HLR_MISALIGNED;
  if ((st = ws_check(ws, ws_bytes, writeback_rows_workspace_size(num_rows, dim, n, mode))) != HLR_OK) return st;
  wb_plan(num_rows, rows, n, mode, ws, stream);
  wb_apply(table, num_rows, dim, src, n, mode, lr, ws, stream);
  return launch_status();
}

extern "C" hlr_status writeback_plan(int64_t num_rows, const int64_t *rows, int64_t n, int32_t mode, void *ws,
                                     size_t ws_bytes, hipStream_t stream) {
  hlr_status st = wb_args(num_rows, n, mode);
  if (st != HLR_OK) return st;
  if (n == 0 || num_rows == 0) return HLR_OK;
  if (!rows) return HLR_INVALID_ARG;
  if (!aligned(rows, 8)) return HLR_MISALIGNED;
  if ((st = ws_check(ws, ws_bytes, writeback_rows_workspace_size(num_rows, 4, n, mode))) != HLR_OK) return st;
  wb_plan(num_rows, rows, n, mode, ws, stream);
  return launch_status();
}

extern "C" hlr_status writeback_apply(float *table, int64_t num_rows, int64_t dim, const float *src, int64_t n,
                                      int32_t mode, float lr, void *ws, size_t ws_bytes, hipStream_t stream) {
  hlr_status st = wb_args(num_rows, n, mode);
  if (st != HLR_OK) return st;
  if (mode == HLR_WB_LAST_WINS && lr != 1.0f) return HLR_INVALID_ARG;
  if (dim <= 0 || dim % 4 != 0 || dim > 1024) return HLR_UNSUPPORTED_DIM;
  if (n == 0 || num_rows == 0) return HLR_OK;
  if (!table || !src) return HLR_INVALID_ARG;
  if (!aligned(table, 16) || !aligned(src, 16)) return HLR_MISALIGNED;
  if ((st = ws_check(ws, ws_bytes, writeback_rows_workspace_size(num_rows, dim, n, mode))) != HLR_OK) return st;
  wb_apply(table, num_rows, dim, src, n, mode, lr, ws, stream);
  return launch_status();
}

hlr_status hlr::writeback_apply_last_fresh(float *table, int64_t num_rows, int64_t dim, const float *src, int64_t n,
                                           const int8_t *hit, void *ws, size_t ws_bytes, hipStream_t stream) {
  hlr_status st = wb_args(num_rows, n, HLR_WB_LAST_WINS);
  if (st != HLR_OK) return st;
  if (dim <= 0 || dim % 4 != 0 || dim > 1024) return HLR_UNSUPPORTED_DIM;
  if (n == 0 || num_rows == 0) return HLR_OK;
  if (!table || !src || !hit) return HLR_INVALID_ARG;
  if (!aligned(table, 16) || !aligned(src, 16)) return HLR_MISALIGNED;
  if ((st = ws_check(ws, ws_bytes, writeback_rows_workspace_size(num_rows, dim, n, HLR_WB_LAST_WINS))) != HLR_OK)
    return st;
  wb_apply(table, num_rows, dim, src, n, HLR_WB_LAST_WINS, 1.0f, ws, stream, hit);
  return launch_status();
}

extern "C" hlr_status writeback_apply_batch(int32_t count, const hlr_wb_apply *updates, int32_t mode,
                                            hipStream_t stream) {
  if (count < 0 || count > kMaxSgdJobs || (count > 0 && !updates)) return HLR_INVALID_ARG;
  if (mode != HLR_WB_SGD_SUM && mode != HLR_WB_L2_ALIGN) return HLR_INVALID_ARG;
  SgdJobs js{};
  js.D = 0;
  for (int32_t i = 0; i < count; ++i) {
    const hlr_wb_apply &u = updates[i];
    hlr_status st = wb_args(u.num_rows, u.n, mode);
    if (st != HLR_OK) return st;
    if (u.dim <= 0 || u.dim % 4 != 0 || u.dim > 1024) return HLR_UNSUPPORTED_DIM;
    if (u.n == 0 || u.num_rows == 0) continue;
    if (!u.table || !u.src) return HLR_INVALID_ARG;
    if (!aligned(u.table, 16) || !aligned(u.src, 16)) return HLR_MISALIGNED;
    const size_t wb = writeback_rows_workspace_size(u.num_rows, u.dim, u.n, mode);
    if ((st = ws_check(u.ws, u.ws_bytes, wb)) != HLR_OK) return st;
    if (js.D != 0 && u.dim != js.D) return HLR_INVALID_ARG;  // one dim per launch
    js.D = u.dim;
    const size_t tb = static_cast<size_t>(u.num_rows) * static_cast<size_t>(u.dim) * sizeof(float);
    for (int32_t k = 0; k < i; ++k) {  // the updates run at once: no shared table or workspace
      const hlr_wb_apply &v = updates[k];
      if (v.n == 0 || v.num_rows == 0) continue;
      const size_t vb = static_cast<size_t>(v.num_rows) * static_cast<size_t>(v.dim) * sizeof(float);
      const char *ut = reinterpret_cast<const char *>(u.table), *vt = reinterpret_cast<const char *>(v.table);
      const char *uw = static_cast<const char *>(u.ws), *vw = static_cast<const char *>(v.ws);
      const size_t vwb = writeback_rows_workspace_size(v.num_rows, v.dim, v.n, mode);
      if ((ut < vt + vb && vt < ut + tb) || (uw < vw + vwb && vw < uw + wb)) return HLR_INVALID_ARG;
    }
    js.job[js.count++] = sgd_job(u.table, u.src, u.n, u.dim, u.lr, u.ws, u.num_rows);
  }
  if (js.count == 0) return HLR_OK;
  if (mode == HLR_WB_L2_ALIGN) sgd_launch<true>(js, stream);
  else sgd_launch<false>(js, stream);
  return launch_status();
}

extern "C" hlr_status writeback_plan_rows(int64_t num_rows, int64_t n, const void *ws, size_t ws_bytes,
                                          int64_t *out_rows, int64_t *out_count, hipStream_t stream) {
  hlr_status st = wb_args(num_rows, n, HLR_WB_LAST_WINS);
  if (st != HLR_OK) return st;
  if (!out_count) return HLR_INVALID_ARG;
  if (n > 0 && !out_rows) return HLR_INVALID_ARG;
  if ((out_rows && !aligned(out_rows, 8)) || !aligned(out_count, 8)) return HLR_MISALIGNED;
  if (n == 0 || num_rows == 0) {
    hlr_fill(out_count, 1, int64_t(0), stream);
    return launch_status();
  }
  if ((st = ws_check(const_cast<void *>(ws), ws_bytes, writeback_rows_workspace_size(num_rows, 4, n,
                                                                                     HLR_WB_LAST_WINS))) != HLR_OK)
    return st;
  LWWork w;
  lw_layout(n, &w, const_cast<void *>(ws));
  lw_rows<<<grid_for(n, kThreads), kThreads, 0, stream>>>(w, n, out_rows, out_count);
  return launch_status();
}
