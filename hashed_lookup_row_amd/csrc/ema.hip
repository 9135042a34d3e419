// EMA row updates ("CS3: Efficient Online Capability Synergy for Two-Tower
// Recommendation", sec. 2): CTS keeps c <- a*c + (1-a)*v for positive
// interactions only (mask = labels), CMS keeps s <- b*s + (1-b)*h for every
// interaction (mask = NULL).  Duplicates of a row are applied in batch order.
//
// Plan: positions that take part are grouped by row with a stable radix sort
// (radix.hpp), so each row's positions come out in batch order.  A row's
// positions are applied in order (T = fl(fl(a*T) + fl(b*v))): short rows by
// one wave each (light part), long rows by one wave per (chunk, 32-element
// slice), the chunks of a row running in parallel from speculative
// warmed-up states (heavy part) that ema_combine verifies bit for bit.  The
// result equals the sequential loop bit for bit.  The plan lists the long
// rows' runs, so one launch (ema_apply_kernel) holds both parts, for up to
// four independent updates at once: its first blocks start the long dependent
// chains of every update and the rest stream the short rows beside them; one
// more launch (ema_combine_kernel) finishes the rows cut into chunks.  A plan
// for a subset of another plan's positions (ema_update_plan_subset) is cut out
// of that plan's sorted pairs instead of being sorted again.
#include <cmath>

#include "radix.hpp"

namespace {
using namespace hlr;

constexpr int kThreads = 256;

__device__ __forceinline__ float4 ema_step(float4 t, float4 v, float a, float b) {
  return make_float4(a * t.x + b * v.x, a * t.y + b * v.y, a * t.z + b * v.z, a * t.w + b * v.w);
}

// Row loads in flight per wave in the light part.  The launch's register
// budget is set by the heavy part's slice walk (about 117 registers, four
// waves per SIMD), so the light rows at dim <= 256 keep 16 rows in flight per
// wave to make up for the lower occupancy.
template <int NC>
constexpr int light_batch() { return NC == 4 ? 4 : (NC == 2 ? 8 : 16); }

// Light rows (fewer than kHeavyMin occurrences): one wave per row, exact.  A
// wave walks rows k, k + waves, ...; the next row's (start, end, row) is loaded
// while the current row is processed (wave-uniform, so scalar loads).  Longer
// rows belong to the heavy part.
template <int NC>
__device__ __forceinline__ void ema_light(float4 *table0, const float4 *__restrict__ vals0, float4 *table1,
                                          const float4 *__restrict__ vals1, uint32_t split,
                                          const uint32_t *__restrict__ seg_key, const uint32_t *__restrict__ spos,
                                          const int32_t *__restrict__ seg_start, const int32_t *__restrict__ seg_end,
                                          const int64_t *__restrict__ nseg_p, float a, float b, int64_t v4,
                                          int block, int nblocks) {
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
    if (e - s < kHeavyMin) {
      // a pair plan's keys from split on are rows of the second table
      const bool second = r >= split;
      float4 *table = second ? table1 : table0;
      const float4 *vals = second ? vals1 : vals0;
      if (second) r -= split;
      float4 st[NC];
#pragma unroll
      for (int q = 0; q < NC; ++q) {
        const int64_t c = lane + q * kWave;
        st[q] = table[r * v4 + (c < v4 ? c : 0)];
      }
      rows_run<light_batch<NC>(), NC>(vals, spos, s, e, v4, lane, [&](int32_t, const float4(&x)[NC]) {
#pragma unroll
        for (int q = 0; q < NC; ++q) st[q] = ema_step(st[q], x[q], a, b);
      });
#pragma unroll
      for (int q = 0; q < NC; ++q) {
        const int64_t c = lane + q * kWave;
        if (c < v4) table[r * v4 + c] = st[q];
      }
    }
    if (kn >= nseg) break;
    k = kn;
    s = sn;
    e = en;
    r = rn;
  }
}

__device__ __forceinline__ float ema1(float t, float v, float a, float b) { return a * t + b * v; }

// A heavy chunk is one dependent chain per element, so its speed is set by how
// many of its positions are requested ahead, and by how well its scattered
// value reads use the lines they fetch: its waves walk 32-element slices (one
// 128-byte line of a position's value row), two positions per load
// instruction, 48 instructions (96 positions) a batch, which keeps the launch
// at 117 registers and four waves per SIMD (56 instructions: 125-133
// registers, three waves per SIMD, 183 us).  Measured on the CS3 step's
// batched apply (four updates, dim 128): 164 us, against 183 us with
// 16-element slices (four positions per instruction, each fetching half a
// line that another wave fetches again) and 8-element slices for the longest
// chunks, and 200 us with 64-element slices (one position per instruction).
constexpr int kHeavyG = 2;  // lane groups (positions per load instruction)
constexpr int kHeavyP = 48;

// Heavy rows: one wave per (chunk of <= L occurrences, 32-element slice).  A
// row with one chunk is applied exactly from its stored value.  For a longer
// row, chunk 0 runs exactly; chunk m > 0 starts W occurrences early from a zero
// state (the recurrence contracts by a per step, so after W steps the state no
// longer depends on where it started) and records sigma (the state entering
// its first occurrence) and tau (the state after its last) for ema_combine.
// The plan lists runs of kBaseRun; a chunk is L / kBaseRun of them, and the
// wave of a run that does not start a chunk has nothing to do.
template <int G, bool Off32>
__device__ __forceinline__ void ema_heavy(float *table0, const float *__restrict__ vals0, float *table1,
                                          const float *__restrict__ vals1, uint32_t split,
                                          const uint32_t *__restrict__ skey, const uint32_t *__restrict__ spos,
                                          const int32_t *__restrict__ seg_start, const int32_t *__restrict__ seg_end,
                                          const uint32_t *__restrict__ counters, const int2 *__restrict__ hlist,
                                          float a, float b, int64_t D, int L, int W, float *partial, int block,
                                          int nblocks) {
  using HeavySlices = Narrow<G>;
  const int64_t S = HeavySlices::slices(D);
  const int64_t items = static_cast<int64_t>(counters[0]) * S;
  const int64_t waves = static_cast<int64_t>(nblocks) * (kThreads / kWave);
  const int32_t per_chunk = L / kBaseRun;
  for (int64_t it = (static_cast<int64_t>(block) * kThreads + threadIdx.x) / kWave; it < items; it += waves) {
    const int2 km = hlist[it / S];
    if (km.y % per_chunk != 0) continue;
    const int32_t m = km.y / per_chunk;
    const int lane = lane_id();
    const int64_t e = (it % S) * HeavySlices::kWidth + (lane % HeavySlices::kWidth);
    const bool act = lane < HeavySlices::kWidth && e < D;  // lane group 0 holds the chain
    const int32_t s = seg_start[km.x], end = seg_end[km.x];
    const uint32_t key = skey[s];
    const bool second = key >= split;  // a pair plan's row of the second table
    float *table = second ? table1 : table0;
    const float *vals = second ? vals1 : vals0;
    const int64_t r = second ? key - split : key;
    const int32_t j0 = s + m * L;
    const int32_t j1 = static_cast<int64_t>(j0) + L < end ? j0 + L : end;
    const bool exact_start = m == 0 || j0 - W <= s;
    const int32_t from = exact_start ? s : j0 - W;
    float st = (exact_start && act) ? table[r * D + e] : 0.f;
    // A row in one chunk is walked whole.  Otherwise the warm-up (or the exact
    // prefix) is walked first and the chunk second; sigma is the state between
    // them.  (One call site for both walks keeps the kernel's code small.)
    const bool whole = end - s <= L;
    int32_t w0 = whole ? s : from, w1 = whole ? end : j0;
    float sig = st;
    for (int k = 0; k < 2; ++k) {
      slice_run_narrow<G, kHeavyP, Off32>(vals, spos, w0, w1, D, e, [&](int32_t, float x) { st = ema1(st, x, a, b); });
      if (k == 0) {
        sig = st;
        w0 = w1;
        w1 = whole ? w1 : j1;
      }
    }
    if (whole) {
      if (act) table[r * D + e] = st;
      continue;
    }
    if (act) {
      const int64_t slot = run_slot(j0, m, L);
      partial[(2 * slot) * D + e] = sig;
      partial[(2 * slot + 1) * D + e] = st;
    }
  }
}

// One update (table, values, plan) of a launch, and the blocks it owns.
struct EmaJob {
  float *table;
  const float *vals;
  float *table1;        // a pair plan: keys from split on are rows of table1, valued by vals1
  const float *vals1;
  uint32_t split;       // 0xffffffff: one table
  const uint32_t *seg_key, *skey, *spos;
  const int32_t *seg_start, *seg_end;
  const int64_t *nseg;
  const uint32_t *counters;
  const int2 *hlist;
  const int32_t *clist;
  float *partial;
  int64_t n;  // positions (rows of vals)
  float a, b;
  int L, W;
  int heavy_begin, heavy_blocks, light_begin, light_blocks, comb_begin, comb_blocks;
};

// Independent updates (distinct tables) applied by one launch: a launch holds
// the heavy blocks of every update first (so all the long chains start at
// once), then the light blocks of every update, which stream beside them.
constexpr int kMaxEmaJobs = 4;
struct EmaJobs {
  EmaJob job[kMaxEmaJobs];
  int count;
  int64_t D;
};

// Off32: every update's values are under 2 GiB (32-bit offsets in the heavy walk).
template <int NC, bool Off32>
__global__ void __launch_bounds__(kThreads) ema_apply_kernel(EmaJobs js) {
  const int blk = static_cast<int>(blockIdx.x);
  for (int i = 0; i < js.count; ++i) {
    const EmaJob &j = js.job[i];
    if (blk >= j.heavy_begin && blk < j.heavy_begin + j.heavy_blocks) {
      ema_heavy<kHeavyG, Off32>(j.table, j.vals, j.table1, j.vals1, j.split, j.skey, j.spos, j.seg_start, j.seg_end, j.counters, j.hlist, j.a,
                                j.b, js.D, j.L, j.W, j.partial, blk - j.heavy_begin, j.heavy_blocks);
      return;
    }
    if (blk >= j.light_begin && blk < j.light_begin + j.light_blocks) {
      ema_light<NC>(reinterpret_cast<float4 *>(j.table), reinterpret_cast<const float4 *>(j.vals),
                    reinterpret_cast<float4 *>(j.table1), reinterpret_cast<const float4 *>(j.vals1), j.split,
                    j.seg_key, j.spos,
                    j.seg_start, j.seg_end, j.nseg, j.a, j.b, js.D / 4, blk - j.light_begin, j.light_blocks);
      return;
    }
  }
}

// Rows with several chunks: one wave per (row, slice) walks the chunks in
// order.  If sigma_m equals the exact state entering chunk m bit for bit, tau_m
// is exact; otherwise chunk m is recomputed from the exact state.  The result
// equals the sequential loop bit for bit in every case; speculation only
// decides how much ran in parallel.  sigma and tau do not depend on the walk,
// so they are loaded kCombineBatch chunks at a time ahead of it.
constexpr int kCombineBatch = 16;

__device__ __forceinline__ void ema_combine(float *table0, const float *__restrict__ vals0, float *table1,
                                            const float *__restrict__ vals1, uint32_t split,
                                            const uint32_t *__restrict__ skey, const uint32_t *__restrict__ spos,
                                            const int32_t *__restrict__ seg_start,
                                            const int32_t *__restrict__ seg_end,
                                            const uint32_t *__restrict__ counters,
                                            const int32_t *__restrict__ clist, float a, float b, int64_t D, int L,
                                            const float *__restrict__ partial, int block, int nblocks) {
  const int64_t S = num_slices(D);
  const int64_t items = static_cast<int64_t>(counters[1]) * S;
  const int64_t waves = static_cast<int64_t>(nblocks) * (kThreads / kWave);
  for (int64_t it = (static_cast<int64_t>(block) * kThreads + threadIdx.x) / kWave; it < items; it += waves) {
    const int32_t k = clist[it / S];
    const int32_t s = seg_start[k], end = seg_end[k];
    if (end - s <= L) continue;  // one chunk: walked whole by the heavy part
    const uint32_t key = skey[s];
    const bool second = key >= split;  // a pair plan's row of the second table
    float *table = second ? table1 : table0;
    const float *vals = second ? vals1 : vals0;
    const int64_t row = second ? key - split : key;
    const int64_t e = (it % S) * kSliceElems + lane_id();
    const bool act = e < D;
    const int64_t ec = act ? e : 0;
    const int32_t nch = static_cast<int32_t>((static_cast<int64_t>(end - s) + L - 1) / L);
    auto slot2 = [&](int32_t m) { return partial + 2 * run_slot(s + m * L, m, L) * D; };
    float cur = slot2(0)[D + ec];
    int32_t m = 1;
    while (m < nch) {
      float sg[kCombineBatch], tau[kCombineBatch];
#pragma unroll
      for (int u = 0; u < kCombineBatch; ++u) {
        const float *q = slot2(m + u < nch ? m + u : nch - 1);
        sg[u] = q[ec];
        tau[u] = q[D + ec];
      }
      // walk the batch in registers up to the first chunk whose sigma differs anywhere in the slice
      int bad = kCombineBatch;
#pragma unroll
      for (int u = 0; u < kCombineBatch; ++u) {
        const bool eq = !act || __float_as_uint(sg[u]) == __float_as_uint(cur);
        const bool all = __ballot(!eq) == 0ull;
        if (bad == kCombineBatch && m + u < nch) {
          if (all) cur = tau[u];
          else bad = u;
        }
      }
      if (bad == kCombineBatch) {
        m += kCombineBatch;
        continue;
      }
      // chunk m + bad started from a wrong state in this slice: recompute it from the exact state
      const int32_t c0 = s + (m + bad) * L;
      const int32_t c1 = static_cast<int64_t>(c0) + L < end ? c0 + L : end;
      slice_run(vals, spos, c0, c1, D, e, [&](int32_t, float x) { cur = ema1(cur, x, a, b); });
      m += bad + 1;
    }
    if (act) table[row * D + e] = cur;
  }
}

__global__ void __launch_bounds__(kThreads) ema_combine_kernel(EmaJobs js) {
  const int blk = static_cast<int>(blockIdx.x);
  for (int i = 0; i < js.count; ++i) {
    const EmaJob &j = js.job[i];
    if (blk >= j.comb_begin && blk < j.comb_begin + j.comb_blocks) {
      ema_combine(j.table, j.vals, j.table1, j.vals1, j.split, j.skey, j.spos, j.seg_start, j.seg_end, j.counters,
                  j.clist, j.a, j.b, js.D, j.L, j.partial, blk - j.comb_begin, j.comb_blocks);
      return;
    }
  }
}

// Chunking: a warm-up of W = ceil(28 / -ln a) steps shrinks a start error by
// e^-28, about 2^-40: far below fp32 resolution, with the remaining steps
// spent while the two trajectories' roundings fall onto the same value (for
// a = 0.95 and 0.99 about one 128-element slice in a thousand still differs
// after W steps; a slice that differs is recomputed by ema_combine).  A chunk's
// wave walks W + L positions and reads a value row for each, so L >= max(256,
// 3W) keeps the redundant warm-up reads at most a third of a chunk's (against
// 2W: a third fewer redundant reads for chains a third longer, 1% faster on
// the CS3 step); L is a whole number of the plan's runs
// (kBaseRun), and a row of at most L occurrences runs whole, as one exact
// chain.  Without contraction (a outside (0, 1)) rows run whole.
inline void ema_plan(float a, int64_t n, int *L, int *W) {
  int64_t len;
  if (a > 0.f && a < 1.f) {
    const double w = std::ceil(28.0 / -std::log(static_cast<double>(a)));
    *W = static_cast<int>(w < 1048576.0 ? w : 1048576.0);
    len = 3 * static_cast<int64_t>(*W);
  } else {
    *W = 0;
    len = n;
  }
  constexpr int64_t kMaxL = 0x7fffffff / kBaseRun * kBaseRun;
  len = len > kBaseRun ? len : kBaseRun;
  len = (len + kBaseRun - 1) / kBaseRun * kBaseRun;
  *L = static_cast<int>(len < kMaxL ? len : kMaxL);
}

inline size_t ema_partial_elems(int64_t n, int64_t dim) {
  // sized for the smallest chunk length (256): (2 * ceil(n / 256) + 2) slots x (sigma, tau) x dim floats
  return static_cast<size_t>(2 * ((n + 255) / 256) + 2) * 2 * static_cast<size_t>(dim / 4);
}

// The job of one update: its plan's buffers in ws (grouped by group_by_row),
// chunking for a, and its block counts.
// A pair plan (table1 != NULL): n counts both updates' pairs, num_rows both
// tables' rows, and keys from split (the first table's rows) on belong to table1.
EmaJob ema_job(float *table, const float *vals, int64_t n, int64_t dim, float a, float b, void *ws,
               int64_t num_rows, float *table1 = nullptr, const float *vals1 = nullptr,
               uint32_t split = 0xffffffffu) {
  SegWork<uint32_t> w;
  Carver c(ws);
  c.off = segwork_layout<uint32_t>(n, &w, ws);
  float *partial = reinterpret_cast<float *>(c.take<float4>(ema_partial_elems(n, dim)));
  const int cur = sorted_buffer(num_rows);
  EmaJob j{};
  j.table = table;
  j.vals = vals;
  j.table1 = table1;
  j.vals1 = vals1;
  j.split = table1 ? split : 0xffffffffu;
  j.n = n;
  j.seg_key = w.seg_key;
  j.skey = w.k[cur];
  j.spos = w.v[cur];
  j.seg_start = w.seg_start;
  j.seg_end = w.seg_end;
  j.nseg = w.nseg;
  j.counters = w.ticket;
  j.hlist = w.hlist;
  j.clist = w.clist;
  j.partial = partial;
  j.a = a;
  j.b = b;
  ema_plan(a, n, &j.L, &j.W);
  j.light_blocks = grid_for(n, 4 * 4) < 4096 ? grid_for(n, 4 * 4) : 4096;
  const int64_t hs = Narrow<kHeavyG>::slices(dim);
  j.heavy_blocks = grid_for(n / 32 * hs, 4) < 2048 ? grid_for(n / 32 * hs, 4) : 2048;
  j.comb_blocks = grid_for(n / 256 * num_slices(dim), 4) < 1024 ? grid_for(n / 256 * num_slices(dim), 4) : 1024;
  return j;
}

// Two launches for up to kMaxEmaJobs updates of one dim: heavy blocks of every
// job, then light blocks of every job; then the combine of every job.
void ema_launch(EmaJobs &js, hipStream_t s) {
  int next = 0;
  for (int i = 0; i < js.count; ++i) {
    js.job[i].heavy_begin = next;
    next += js.job[i].heavy_blocks;
  }
  for (int i = 0; i < js.count; ++i) {
    js.job[i].light_begin = next;
    next += js.job[i].light_blocks;
  }
  int comb = 0;
  for (int i = 0; i < js.count; ++i) {
    js.job[i].comb_begin = comb;
    comb += js.job[i].comb_blocks;
  }
  if (next == 0) return;
  const int64_t nc = (js.D / 4 + kWave - 1) / kWave;
  bool off32 = true;
  for (int i = 0; i < js.count; ++i) off32 = off32 && js.job[i].n * js.D * 4 < (int64_t(1) << 31);
  if (off32) {
    if (nc == 1) ema_apply_kernel<1, true><<<next, kThreads, 0, s>>>(js);
    else if (nc == 2) ema_apply_kernel<2, true><<<next, kThreads, 0, s>>>(js);
    else ema_apply_kernel<4, true><<<next, kThreads, 0, s>>>(js);
  } else {
    if (nc == 1) ema_apply_kernel<1, false><<<next, kThreads, 0, s>>>(js);
    else if (nc == 2) ema_apply_kernel<2, false><<<next, kThreads, 0, s>>>(js);
    else ema_apply_kernel<4, false><<<next, kThreads, 0, s>>>(js);
  }
  if (comb > 0) ema_combine_kernel<<<comb, kThreads, 0, s>>>(js);
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

namespace {

hlr_status ema_args(int64_t num_rows, int64_t n) {
  if (n < 0 || n > kMaxN || num_rows < 0 || num_rows >= 0x7fffffff) return HLR_INVALID_ARG;
  return HLR_OK;
}

hlr_status ema_ws(void *ws, size_t ws_bytes, size_t need) {
  if (!ws || ws_bytes < need) return HLR_WORKSPACE_TOO_SMALL;
  if (!aligned(ws, 256)) return HLR_MISALIGNED;
  return HLR_OK;
}

void ema_apply(float *table, int64_t num_rows, int64_t dim, const float *vals, int64_t n, float a, float b, void *ws,
               hipStream_t stream) {
  EmaJobs js{};
  js.count = 1;
  js.D = dim;
  js.job[0] = ema_job(table, vals, n, dim, a, b, ws, num_rows);
  ema_launch(js, stream);
}

}  // namespace

extern "C" hlr_status ema_update_rows(float *table, int64_t num_rows, int64_t dim, const int64_t *rows,
                                      const float *vals, const uint8_t *mask, int64_t n, float a, float b, void *ws,
                                      size_t ws_bytes, hipStream_t stream) {
  hlr_status st = ema_args(num_rows, n);
  if (st != HLR_OK) return st;
  if (dim <= 0 || dim % 4 != 0 || dim > 1024) return HLR_UNSUPPORTED_DIM;
  if (n == 0 || num_rows == 0) return HLR_OK;
  if (!table || !rows || !vals) return HLR_INVALID_ARG;
  if (!aligned(table, 16) || !aligned(vals, 16) || !aligned(rows, 8)) return HLR_MISALIGNED;
  if ((st = ema_ws(ws, ws_bytes, ema_update_rows_workspace_size(num_rows, dim, n))) != HLR_OK) return st;
  SegWork<uint32_t> w;
  segwork_layout<uint32_t>(n, &w, ws);
  group_by_row(w, rows, mask, num_rows, stream);
  list_heavy_units(w, stream);
  ema_apply(table, num_rows, dim, vals, n, a, b, ws, stream);
  return launch_status();
}

extern "C" hlr_status ema_update_plan(int64_t num_rows, const int64_t *rows, const uint8_t *mask, int64_t n,
                                      void *ws, size_t ws_bytes, hipStream_t stream) {
  hlr_status st = ema_args(num_rows, n);
  if (st != HLR_OK) return st;
  if (n == 0 || num_rows == 0) return HLR_OK;
  if (!rows) return HLR_INVALID_ARG;
  if (!aligned(rows, 8)) return HLR_MISALIGNED;
  if ((st = ema_ws(ws, ws_bytes, ema_update_rows_workspace_size(num_rows, 4, n))) != HLR_OK) return st;
  SegWork<uint32_t> w;
  segwork_layout<uint32_t>(n, &w, ws);
  group_by_row(w, rows, mask, num_rows, stream);
  list_heavy_units(w, stream);
  return launch_status();
}

namespace {

bool ranges_overlap(const void *a, size_t an, const void *b, size_t bn) {
  const char *x = static_cast<const char *>(a), *y = static_cast<const char *>(b);
  return x < y + bn && y < x + an;
}

}  // namespace

extern "C" hlr_status ema_update_apply_batch(int32_t count, const hlr_ema_apply *updates, hipStream_t stream) {
  if (count < 0 || count > kMaxEmaJobs || (count > 0 && !updates)) return HLR_INVALID_ARG;
  EmaJobs js{};
  js.D = 0;
  for (int32_t i = 0; i < count; ++i) {
    const hlr_ema_apply &u = updates[i];
    hlr_status st = ema_args(u.num_rows, u.n);
    if (st != HLR_OK) return st;
    if (u.dim <= 0 || u.dim % 4 != 0 || u.dim > 1024) return HLR_UNSUPPORTED_DIM;
    if (u.n == 0 || u.num_rows == 0) continue;
    if (!u.table || !u.vals) return HLR_INVALID_ARG;
    if (!aligned(u.table, 16) || !aligned(u.vals, 16)) return HLR_MISALIGNED;
    if ((st = ema_ws(u.ws, u.ws_bytes, ema_update_rows_workspace_size(u.num_rows, u.dim, u.n))) != HLR_OK) return st;
    if (js.D != 0 && u.dim != js.D) return HLR_INVALID_ARG;  // one dim per launch
    js.D = u.dim;
    const size_t tb = static_cast<size_t>(u.num_rows) * static_cast<size_t>(u.dim) * sizeof(float);
    const size_t wb = ema_update_rows_workspace_size(u.num_rows, u.dim, u.n);
    for (int32_t k = 0; k < i; ++k) {  // the updates run at once: no shared table or workspace
      const hlr_ema_apply &v = updates[k];
      if (v.n == 0 || v.num_rows == 0) continue;
      const size_t vb = static_cast<size_t>(v.num_rows) * static_cast<size_t>(v.dim) * sizeof(float);
      if (ranges_overlap(u.table, tb, v.table, vb) ||
          ranges_overlap(u.ws, wb, v.ws, ema_update_rows_workspace_size(v.num_rows, v.dim, v.n)))
        return HLR_INVALID_ARG;
    }
    js.job[js.count++] = ema_job(u.table, u.vals, u.n, u.dim, u.a, u.b, u.ws, u.num_rows);
  }
  if (js.count == 0) return HLR_OK;
  ema_launch(js, stream);
  return launch_status();
}

namespace {

// A pair plan's sizes: both tables' rows below the 32-bit key range (the
// sentinel num_rows0 + num_rows1 is a key too), both updates' pairs within
// the batch limit.
hlr_status pair_args(int64_t num_rows0, int64_t num_rows1, int64_t n) {
  if (num_rows0 < 0 || num_rows1 < 0 || n < 0 || n > kMaxN / 2) return HLR_INVALID_ARG;
  return ema_args(num_rows0 + num_rows1, 2 * n);
}

}  // namespace

extern "C" size_t ema_update_pair_workspace_size(int64_t num_rows0, int64_t num_rows1, int64_t dim, int64_t n) {
  if (pair_args(num_rows0, num_rows1, n) != HLR_OK) return 0;
  return ema_update_rows_workspace_size(num_rows0 + num_rows1, dim, 2 * n);
}

extern "C" hlr_status ema_update_plan_pair(int64_t num_rows0, const int64_t *rows0, int64_t num_rows1,
                                           const int64_t *rows1, const uint8_t *mask, int64_t n, void *ws,
                                           size_t ws_bytes, hipStream_t stream) {
  hlr_status st = pair_args(num_rows0, num_rows1, n);
  if (st != HLR_OK) return st;
  if (n == 0 || num_rows0 + num_rows1 == 0) return HLR_OK;
  if (!rows0 || !rows1) return HLR_INVALID_ARG;
  if (!aligned(rows0, 8) || !aligned(rows1, 8)) return HLR_MISALIGNED;
  if ((st = ema_ws(ws, ws_bytes, ema_update_pair_workspace_size(num_rows0, num_rows1, 4, n))) != HLR_OK) return st;
  SegWork<uint32_t> w;
  segwork_layout<uint32_t>(2 * n, &w, ws);
  group_by_row_pair(w, rows0, num_rows0, rows1, num_rows1, mask, stream);
  list_heavy_units(w, stream);
  return launch_status();
}

extern "C" hlr_status ema_update_apply_pairs(int32_t count, const hlr_ema_apply_pair *pairs, hipStream_t stream) {
  if (count < 0 || count > kMaxEmaJobs || (count > 0 && !pairs)) return HLR_INVALID_ARG;
  EmaJobs js{};
  js.D = 0;
  for (int32_t i = 0; i < count; ++i) {
    const hlr_ema_apply_pair &u = pairs[i];
    hlr_status st = pair_args(u.num_rows0, u.num_rows1, u.n);
    if (st != HLR_OK) return st;
    if (u.dim <= 0 || u.dim % 4 != 0 || u.dim > 1024) return HLR_UNSUPPORTED_DIM;
    if (u.n == 0 || u.num_rows0 + u.num_rows1 == 0) continue;
    if ((u.num_rows0 > 0 && (!u.table0 || !u.vals0)) || (u.num_rows1 > 0 && (!u.table1 || !u.vals1)))
      return HLR_INVALID_ARG;
    if ((u.table0 && !aligned(u.table0, 16)) || (u.vals0 && !aligned(u.vals0, 16)) ||
        (u.table1 && !aligned(u.table1, 16)) || (u.vals1 && !aligned(u.vals1, 16)))
      return HLR_MISALIGNED;
    const size_t wb = ema_update_pair_workspace_size(u.num_rows0, u.num_rows1, u.dim, u.n);
    if ((st = ema_ws(u.ws, u.ws_bytes, wb)) != HLR_OK) return st;
    if (js.D != 0 && u.dim != js.D) return HLR_INVALID_ARG;  // one dim per launch
    js.D = u.dim;
    const size_t tb0 = static_cast<size_t>(u.num_rows0) * static_cast<size_t>(u.dim) * sizeof(float);
    const size_t tb1 = static_cast<size_t>(u.num_rows1) * static_cast<size_t>(u.dim) * sizeof(float);
    if (u.num_rows0 > 0 && u.num_rows1 > 0 && ranges_overlap(u.table0, tb0, u.table1, tb1)) return HLR_INVALID_ARG;
    for (int32_t k = 0; k < i; ++k) {  // the updates run at once: no shared table or workspace
      const hlr_ema_apply_pair &v = pairs[k];
      if (v.n == 0 || v.num_rows0 + v.num_rows1 == 0) continue;
      const size_t vb0 = static_cast<size_t>(v.num_rows0) * static_cast<size_t>(v.dim) * sizeof(float);
      const size_t vb1 = static_cast<size_t>(v.num_rows1) * static_cast<size_t>(v.dim) * sizeof(float);
      if ((tb0 && vb0 && ranges_overlap(u.table0, tb0, v.table0, vb0)) ||
          (tb0 && vb1 && ranges_overlap(u.table0, tb0, v.table1, vb1)) ||
          (tb1 && vb0 && ranges_overlap(u.table1, tb1, v.table0, vb0)) ||
          (tb1 && vb1 && ranges_overlap(u.table1, tb1, v.table1, vb1)) ||
          ranges_overlap(u.ws, wb, v.ws, ema_update_pair_workspace_size(v.num_rows0, v.num_rows1, v.dim, v.n)))
        return HLR_INVALID_ARG;
    }
    js.job[js.count++] = ema_job(u.table0, u.vals0, 2 * u.n, u.dim, u.a, u.b, u.ws, u.num_rows0 + u.num_rows1,
                                 u.table1, u.vals1, static_cast<uint32_t>(u.num_rows0));
  }
  if (js.count == 0) return HLR_OK;
  ema_launch(js, stream);
  return launch_status();
}

extern "C" hlr_status ema_update_plan_subset(int64_t num_rows, const uint8_t *mask, int64_t n, const void *src_ws,
                                             size_t src_ws_bytes, void *ws, size_t ws_bytes, hipStream_t stream) {
  hlr_status st = ema_args(num_rows, n);
  if (st != HLR_OK) return st;
  if (n == 0 || num_rows == 0) return HLR_OK;
  if (!mask) return HLR_INVALID_ARG;
  const size_t need = ema_update_rows_workspace_size(num_rows, 4, n);
  if ((st = ema_ws(const_cast<void *>(src_ws), src_ws_bytes, need)) != HLR_OK) return st;
  if ((st = ema_ws(ws, ws_bytes, need)) != HLR_OK) return st;
  const char *a0 = static_cast<const char *>(src_ws), *b0 = static_cast<const char *>(ws);
  if (a0 < b0 + need && b0 < a0 + need) return HLR_INVALID_ARG;  // the two plans must not overlap
  SegWork<uint32_t> src, w;
  segwork_layout<uint32_t>(n, &src, const_cast<void *>(src_ws));
  segwork_layout<uint32_t>(n, &w, ws);
  subset_of_group(w, src, mask, num_rows, stream);
  list_heavy_units(w, stream);
  return launch_status();
}

extern "C" hlr_status ema_update_apply(float *table, int64_t num_rows, int64_t dim, const float *vals, int64_t n,
                                       float a, float b, void *ws, size_t ws_bytes, hipStream_t stream) {
  hlr_status st = ema_args(num_rows, n);
  if (st != HLR_OK) return st;
  if (dim <= 0 || dim % 4 != 0 || dim > 1024) return HLR_UNSUPPORTED_DIM;
  if (n == 0 || num_rows == 0) return HLR_OK;
  if (!table || !vals) return HLR_INVALID_ARG;
  if (!aligned(table, 16) || !aligned(vals, 16)) return HLR_MISALIGNED;
  if ((st = ema_ws(ws, ws_bytes, ema_update_rows_workspace_size(num_rows, dim, n))) != HLR_OK) return st;
  ema_apply(table, num_rows, dim, vals, n, a, b, ws, stream);
  return launch_status();
}
