// Stable LSD radix sort of (key, position) pairs and the segment table of the
// sorted keys.  Used to group a batch's positions by key (dedup) or by row
// (duplicate-summed SGD, EMA), positions ascending inside every group.
//
// Row keys (at most 31 bits) take 3-4 passes here; 64-bit ID keys (dedup)
// are sorted by msort.hpp instead, where 8 radix passes would cost more.
//
// Per pass: hist_kernel (per-tile digit histograms) and scatter_kernel (each
// tile derives its output offsets from all tiles' histograms, then stable
// ranks inside the tile from wave ballots + per-wave LDS counters).  No kernel
// waits on another block: cross-block data only crosses kernel boundaries (an
// agent-scope fence inside a kernel writes back the XCD's L2 and is avoided).  Digits are up to 8 bits, chosen so the key width is covered in
// ceil(bits/8) passes.
#pragma once

#include <utility>

#include "hlr_common.hpp"

namespace {

constexpr int kSortThreads = 256;
constexpr int kMaxSortItems = 16;                      // elements per thread, at most
constexpr int kMaxDigitBits = 8;
constexpr int kPosPad = 128;  // slack after the position buffers: batched reads may run past n
constexpr int kMaxBins = 1 << kMaxDigitBits;           // one digit per thread in the offset scan

// Segments long enough for whole-segment chains (kChainMin or more
// occurrences) listed by length: bucket b holds lengths in
// [2^(9+b), 2^(10+b)) (the last bucket also everything longer), in a region of
// (n >> (9+b)) + 1 entries, since at most n / 2^(9+b) segments of n positions
// can be that long.
constexpr int kLenBuckets = 16;
constexpr int kLenShift = 9;  // log2 of the shortest chained segment
constexpr int kChainMin = 1 << kLenShift;
constexpr int kTickets = 4 + kLenBuckets;
__host__ __device__ __forceinline__ int64_t len_bucket_cap(int64_t n, int b) { return (n >> (kLenShift + b)) + 1; }
__host__ __device__ __forceinline__ int64_t len_bucket_off(int64_t n, int b) {
  int64_t o = 0;
  for (int i = 0; i < b; ++i) o += len_bucket_cap(n, i);
  return o;
}

// Elements per thread: tiles of 1024..4096 so that a sort runs about 128 tiles
// (the passes are latency-bound at these sizes: against about 64 tiles, a
// hashed-tables step of 8 x 131,072 rows took 1.32 ms instead of 1.37 and a
// CS3 step of 262,144 pairs 0.217 ms instead of 0.222; about 256 tiles were
// slower for the CS3 step, whose scatter then reads four rounds of counts).
inline int sort_items(int64_t n) {
  if (n <= 128 * 1024) return 4;
  if (n <= 128 * 2048) return 8;
  return 16;
}

struct SortPlan {
  int passes = 0;
  int shift[8] = {0};
  int bits[8] = {0};
};

inline SortPlan make_plan(int total_bits) {
  SortPlan p;
  if (total_bits <= 0) total_bits = 1;
  p.passes = (total_bits + kMaxDigitBits - 1) / kMaxDigitBits;
  int s = 0;
  for (int i = 0; i < p.passes; ++i) {
    const int left = total_bits - s;
    const int b = (left + (p.passes - i) - 1) / (p.passes - i);
    p.shift[i] = s;
    p.bits[i] = b;
    s += b;
  }
  return p;
}

inline int bit_width_u64(uint64_t x) {
  int b = 0;
  while (x) {
    ++b;
    x >>= 1;
  }
  return b;
}

template <typename K>
struct SegWork {
  K *k[2];
  uint32_t *v[2];
  uint32_t *counts;  // [kMaxBins * nblocks]
  uint32_t *ticket;  // [kTickets]: heavy-run and combine list counts, the SGD apply's item and
                     // finished-block counters, then the length-bucket counts
  uint32_t *bcount;  // [nblocks]
  int32_t *segidx;   // [n]   segment of each sorted element (-1: excluded)
  int32_t *seg_start;  // [n]
  int32_t *seg_end;    // [n]
  K *seg_key;          // [n]   key of each segment (row grouping only)
  int64_t *nseg;       // [1]
  uint32_t *nact;      // [1]   elements that take part (sorted first); the rest of the n slots are unused
  int2 *hlist;         // heavy work units (segment, run), listed by the plan (list_heavy_units)
  int32_t *clist;      // segments with more than one run (combined after the heavy kernel)
  int32_t *slist;      // heavy segments by length bucket, longest bucket first (list_heavy_segments)
  int64_t n;
  int nblocks;
  int items;  // elements per thread (tile = 256 * items)
};

template <typename K>
inline size_t segwork_layout(int64_t n, SegWork<K> *w, void *base) {
  hlr::Carver c(base);
  const int items = sort_items(n);
  const int64_t tile = static_cast<int64_t>(kSortThreads) * items;
  const int nb = static_cast<int>((n + tile - 1) / tile);
  const size_t nn = static_cast<size_t>(n > 0 ? n : 1);
  w->k[0] = c.take<K>(nn);
  w->k[1] = c.take<K>(nn);
  w->v[0] = c.take<uint32_t>(nn + kPosPad);
  w->v[1] = c.take<uint32_t>(nn + kPosPad);
  // per-tile tables sized for the smallest tile (a masked grouping sorts with 4 items per thread)
  const int64_t nb_max = (n + kSortThreads * 4 - 1) / (kSortThreads * 4);
  w->counts = c.take<uint32_t>(static_cast<size_t>(kMaxBins) * (nb_max > 0 ? nb_max : 1));
  w->ticket = c.take<uint32_t>(kTickets);
  w->bcount = c.take<uint32_t>(2 * static_cast<size_t>(nb_max > 0 ? nb_max : 1));
  w->segidx = c.take<int32_t>(nn);
  w->seg_start = c.take<int32_t>(nn);
  w->seg_end = c.take<int32_t>(nn);
  w->seg_key = c.take<K>(nn);
  w->nseg = c.take<int64_t>(1);
  w->nact = c.take<uint32_t>(1);
  w->hlist = c.take<int2>(nn / 32 + 64);
  w->clist = c.take<int32_t>(nn / 256 + 64);
  w->slist = c.take<int32_t>(static_cast<size_t>(len_bucket_off(static_cast<int64_t>(nn), kLenBuckets)));
  w->n = n;
  w->nblocks = nb;
  w->items = items;
  return c.off;
}

// ------------------------------------------------------------------ kernels
// Elements in use: the first *nact of the n slots when a device count is
// given (a compacted input), else all n.
__device__ __forceinline__ int64_t active_count(int64_t n, const uint32_t *nact) {
  if (!nact) return n;
  const int64_t m = static_cast<int64_t>(*nact);
  return m < n ? m : n;
}

// Tiles holding elements in use; per-tile tables are read only for these.
__device__ __forceinline__ int used_tiles(int64_t m, int tile, int nblocks) {
  const int64_t t = (m + tile - 1) / tile;
  return static_cast<int>(t < nblocks ? t : nblocks);
}

// Block-wide exclusive scan of one uint32 per thread (256 threads); returns the
// exclusive prefix and writes the block total to *total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t *sh /*[256+]*/, uint32_t *total) {
  const int t = threadIdx.x;
  sh[t] = x;
  __syncthreads();
  for (int off = 1; off < kSortThreads; off <<= 1) {
    const uint32_t y = t >= off ? sh[t - off] : 0u;
    __syncthreads();
    sh[t] += y;
    __syncthreads();
  }
  const uint32_t incl = sh[t];
  *total = sh[kSortThreads - 1];
  __syncthreads();
  return incl - x;
}

// Where a pass reads its (key, position) pairs: the ping-pong buffers, or, in
// the first pass of a grouping by row, the batch's rows themselves (key = the
// row, or the sentinel num_rows for a row out of range; position = index),
// which saves the kernel that would write them out first.
template <typename K>
struct BufPairs {
  const K *k;
  const uint32_t *v;
  __device__ __forceinline__ K key(int64_t i) const { return k[i]; }
  __device__ __forceinline__ uint32_t pos(int64_t i) const { return v[i]; }
};

struct RowPairs {
  const int64_t *rows;
  int64_t num_rows;
  __device__ __forceinline__ uint32_t key(int64_t i) const {
    const int64_t r = rows[i];
    return static_cast<uint32_t>(r >= 0 && r < num_rows ? r : num_rows);
  }
  __device__ __forceinline__ uint32_t pos(int64_t i) const { return static_cast<uint32_t>(i); }
};

// The rows of two tables as one key space (a pair plan: two updates keyed by
// different rows, planned by one sort).  Pair i < n is position i of rows0
// with its row; pair n + i is position i of rows1 with num_rows0 + its row.
// A row out of range takes the sentinel num_rows0 + num_rows1.
struct PairRowPairs {
  const int64_t *rows0, *rows1;
  int64_t n, num_rows0, num_rows1;
  __device__ __forceinline__ uint32_t key(int64_t i) const {
    const bool second = i >= n;
    const int64_t r = second ? rows1[i - n] : rows0[i];
    const int64_t lim = second ? num_rows1 : num_rows0;
    return static_cast<uint32_t>(r >= 0 && r < lim ? (second ? num_rows0 + r : r) : num_rows0 + num_rows1);
  }
  __device__ __forceinline__ uint32_t pos(int64_t i) const { return static_cast<uint32_t>(i >= n ? i - n : i); }
};

// init_ticket / init_nact (first pass over RowPairs only): block 0 also clears
// the plan's counters and records that all n pairs take part.
template <typename K, int ITEMS, typename Src>
__global__ void __launch_bounds__(kSortThreads)
    hist_kernel(Src src, int64_t n, const uint32_t *__restrict__ nact, int shift, int bits, uint32_t *counts,
                uint32_t *init_ticket, uint32_t *init_nact) {
  constexpr int TILE = kSortThreads * ITEMS;
  if (blockIdx.x == 0 && init_ticket && threadIdx.x < kTickets) init_ticket[threadIdx.x] = 0u;
  if (blockIdx.x == 0 && init_nact && threadIdx.x == 0) *init_nact = static_cast<uint32_t>(n);
  n = active_count(n, nact);
  if (static_cast<int64_t>(blockIdx.x) * TILE >= n) return;  // empty tiles are never read (see used_tiles)
  __shared__ uint32_t h[kMaxBins];
  const int bins = 1 << bits;
  const uint32_t mask = static_cast<uint32_t>(bins - 1);
  h[threadIdx.x] = 0;
  __syncthreads();
  const int64_t base = static_cast<int64_t>(blockIdx.x) * TILE;
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    const int64_t idx = base + k * kSortThreads + threadIdx.x;
    if (idx < n) atomicAdd(&h[static_cast<uint32_t>(src.key(idx) >> shift) & mask], 1u);
  }
  __syncthreads();
  counts[static_cast<int64_t>(blockIdx.x) * kMaxBins + threadIdx.x] = threadIdx.x < bins ? h[threadIdx.x] : 0u;
}

template <typename K, int ITEMS, typename Src>
__global__ void __launch_bounds__(kSortThreads)
    scatter_kernel(Src src, K *__restrict__ kout, uint32_t *__restrict__ vout, int64_t n,
                   const uint32_t *__restrict__ nact, int shift, int bits, const uint32_t *__restrict__ counts,
                   int nblocks) {
  constexpr int TILE = kSortThreads * ITEMS;
  n = active_count(n, nact);
  if (static_cast<int64_t>(blockIdx.x) * TILE >= n) return;  // an empty tile writes nothing
  __shared__ uint32_t cnt[4][kMaxBins];
  __shared__ uint32_t sh[kSortThreads];
  __shared__ uint32_t offs[kMaxBins];
  const int bins = 1 << bits;
  const uint32_t mask = static_cast<uint32_t>(bins - 1);
  const int w = threadIdx.x >> 6;
  // This tile's output offset of every digit: (keys with smaller digits) + (same digit, earlier tiles).
  // Thread d reads digit d of every tile's histogram (rows of 256 counts, coalesced across the block),
  // 64 tiles per round of loads (a sort here runs about 128 tiles, so two round trips).
  nblocks = used_tiles(n, TILE, nblocks);
  {
    constexpr int kRound = 64;
    const int d = threadIdx.x;
    uint32_t before = 0, total = 0;
    for (int b0 = 0; b0 < nblocks; b0 += kRound) {
      uint32_t v[kRound];
#pragma unroll
      for (int u = 0; u < kRound; ++u)
        v[u] = b0 + u < nblocks ? counts[static_cast<int64_t>(b0 + u) * kMaxBins + d] : 0u;
#pragma unroll
      for (int u = 0; u < kRound; ++u) {
        if (b0 + u < static_cast<int>(blockIdx.x)) before += v[u];
        total += v[u];
      }
    }
    uint32_t all;
    offs[d] = block_exclusive_scan(total, sh, &all) + before;
  }
  for (int x = threadIdx.x; x < 4 * bins; x += kSortThreads) cnt[x / bins][x % bins] = 0;
  __syncthreads();
  const int64_t base = static_cast<int64_t>(blockIdx.x) * TILE + w * (TILE / 4);
  const uint64_t lt = hlr::lanemask_lt();
  K kk[ITEMS];
  uint32_t vv[ITEMS];
  uint32_t rk[ITEMS];
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    const int64_t idx = base + r * hlr::kWave + hlr::lane_id();
    const bool valid = idx < n;
    const K k = valid ? src.key(idx) : K(0);
    const uint32_t d = static_cast<uint32_t>(k >> shift) & mask;
    uint64_t peers = hlr::ballot(valid);
    for (int b = 0; b < bits; ++b) {
      const bool bit = (d >> b) & 1u;
      const uint64_t bb = hlr::ballot(bit);
      peers &= bit ? bb : ~bb;
    }
    const uint32_t rin = static_cast<uint32_t>(__popcll(peers & lt));
    const uint32_t prev = valid ? cnt[w][d] : 0u;
    if (valid && rin == 0) cnt[w][d] = prev + static_cast<uint32_t>(__popcll(peers));
    kk[r] = k;
    vv[r] = valid ? src.pos(idx) : 0u;
    rk[r] = prev + rin;
  }
  __syncthreads();
  for (int d = threadIdx.x; d < bins; d += kSortThreads) {
    uint32_t run = offs[d];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t c = cnt[q][d];
      cnt[q][d] = run;
      run += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    const int64_t idx = base + r * hlr::kWave + hlr::lane_id();
    if (idx < n) {
      const uint32_t d = static_cast<uint32_t>(kk[r] >> shift) & mask;
      const uint32_t dst = cnt[w][d] + rk[r];
      kout[dst] = kk[r];
      vout[dst] = vv[r];
    }
  }
}

// Segment passes.  A tile of 256 * ITEMS sorted elements is read as ITEMS
// chunks of 256 consecutive elements (thread t takes element t of each chunk),
// so every load is coalesced; heads (an element whose key differs from its
// predecessor's) are counted with wave ballots.  Elements whose key equals
// `excluded` belong to no segment.
template <typename K, int ITEMS>
__device__ __forceinline__ void seg_heads(const K *__restrict__ keys, int64_t n, K excluded, bool use_excluded,
                                          K (&kk)[ITEMS], bool (&head)[ITEMS], bool (&tail)[ITEMS],
                                          bool (&ok)[ITEMS]) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kSortThreads * ITEMS + threadIdx.x;
  K prev[ITEMS], next[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int64_t j = base + i * kSortThreads;
    kk[i] = j < n ? keys[j] : K(0);
    prev[i] = (j > 0 && j < n) ? keys[j - 1] : K(0);
    next[i] = j + 1 < n ? keys[j + 1] : K(0);
  }
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int64_t j = base + i * kSortThreads;
    ok[i] = j < n && !(use_excluded && kk[i] == excluded);
    head[i] = ok[i] && (j == 0 || prev[i] != kk[i]);
    tail[i] = ok[i] && (j == n - 1 || next[i] != kk[i]);
  }
}

// Segment pass 1: number of segment heads per tile.
template <typename K, int ITEMS>
__global__ void __launch_bounds__(kSortThreads)
    seg_count_kernel(const K *__restrict__ keys, int64_t n, const uint32_t *__restrict__ nact, K excluded,
                     bool use_excluded, uint32_t *bcount) {
  __shared__ uint32_t wsum[kSortThreads / hlr::kWave];
  n = active_count(n, nact);
  if (static_cast<int64_t>(blockIdx.x) * kSortThreads * ITEMS >= n) return;  // never read (see used_tiles)
  K kk[ITEMS];
  bool head[ITEMS], tail[ITEMS], ok[ITEMS];
  seg_heads<K, ITEMS>(keys, n, excluded, use_excluded, kk, head, tail, ok);
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) c += static_cast<uint32_t>(__popcll(hlr::ballot(head[i])));
  const int w = threadIdx.x / hlr::kWave;
  if (hlr::lane_id() == 0) wsum[w] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int q = 0; q < kSortThreads / hlr::kWave; ++q) t += wsum[q];
    bcount[blockIdx.x] = t;
  }
}

// Segment pass 2: per sorted element its segment index; heads and tails record
// the segment bounds (and, when seg_key is given, the segment's key).  The
// functor `emit(j, seg, head, tail, key, val)` adds mode-specific outputs
// (dedup: unique keys, last positions, inverse).  A head's segment index is
// the number of heads before it: earlier tiles (from bcount), earlier chunks
// and waves of this tile (per-wave ballot counts in LDS), earlier lanes.
template <typename K, typename Emit, int ITEMS>
__global__ void __launch_bounds__(kSortThreads)
    seg_index_kernel(const K *__restrict__ keys, const uint32_t *__restrict__ vals, int64_t n,
                     const uint32_t *__restrict__ nact, K excluded, bool use_excluded,
                     const uint32_t *__restrict__ bcount, int nblocks, int32_t *segidx, int32_t *seg_start,
                     int32_t *seg_end, K *seg_key, int64_t *nseg, Emit emit) {
  constexpr int NW = kSortThreads / hlr::kWave;
  n = active_count(n, nact);
  nblocks = used_tiles(n, kSortThreads * ITEMS, nblocks);
  if (static_cast<int>(blockIdx.x) >= nblocks && blockIdx.x != 0) return;  // tile 0 publishes nseg even if m == 0
  __shared__ uint32_t sh[kSortThreads];
  __shared__ uint32_t wcnt[ITEMS][NW];
  __shared__ uint32_t blk_off;
  // This tile's first segment index = heads in earlier tiles; tile 0 also publishes the total.
  {
    uint32_t before = 0, total = 0;
    for (int b = threadIdx.x; b < nblocks; b += kSortThreads) {
      const uint32_t v = bcount[b];
      if (b < static_cast<int>(blockIdx.x)) before += v;
      total += v;
    }
    uint32_t all;
    block_exclusive_scan(before, sh, &all);
    if (threadIdx.x == 0) blk_off = all;
    uint32_t tall;
    block_exclusive_scan(total, sh, &tall);
    if (blockIdx.x == 0 && threadIdx.x == 0) *nseg = tall;
  }
  K kk[ITEMS];
  bool head[ITEMS], tail[ITEMS], ok[ITEMS];
  seg_heads<K, ITEMS>(keys, n, excluded, use_excluded, kk, head, tail, ok);
  const int w = threadIdx.x / hlr::kWave;
  const uint64_t lt = hlr::lanemask_lt();
  uint32_t rank[ITEMS];  // heads before this element within its wave's 64 elements, this one included
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const uint64_t m = hlr::ballot(head[i]);
    rank[i] = static_cast<uint32_t>(__popcll(m & lt)) + (head[i] ? 1u : 0u);
    if (hlr::lane_id() == 0) wcnt[i][w] = static_cast<uint32_t>(__popcll(m));
  }
  __syncthreads();
  uint32_t run = blk_off;  // heads before chunk i
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kSortThreads * ITEMS + threadIdx.x;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    uint32_t before_w = 0, chunk = 0;
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      const uint32_t c = wcnt[i][q];
      before_w += q < w ? c : 0u;
      chunk += c;
    }
    const int64_t j = base + i * kSortThreads;
    if (j < n) {
      if (!ok[i]) {
        segidx[j] = -1;
      } else {
        // the segment this element belongs to: heads up to and including it, minus one
        const int32_t seg = static_cast<int32_t>(run + before_w + rank[i]) - 1;
        segidx[j] = seg;
        if (head[i]) {
          seg_start[seg] = static_cast<int32_t>(j);
          if (seg_key) seg_key[seg] = kk[i];
        }
        if (tail[i]) seg_end[seg] = static_cast<int32_t>(j + 1);
        emit(j, seg, head[i], tail[i], kk[i], vals[j]);
      }
    }
    run += chunk;
  }
}

struct NoEmit {
  template <typename K>
  __device__ void operator()(int64_t, int32_t, bool, bool, K, uint32_t) const {}
};

// Runs every radix pass; returns the index (0/1) of the buffer holding the result.
// first != NULL: the first pass reads the pairs from the batch's rows (RowPairs
// or PairRowPairs) and sets up the plan's counters and active count on the
// way; then every element takes part (nact is written, not read, by that pass).
template <typename K, int ITEMS, typename First>
inline int radix_sort_pairs_t(SegWork<K> &w, int total_bits, const uint32_t *nact, hipStream_t s, const First *first) {
  const SortPlan plan = make_plan(total_bits);
  int cur = 0;
  for (int p = 0; p < plan.passes; ++p) {
    if (p == 0 && first) {
      hist_kernel<K, ITEMS, First><<<w.nblocks, kSortThreads, 0, s>>>(*first, w.n, nullptr, plan.shift[p],
                                                                       plan.bits[p], w.counts, w.ticket, w.nact);
      scatter_kernel<K, ITEMS, First><<<w.nblocks, kSortThreads, 0, s>>>(
          *first, w.k[cur ^ 1], w.v[cur ^ 1], w.n, nullptr, plan.shift[p], plan.bits[p], w.counts, w.nblocks);
    } else {
      const BufPairs<K> src{w.k[cur], w.v[cur]};
      hist_kernel<K, ITEMS, BufPairs<K>><<<w.nblocks, kSortThreads, 0, s>>>(src, w.n, nact, plan.shift[p],
                                                                             plan.bits[p], w.counts, nullptr,
                                                                             nullptr);
      scatter_kernel<K, ITEMS, BufPairs<K>><<<w.nblocks, kSortThreads, 0, s>>>(
          src, w.k[cur ^ 1], w.v[cur ^ 1], w.n, nact, plan.shift[p], plan.bits[p], w.counts, w.nblocks);
    }
    cur ^= 1;
  }
  return cur;
}

// nact: device count of the elements in use (the first *nact slots), or NULL for all n.
template <typename K, typename First = RowPairs>
inline int radix_sort_pairs(SegWork<K> &w, int total_bits, hipStream_t s, const uint32_t *nact = nullptr,
                            const First *first = nullptr) {
  if (w.items == 4) return radix_sort_pairs_t<K, 4, First>(w, total_bits, nact, s, first);
  if (w.items == 8) return radix_sort_pairs_t<K, 8, First>(w, total_bits, nact, s, first);
  return radix_sort_pairs_t<K, 16, First>(w, total_bits, nact, s, first);
}

template <typename K, typename Emit, int ITEMS>
inline void segment_sorted_t(SegWork<K> &w, int cur, K excluded, bool use_excluded, K *seg_key, Emit emit,
                             const uint32_t *nact, hipStream_t s) {
  seg_count_kernel<K, ITEMS><<<w.nblocks, kSortThreads, 0, s>>>(w.k[cur], w.n, nact, excluded, use_excluded,
                                                                 w.bcount);
  seg_index_kernel<K, Emit, ITEMS><<<w.nblocks, kSortThreads, 0, s>>>(
      w.k[cur], w.v[cur], w.n, nact, excluded, use_excluded, w.bcount, w.nblocks, w.segidx, w.seg_start, w.seg_end,
      seg_key, w.nseg, emit);
}

template <typename K, typename Emit>
inline void segment_sorted(SegWork<K> &w, int cur, K excluded, bool use_excluded, K *seg_key, Emit emit,
                           hipStream_t s, const uint32_t *nact = nullptr) {
  if (w.items == 4) segment_sorted_t<K, Emit, 4>(w, cur, excluded, use_excluded, seg_key, emit, nact, s);
  else if (w.items == 8) segment_sorted_t<K, Emit, 8>(w, cur, excluded, use_excluded, seg_key, emit, nact, s);
  else segment_sorted_t<K, Emit, 16>(w, cur, excluded, use_excluded, seg_key, emit, nact, s);
}

}  // namespace

namespace {

// With a mask, only the positions that take part are sorted: they are first
// compacted, in position order, into the first *nact slots (a masked update
// such as CTS's positives is a few percent of the batch, and the sort then
// handles only those).  Tiles as in the sort (256 * ITEMS elements, chunks of
// 256 consecutive elements); pass 1 counts each tile's elements that take
// part, pass 2 places them: earlier tiles, then earlier chunks and waves of
// this tile (ballot counts in LDS), then earlier lanes.  The compaction is
// stable, so it also cuts a subset out of an existing plan's sorted pairs
// without sorting again (FromPlan).
//
// Element i of a batch: position i, if its row is in range and its mask set.
struct FromPositions {
  const int64_t *rows;
  const uint8_t *mask;
  int64_t num_rows;
  __device__ __forceinline__ int64_t count(int64_t n) const { return n; }
  __device__ __forceinline__ bool get(int64_t i, int64_t m, uint32_t *key, uint32_t *pos) const {
    if (i >= m) return false;
    const int64_t r = rows[i];
    *key = static_cast<uint32_t>(r);
    *pos = static_cast<uint32_t>(i);
    return r >= 0 && r < num_rows && mask[i] != 0;
  }
};

// Element i of a plan's sorted (row, position) pairs: kept if it belongs to a
// row (not the sentinel) and the mask is set at its position.
// Pair i of a pair plan's 2n pairs (see PairRowPairs), kept if its row is in
// range and the mask is set at its position.
struct FromPositionsPair {
  const int64_t *rows0, *rows1;
  const uint8_t *mask;
  int64_t n, num_rows0, num_rows1;
  __device__ __forceinline__ int64_t count(int64_t m) const { return m; }
  __device__ __forceinline__ bool get(int64_t i, int64_t m, uint32_t *key, uint32_t *pos) const {
    if (i >= m) return false;
    const bool second = i >= n;
    const int64_t p = second ? i - n : i;
    const int64_t r = second ? rows1[p] : rows0[p];
    const int64_t lim = second ? num_rows1 : num_rows0;
    *key = static_cast<uint32_t>(second ? num_rows0 + r : r);
    *pos = static_cast<uint32_t>(p);
    return r >= 0 && r < lim && mask[p] != 0;
  }
};

struct FromPlan {
  const uint32_t *keys;
  const uint32_t *spos;
  const uint32_t *nact;
  uint32_t sentinel;
  const uint8_t *mask;
  __device__ __forceinline__ int64_t count(int64_t n) const { return active_count(n, nact); }
  __device__ __forceinline__ bool get(int64_t i, int64_t m, uint32_t *key, uint32_t *pos) const {
    if (i >= m) return false;
    *key = keys[i];
    *pos = spos[i];
    return *key != sentinel && mask[*pos] != 0;
  }
};

template <int ITEMS, typename Src>
__global__ void __launch_bounds__(kSortThreads)
    mask_count_kernel(Src src, int64_t n, uint32_t *bcount) {
  __shared__ uint32_t wsum[kSortThreads / hlr::kWave];
  const int64_t m = src.count(n);
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kSortThreads * ITEMS + threadIdx.x;
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    uint32_t key, pos;
    c += static_cast<uint32_t>(__popcll(hlr::ballot(src.get(base + i * kSortThreads, m, &key, &pos))));
  }
  if (hlr::lane_id() == 0) wsum[threadIdx.x / hlr::kWave] = c;
  __syncthreads();
  if (threadIdx.x == 0) {  // every tile writes its count, empty or not
    uint32_t t = 0;
    for (int q = 0; q < kSortThreads / hlr::kWave; ++q) t += wsum[q];
    bcount[blockIdx.x] = t;
  }
}

template <int ITEMS, typename Src>
__global__ void __launch_bounds__(kSortThreads)
    mask_compact_kernel(Src src, int64_t n, const uint32_t *__restrict__ bcount, int nblocks,
                        uint32_t *__restrict__ k, uint32_t *__restrict__ v, uint32_t *ticket, uint32_t *nact) {
  constexpr int NW = kSortThreads / hlr::kWave;
  __shared__ uint32_t sh[kSortThreads];
  __shared__ uint32_t wcnt[ITEMS][NW];
  __shared__ uint32_t blk_off;
  {
    uint32_t before = 0, total = 0;
    for (int b = threadIdx.x; b < nblocks; b += kSortThreads) {
      const uint32_t c = bcount[b];
      if (b < static_cast<int>(blockIdx.x)) before += c;
      total += c;
    }
    uint32_t all;
    block_exclusive_scan(before, sh, &all);
    if (threadIdx.x == 0) blk_off = all;
    uint32_t tall;
    block_exclusive_scan(total, sh, &tall);
    if (blockIdx.x == 0 && threadIdx.x == 0) *nact = tall;
    if (blockIdx.x == 0 && threadIdx.x < kTickets) ticket[threadIdx.x] = 0u;
  }
  const int64_t m = src.count(n);
  const int w = threadIdx.x / hlr::kWave;
  const uint64_t lt = hlr::lanemask_lt();
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kSortThreads * ITEMS + threadIdx.x;
  bool ok[ITEMS];
  uint32_t key[ITEMS], pos[ITEMS], rank[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    ok[i] = src.get(base + i * kSortThreads, m, &key[i], &pos[i]);
    const uint64_t bm = hlr::ballot(ok[i]);
    rank[i] = static_cast<uint32_t>(__popcll(bm & lt));
    if (hlr::lane_id() == 0) wcnt[i][w] = static_cast<uint32_t>(__popcll(bm));
  }
  __syncthreads();
  uint32_t run = blk_off;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    uint32_t before_w = 0, chunk = 0;
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      const uint32_t c = wcnt[i][q];
      before_w += q < w ? c : 0u;
      chunk += c;
    }
    if (ok[i]) {
      const uint32_t dst = run + before_w + rank[i];
      k[dst] = key[i];
      v[dst] = pos[i];
    }
    run += chunk;
  }
}

// Index (0/1) of the buffer that holds the sorted result for a table of num_rows rows.
inline int sorted_buffer(int64_t num_rows) {
  return make_plan(bit_width_u64(static_cast<uint64_t>(num_rows))).passes & 1;
}

// Compacts the elements of src that take part into (k[buf], v[buf]), in order;
// count in *nact.
template <int ITEMS, typename Src>
inline void compact_into(SegWork<uint32_t> &w, const Src &src, int buf, hipStream_t s) {
  mask_count_kernel<ITEMS, Src><<<w.nblocks, kSortThreads, 0, s>>>(src, w.n, w.bcount);
  mask_compact_kernel<ITEMS, Src><<<w.nblocks, kSortThreads, 0, s>>>(src, w.n, w.bcount, w.nblocks, w.k[buf],
                                                                      w.v[buf], w.ticket, w.nact);
}

inline void small_tiles(SegWork<uint32_t> &w) {
  // a masked grouping usually keeps a few percent of the batch, and tiles past the
  // compacted count cost a launch slot only
  w.items = 4;
  w.nblocks = static_cast<int>((w.n + kSortThreads * 4 - 1) / (kSortThreads * 4));
}

// Groups positions by row: returns the buffer index holding (row, position)
// sorted by row, positions ascending within a row, with the segment table
// (seg_start, seg_end, nseg) built.
inline int group_by_row(SegWork<uint32_t> &w, const int64_t *rows, const uint8_t *mask, int64_t num_rows,
                        hipStream_t s) {
  const int bits = bit_width_u64(static_cast<uint64_t>(num_rows));
  int cur;
  if (mask) {
    small_tiles(w);
    compact_into<4>(w, FromPositions{rows, mask, num_rows}, 0, s);
    cur = radix_sort_pairs<uint32_t>(w, bits, s, w.nact);
  } else {  // the first pass reads the rows directly
    const RowPairs first{rows, num_rows};
    cur = radix_sort_pairs<uint32_t>(w, bits, s, w.nact, &first);
  }
  segment_sorted<uint32_t>(w, cur, static_cast<uint32_t>(num_rows), true, w.seg_key, NoEmit{}, s, w.nact);
  return cur;
}

// Groups the positions of two updates by row in one sort (a pair plan over
// w.n = 2n pairs, keys as in PairRowPairs): returns the buffer index holding
// the sorted pairs, with the segment table built.  Each segment belongs to one
// table (keys below num_rows0: rows0's table), its positions ascending.
inline int group_by_row_pair(SegWork<uint32_t> &w, const int64_t *rows0, int64_t num_rows0, const int64_t *rows1,
                             int64_t num_rows1, const uint8_t *mask, hipStream_t s) {
  const int64_t n = w.n / 2;
  const int64_t sentinel = num_rows0 + num_rows1;
  const int bits = bit_width_u64(static_cast<uint64_t>(sentinel));
  int cur;
  if (mask) {
    small_tiles(w);
    compact_into<4>(w, FromPositionsPair{rows0, rows1, mask, n, num_rows0, num_rows1}, 0, s);
    cur = radix_sort_pairs<uint32_t>(w, bits, s, w.nact);
  } else {
    const PairRowPairs first{rows0, rows1, n, num_rows0, num_rows1};
    cur = radix_sort_pairs<uint32_t>(w, bits, s, w.nact, &first);
  }
  segment_sorted<uint32_t>(w, cur, static_cast<uint32_t>(sentinel), true, w.seg_key, NoEmit{}, s, w.nact);
  return cur;
}

// The grouping of a subset: the pairs of an existing grouping `src` (same n and
// num_rows) whose position has mask set, cut out in order (stable, so positions
// stay ascending within each row) and segmented.  Equals group_by_row over the
// same rows with the two masks combined, without sorting.
inline int subset_of_group(SegWork<uint32_t> &w, const SegWork<uint32_t> &src, const uint8_t *mask, int64_t num_rows,
                           hipStream_t s) {
  const int cur = sorted_buffer(num_rows);
  small_tiles(w);
  compact_into<4>(w, FromPlan{src.k[cur], src.v[cur], src.nact, static_cast<uint32_t>(num_rows), mask}, cur, s);
  segment_sorted<uint32_t>(w, cur, static_cast<uint32_t>(num_rows), true, w.seg_key, NoEmit{}, s, w.nact);
  return cur;
}

}  // namespace

namespace {

// Partial results of the runs (runs of B consecutive occurrences of a row) of
// rows longer than B.  At most one such row starts inside any sorted window
// [x*B, (x+1)*B) and at most one non-first run starts inside it, so
// slot = 2*window + (first run ? 1 : 0) is unique per call and < 2*ceil(n/B) + 2.
__device__ __forceinline__ int64_t run_slot(int32_t j0, int32_t m, int B) {
  return 2 * static_cast<int64_t>(j0 / B) + (m == 0 ? 1 : 0);
}

}  // namespace

namespace {

// Heavy rows are processed as independent wave work items, one per (run, slice):
// a slice is kSliceElems consecutive elements of the row (lanes own one each),
// so a row of D elements has ceil(D / kSliceElems) slices and every slice of
// every run is its own wave.  slice_run() applies f(j, x) to positions j in
// [j0, j1) in order.  Positions go in batches of P: the rows of a batch are
// requested together (one 256-byte access per position), then the position
// indices of the next batch, so they arrive while this batch is consumed.
// Indices are read with one vector load (lane u takes position j + u) and
// broadcast with readlane; a row is then read with a buffer load whose base
// (the row's address) is built in scalar registers and whose offset is the
// lane's byte offset, so a position costs scalar arithmetic and no per-lane
// 64-bit address.  No row load has a per-lane condition: lanes past the end of
// the row read element 0 and their results are dropped by the caller;
// positions past j1 in the last batch re-read position j1 - 1 and are not
// applied.  A batch costs one register per position; P + 1 loads in flight
// stay within the wave's memory counter (at most 63 outstanding).
//
// (Keeping two batches in flight across loop iterations was tried: hipcc
// then copies the in-flight registers at the loop head, which waits for every
// load, so the single batch is kept.)
using SliceV = float;
constexpr int kSliceElems = 64;
constexpr int kSlicePrefetch = 48;
static_assert(kSlicePrefetch <= 62, "one index per lane, counter limit");

__host__ __device__ __forceinline__ int64_t num_slices(int64_t D) { return (D + kSliceElems - 1) / kSliceElems; }

// This lane's index of the batch at j (lanes >= P repeat the last of the batch).
template <int P>
__device__ __forceinline__ uint32_t slice_idx(const uint32_t *__restrict__ spos, int32_t j, int32_t j1) {
  const int l = hlr::lane_id();
  const int32_t jj = j + (l < P ? l : P - 1);
  return spos[jj < j1 ? jj : j1 - 1];
}

// Element `eoff / 4` of row p: word 3 is the gfx9 descriptor for raw 32-bit
// accesses; the record limit exceeds any offset used here.
__device__ __forceinline__ SliceV slice_load(const char *base, uint32_t p, uint32_t row_bytes, uint32_t eoff) {
  char *rp = const_cast<char *>(base) + static_cast<uint64_t>(p) * row_bytes;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(rp, 0, 0x7fffffff, 0x00020000);
  return __builtin_bit_cast(SliceV, __builtin_amdgcn_raw_buffer_load_b32(r, eoff, 0, 0));
}

template <int P = kSlicePrefetch, typename F>
__device__ __forceinline__ void slice_run(const float *__restrict__ src, const uint32_t *__restrict__ spos, int32_t j0,
                                          int32_t j1, int64_t D, int64_t e, F f) {
  static_assert(P <= 62, "one index per lane, counter limit");
  const uint32_t eoff = static_cast<uint32_t>(e < D ? e : 0) * static_cast<uint32_t>(sizeof(SliceV));
  const uint32_t row_bytes = static_cast<uint32_t>(D * sizeof(SliceV));
  const char *base = reinterpret_cast<const char *>(src);
  j0 = __builtin_amdgcn_readfirstlane(j0);
  j1 = __builtin_amdgcn_readfirstlane(j1);
  if (j0 >= j1) return;
  uint32_t pv = slice_idx<P>(spos, j0, j1);
  for (int32_t j = j0; j < j1; j += P) {
    SliceV x[P];
#pragma unroll
    for (int u = 0; u < P; ++u) x[u] = slice_load(base, __builtin_amdgcn_readlane(pv, u), row_bytes, eoff);
    pv = slice_idx<P>(spos, j + P, j1);  // next batch's indices, behind this batch's rows
    __builtin_amdgcn_sched_barrier(0);     // keep both requests ahead of the consumption below
#pragma unroll
    for (int u = 0; u < P; ++u)
      if (j + u < j1) f(j + u, x[u]);
  }
}

// Narrow slices for long dependent chains.  A chain's speed is the number of
// its positions in flight, and a wave has at most 63 loads outstanding, so
// here one load instruction fetches G positions: the wave's lanes form G
// groups of 64/G lanes, group h reading position j + G*u + h of instruction u
// (a slice of 64/G elements, lane l holding element l % (64/G)).  Group 0 runs
// the chain: before each position is applied its value is moved from group h
// to group 0 with a lane permute (off the chain's dependency path).  The
// other groups' lanes run the same arithmetic on values that are dropped: the
// caller keeps only group 0's results.  Indices come in by vector loads of up
// to 64 positions and reach each group by lane permute.  P instructions per
// batch plus the index loads stay within the 63-load counter.
template <int G>
struct Narrow {
  static constexpr int kWidth = 64 / G;  // slice width in elements
  __host__ __device__ static constexpr int64_t slices(int64_t D) { return (D + kWidth - 1) / kWidth; }
};

// Row r (16 lanes) of x in row 0, by gfx950's row swaps (plain VALU
// operations): permlane16_swap moves row 1 onto row 0, permlane32_swap row 2,
// the two together row 3; the other rows receive values the caller drops.
__device__ __forceinline__ uint32_t row_to_row0(uint32_t x, int r) {
  if (r == 0) return x;
  if (r == 1) return __builtin_amdgcn_permlane16_swap(x, x, false, false)[1];
  const uint32_t y = __builtin_amdgcn_permlane32_swap(x, x, false, false)[1];
  if (r == 2) return y;
  return __builtin_amdgcn_permlane16_swap(y, y, false, false)[1];
}

// Group g's value (same lane within the group) in the lanes of group 0.  Two
// groups of 32 lanes are the wave's halves (one permlane32_swap: the walk the
// EMA uses); four groups of 16 lanes are the four rows; eight groups of 8
// lanes are the row halves: the group's row is brought to row 0, then an odd
// group's half is rotated onto lanes 0-7 (DPP row_ror:8).  Other group counts
// use a lane permute through LDS.
template <int G>
__device__ __forceinline__ float from_group(float x, int g, int lane) {
  if constexpr (G == 2) {  // two groups of 32 lanes: rows 2-3 onto rows 0-1
    return g == 0 ? x : __uint_as_float(row_to_row0(__float_as_uint(x), 2 * g));
  } else if constexpr (G == 4) {
    return __uint_as_float(row_to_row0(__float_as_uint(x), g));
  } else if constexpr (G == 8) {
    const uint32_t y = row_to_row0(__float_as_uint(x), g >> 1);
    if ((g & 1) == 0) return __uint_as_float(y);
    return __int_as_float(__builtin_amdgcn_mov_dpp(static_cast<int>(y), 0x128, 0xf, 0xf, false));
  } else {
    constexpr int W = 64 / G;
    return __shfl(x, g * W + (lane & (W - 1)));
  }
}

// Off32: src holds less than 2 GiB, so a position's element is addressed by a
// 32-bit byte offset from src through a buffer load.  With two lane groups the
// offsets are formed without a lane permute (below): a permute per position
// kept one address register live per distinct source lane, which with dozens
// of loads in flight set the walk's register count, hence the occupancy.
template <int G, int P, bool Off32, typename F>
__device__ __forceinline__ void slice_run_narrow(const float *__restrict__ src, const uint32_t *__restrict__ spos,
                                                 int32_t j0, int32_t j1, int64_t D, int64_t e, F f) {
  constexpr int W = 64 / G;
  constexpr int NP = G * P;
  constexpr int NI = (NP + 63) / 64;
  static_assert(64 % G == 0 && P + NI <= 63, "counter limit");
  const int lane = hlr::lane_id();
  const int h = lane / W;
  const int64_t ec = e < D ? e : 0;
  const uint32_t row_bytes = static_cast<uint32_t>(D * 4);
  const uint32_t ecol4 = static_cast<uint32_t>(ec) * 4u;
  j0 = __builtin_amdgcn_readfirstlane(j0);
  j1 = __builtin_amdgcn_readfirstlane(j1);
  if (j0 >= j1) return;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(src), 0, 0x7fffffff, 0x00020000);
  uint32_t pv[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int32_t jj = j0 + 64 * i + lane;
    pv[i] = spos[jj < j1 ? jj : j1 - 1];
  }
  for (int32_t j = j0; j < j1; j += NP) {
    SliceV x[P];
#pragma unroll
    for (int u = 0; u < P; ++u) {
      if constexpr (G == 2 && Off32) {
        // the two positions by readlane, their byte offsets in scalar registers, one select per lane: no
        // lane permute (one address register per distinct source lane, 32 of them here, all live)
        const int q = (2 * u) % 64;
        const uint32_t o0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(pv[(2 * u) / 64]), q));
        const uint32_t o1 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(pv[(2 * u) / 64]), q + 1));
        const uint32_t off = (h ? o1 * row_bytes : o0 * row_bytes) + ecol4;
        x[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
      } else {
        const uint32_t p = static_cast<uint32_t>(__shfl(static_cast<int>(pv[(G * u) / 64]), (G * u) % 64 + h));
        if (Off32)
          x[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, p * row_bytes + ecol4, 0, 0));
        else
          x[u] = src[static_cast<int64_t>(p) * D + ec];
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {  // next batch's indices, behind this batch's rows
      const int32_t jj = j + NP + 64 * i + lane;
      pv[i] = spos[jj < j1 ? jj : j1 - 1];
    }
    __builtin_amdgcn_sched_barrier(0);
    if (j + NP <= j1) {  // a full batch: no per-position condition
#pragma unroll
      for (int u = 0; u < P; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g) f(j + G * u + g, g == 0 ? x[u] : from_group<G>(x[u], g, lane));
    } else {
#pragma unroll
      for (int u = 0; u < P; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g)
          if (j + G * u + g < j1) f(j + G * u + g, g == 0 ? x[u] : from_group<G>(x[u], g, lane));
    }
  }
}

// Same, over rows given by an index function (partial results).
template <typename RowOf, typename F>
__device__ __forceinline__ void slice_run_rows(RowOf row_of, int32_t j0, int32_t j1, int64_t D, int64_t e, F f) {
  constexpr int P = 32;
  const int64_t ec = e < D ? e : 0;
  j0 = __builtin_amdgcn_readfirstlane(j0);
  j1 = __builtin_amdgcn_readfirstlane(j1);
  for (int32_t j = j0; j < j1; j += P) {
    SliceV x[P];
#pragma unroll
    for (int u = 0; u < P; ++u) x[u] = row_of(j + u < j1 ? j + u : j1 - 1)[ec];
#pragma unroll
    for (int u = 0; u < P; ++u)
      if (j + u < j1) f(j + u, x[u]);
  }
}

// Light rows: one wave per row, lanes own 16-byte units (columns lane + 64 q).
// rows_run() applies f(j, x) to positions j in [j0, j1) in order, loading P
// positions at a time with every load issued before any is used and no
// per-lane condition on a load (lanes past the row end read unit 0; their
// results are dropped by the caller).  Short tails go 4 at a time.
template <int P, int NC, typename F>
__device__ __forceinline__ void rows_run(const float4 *__restrict__ src, const uint32_t *__restrict__ spos,
                                         int32_t j0, int32_t j1, int64_t v4, int lane, F f) {
  int64_t col[NC];
#pragma unroll
  for (int q = 0; q < NC; ++q) col[q] = lane + q * hlr::kWave < v4 ? lane + q * hlr::kWave : 0;
  j0 = __builtin_amdgcn_readfirstlane(j0);
  j1 = __builtin_amdgcn_readfirstlane(j1);
  int32_t j = j0;
  for (; j + P <= j1; j += P) {
    int64_t p[P];
#pragma unroll
    for (int u = 0; u < P; ++u) p[u] = static_cast<int64_t>(spos[j + u]) * v4;
    float4 x[P][NC];
#pragma unroll
    for (int u = 0; u < P; ++u)
#pragma unroll
      for (int q = 0; q < NC; ++q) x[u][q] = src[p[u] + col[q]];
#pragma unroll
    for (int u = 0; u < P; ++u) f(j + u, x[u]);
  }
  const uint32_t last = j < j1 ? spos[j1 - 1] : 0u;
  for (; j < j1; j += 4) {
    int64_t p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) p[u] = spos[j + u];  // within the buffer's slack past n
#pragma unroll
    for (int u = 0; u < 4; ++u) p[u] = static_cast<int64_t>(j + u < j1 ? static_cast<uint32_t>(p[u]) : last) * v4;
    float4 x[4][NC];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int q = 0; q < NC; ++q) x[u][q] = src[p[u] + col[q]];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (j + u < j1) f(j + u, x[u]);
  }
}

// Registers a long segment (>= kHeavyMin occurrences, cut into runs of B) as
// work for the slice kernels: one entry (segment, run) per run, and the
// segment in the combine list when it has more than one run.  Called by one
// lane; counters[0] / counters[1] count the two lists (zeroed with the keys).
// Capacity: runs <= n/kHeavyMin + n/B <= n/32 for B >= 64.
__device__ __forceinline__ void push_heavy(int32_t k, int32_t len, int B, uint32_t *counters, int2 *hlist,
                                           int32_t *clist) {
  const int32_t nr = (len + B - 1) / B;
  const uint32_t base = atomicAdd(&counters[0], static_cast<uint32_t>(nr));
  for (int32_t m = 0; m < nr; ++m) hlist[base + m] = make_int2(k, m);
  if (nr > 1) clist[atomicAdd(&counters[1], 1u)] = k;
}

constexpr int kHeavyMin = 64;  // segments with at least this many occurrences go to the slice kernels
constexpr int kBaseRun = 256;  // the plan lists heavy segments in runs of this many occurrences

// The plan's heavy work list: every segment of at least kHeavyMin elements,
// cut into runs of kBaseRun (push_heavy), so that an apply knows its heavy
// work before it starts and can run it beside the light rows in one launch.
// Heavy segments are few (at most n / kHeavyMin), so one atomic per segment.
__global__ void __launch_bounds__(256)
    heavy_units_kernel(const int32_t *__restrict__ seg_start, const int32_t *__restrict__ seg_end,
                       const int64_t *__restrict__ nseg_p, uint32_t *ticket, int2 *hlist, int32_t *clist) {
  const int64_t nseg = *nseg_p;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t k = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; k < nseg; k += stride) {
    const int32_t len = seg_end[k] - seg_start[k];
    if (len >= kHeavyMin) push_heavy(static_cast<int32_t>(k), len, kBaseRun, ticket, hlist, clist);
  }
}

// After group_by_row: lists the heavy runs in hlist (count ticket[0]) and the
// segments of more than one run in clist (count ticket[1]).
inline void list_heavy_units(SegWork<uint32_t> &w, hipStream_t s) {
  int g = hlr::grid_for(w.n, 256);
  if (g > 1024) g = 1024;
  heavy_units_kernel<<<g, 256, 0, s>>>(w.seg_start, w.seg_end, w.nseg, w.ticket, w.hlist, w.clist);
}

// The plan's list of long segments for whole-segment chains (the SGD sum):
// segment k of length len >= kChainMin goes to the region of its length
// bucket; counts in ticket[4 + b].  Such segments are few, so one atomic each.
__global__ void __launch_bounds__(256)
    heavy_segments_kernel(const int32_t *__restrict__ seg_start, const int32_t *__restrict__ seg_end,
                          const int64_t *__restrict__ nseg_p, int64_t n, uint32_t *ticket, int32_t *slist) {
  const int64_t nseg = *nseg_p;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t k = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; k < nseg; k += stride) {
    const int32_t len = seg_end[k] - seg_start[k];
    if (len < kChainMin) continue;
    int b = 31 - __builtin_clz(static_cast<uint32_t>(len)) - kLenShift;
    b = b < kLenBuckets - 1 ? b : kLenBuckets - 1;
    const uint32_t slot = atomicAdd(&ticket[4 + b], 1u);
    slist[len_bucket_off(n, b) + slot] = static_cast<int32_t>(k);
  }
}

// After group_by_row: lists the heavy segments by length bucket (slist).
inline void list_heavy_segments(SegWork<uint32_t> &w, hipStream_t s) {
  int g = hlr::grid_for(w.n, 256);
  if (g > 1024) g = 1024;
  heavy_segments_kernel<<<g, 256, 0, s>>>(w.seg_start, w.seg_end, w.nseg, w.n, w.ticket, w.slist);
}

// Heavy-segment work item it of a plan (items = segments x S slices, the
// longest length bucket first): the segment and the slice.  Returns false
// past the last item.  cnt[b] = ticket[4 + b].
__device__ __forceinline__ bool heavy_item(const uint32_t (&cnt)[kLenBuckets], const int32_t *__restrict__ slist,
                                           int64_t n, int64_t S, int64_t it, int32_t *seg, int64_t *slice) {
  int64_t off = len_bucket_off(n, kLenBuckets);
#pragma unroll
  for (int b = kLenBuckets - 1; b >= 0; --b) {
    off -= len_bucket_cap(n, b);
    const int64_t c = static_cast<int64_t>(cnt[b]) * S;
    if (it < c) {
      *seg = slist[off + it / S];
      *slice = it % S;
      return true;
    }
    it -= c;
  }
  return false;
}

// Long running sums (the SGD sum of a hot row, one dependent fp32 chain per
// element): one element per 16-lane row of the wave (row r takes element
// el_r), 16 positions per load instruction.  Lane l of a row reads position
// j + 16u + l of instruction u; the chain runs in lane 0 of each row.  The 16
// values of a row reach lane 0 through LDS: every lane writes its value to
// the wave's slot, and each lane reads its row's 16 values back as four
// 16-byte reads (a broadcast within the row), so the chain itself is 16 plain
// dependent adds per instruction.  (Folding a DPP row shift into each add
// instead makes every add wait for the cross-lane network: about 14 cycles
// per dependent add on this GPU against about 6 for a plain add.)  The sum
// starts from -0.0 and positions past j1 read -0.0: -0.0 is the identity of
// IEEE addition (s + -0.0 == s for every s, signed zeros included), so the
// result equals the running sum started from the first value, and every batch
// is the same straight-line code.  Indices come in by vector loads of 64
// positions and reach each row by a lane permute; P load instructions per
// batch plus P / 4 index loads stay within the 63-load counter.  (Double
// buffering two batches of half the size measured slower on the hashed-tables
// step; the caller's batch size is measured too: more positions in flight per
// batch is not faster here.)  grad(x) turns
// a loaded value into the term summed (the L2-alignment gradient).  lds: this
// wave's kChainSlots * 64 floats.  Only lane 0 of each row returns a
// meaningful sum.
constexpr int kChainSlots = 4;

// Instruction u of a batch through LDS: each lane writes its term (-0.0 past
// j1) to the slot of u, then reads its row's 16 terms back.
template <typename Grad>
__device__ __forceinline__ void stage1(float *lds, int u, int32_t j, int32_t j1, int l, int lane, int r16, float x,
                                       Grad grad, float4 (&out)[4]) {
  float *sl = lds + (u % kChainSlots) * 64;
  sl[lane] = j + 16 * u + l < j1 ? grad(x) : -0.0f;
  __builtin_amdgcn_wave_barrier();
  const float4 *q = reinterpret_cast<const float4 *>(sl + r16);
#pragma unroll
  for (int k = 0; k < 4; ++k) out[k] = q[k];
  __builtin_amdgcn_wave_barrier();
}

template <int P, bool Off32, typename Grad>
__device__ __forceinline__ float chain_sum16(const float *__restrict__ src, const uint32_t *__restrict__ spos,
                                             int32_t j0, int32_t j1, int64_t D, int64_t el, float *lds, Grad grad) {
  constexpr int NP = 16 * P;
  constexpr int NI = NP / 64;
  static_assert(P % 4 == 0 && P + NI <= 63, "counter limit");
  const int lane = hlr::lane_id();
  const int l = lane & 15;
  const int r16 = lane & ~15;
  const uint32_t ecol = static_cast<uint32_t>(el < D ? el : 0);
  const uint32_t row_bytes = static_cast<uint32_t>(D * 4);
  j0 = __builtin_amdgcn_readfirstlane(j0);
  j1 = __builtin_amdgcn_readfirstlane(j1);
  float s = -0.0f;
  if (j0 >= j1) return s;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(src), 0, 0x7fffffff, 0x00020000);
  uint32_t pv[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int32_t jj = j0 + 64 * i + lane;
    pv[i] = spos[jj < j1 ? jj : j1 - 1];
  }
  for (int32_t j = j0; j < j1; j += NP) {
    float x[P];
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const uint32_t p = static_cast<uint32_t>(__shfl(static_cast<int>(pv[u / 4]), 16 * (u % 4) + l));
      if (Off32) {
        x[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, p * row_bytes + ecol * 4, 0, 0));
      } else {
        x[u] = src[static_cast<int64_t>(p) * D + ecol];
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {  // next batch's indices, behind this batch's rows
      const int32_t jj = j + NP + 64 * i + lane;
      pv[i] = spos[jj < j1 ? jj : j1 - 1];
    }
    __builtin_amdgcn_sched_barrier(0);
    // The next instruction's terms are written and read back before the
    // current one's adds, so the LDS round trip hides behind them.
    float4 cur[4], nxt[4];
    stage1(lds, 0, j, j1, l, lane, r16, x[0], grad, cur);
#pragma unroll
    for (int u = 0; u < P; ++u) {
      if (u + 1 < P) stage1(lds, u + 1, j, j1, l, lane, r16, x[u + 1], grad, nxt);
      __builtin_amdgcn_sched_barrier(0);  // keep the next stage's LDS traffic ahead of these adds
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        s = s + cur[q].x;
        s = s + cur[q].y;
        s = s + cur[q].z;
        s = s + cur[q].w;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) cur[q] = nxt[q];
    }
  }
  return s;
}

}  // namespace
