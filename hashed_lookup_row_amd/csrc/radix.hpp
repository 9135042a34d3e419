// Stable LSD radix sort of (key, position) pairs and the segment table of the
// sorted keys.  Used to group a batch's positions by key (dedup) or by row
// (duplicate-summed SGD, EMA), positions ascending inside every group.
//
// Per pass: hist_kernel (per-tile digit histograms; the last tile to finish
// turns the digit-major count matrix into exclusive offsets) and
// scatter_kernel (stable ranks inside the tile from wave ballots + per-wave
// LDS counters).  Digits are 8..11 bits, chosen so the key width is covered in
// ceil(bits/11) passes.
#pragma once

#include "hlr_common.hpp"

namespace {

constexpr int kSortThreads = 256;
constexpr int kSortItems = 16;
constexpr int kSortTile = kSortThreads * kSortItems;  // 4096 elements per tile
constexpr int kMaxDigitBits = 11;
constexpr int kMaxBins = 1 << kMaxDigitBits;

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
  uint32_t *ticket;  // [4]
  uint32_t *bcount;  // [nblocks]
  int32_t *segidx;   // [n]   segment of each sorted element (-1: excluded)
  int32_t *seg_start;  // [n]
  int32_t *seg_end;    // [n]
  int64_t *nseg;       // [1]
  int64_t n;
  int nblocks;
};

template <typename K>
inline size_t segwork_layout(int64_t n, SegWork<K> *w, void *base) {
  hlr::Carver c(base);
  const int nb = static_cast<int>((n + kSortTile - 1) / kSortTile);
  const size_t nn = static_cast<size_t>(n > 0 ? n : 1);
  w->k[0] = c.take<K>(nn);
  w->k[1] = c.take<K>(nn);
  w->v[0] = c.take<uint32_t>(nn);
  w->v[1] = c.take<uint32_t>(nn);
  w->counts = c.take<uint32_t>(static_cast<size_t>(kMaxBins) * (nb > 0 ? nb : 1));
  w->ticket = c.take<uint32_t>(4);
  w->bcount = c.take<uint32_t>(2 * static_cast<size_t>(nb > 0 ? nb : 1));
  w->segidx = c.take<int32_t>(nn);
  w->seg_start = c.take<int32_t>(nn);
  w->seg_end = c.take<int32_t>(nn);
  w->nseg = c.take<int64_t>(1);
  w->n = n;
  w->nblocks = nb;
  return c.off;
}

// ------------------------------------------------------------------ kernels
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

template <typename K>
__global__ void __launch_bounds__(kSortThreads)
    hist_kernel(const K *__restrict__ keys, int64_t n, int shift, int bits, uint32_t *counts, int nblocks,
                uint32_t *ticket) {
  __shared__ uint32_t h[kMaxBins];
  __shared__ uint32_t sh[kSortThreads];
  __shared__ int is_last;
  const int bins = 1 << bits;
  const uint32_t mask = static_cast<uint32_t>(bins - 1);
  for (int d = threadIdx.x; d < bins; d += kSortThreads) h[d] = 0;
  __syncthreads();
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kSortTile;
#pragma unroll
  for (int k = 0; k < kSortItems; ++k) {
    const int64_t idx = base + k * kSortThreads + threadIdx.x;
    if (idx < n) atomicAdd(&h[static_cast<uint32_t>(keys[idx] >> shift) & mask], 1u);
  }
  __syncthreads();
  for (int d = threadIdx.x; d < bins; d += kSortThreads) counts[static_cast<int64_t>(d) * nblocks + blockIdx.x] = h[d];
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) is_last = (atomicAdd(ticket, 1u) == static_cast<uint32_t>(nblocks - 1));
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  // Digit totals, then an exclusive scan over digits, then per-(digit, tile) offsets.
  for (int d = threadIdx.x; d < bins; d += kSortThreads) {
    uint32_t s = 0;
    for (int b = 0; b < nblocks; ++b) s += counts[static_cast<int64_t>(d) * nblocks + b];
    h[d] = s;
  }
  __syncthreads();
  const int per = (bins + kSortThreads - 1) / kSortThreads;
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) {
    const int d = threadIdx.x * per + i;
    if (d < bins) local += h[d];
  }
  uint32_t tot;
  uint32_t run = block_exclusive_scan(local, sh, &tot);
  for (int i = 0; i < per; ++i) {
    const int d = threadIdx.x * per + i;
    if (d < bins) {
      const uint32_t c = h[d];
      h[d] = run;
      run += c;
    }
  }
  __syncthreads();
  for (int d = threadIdx.x; d < bins; d += kSortThreads) {
    uint32_t r = h[d];
    for (int b = 0; b < nblocks; ++b) {
      const int64_t at = static_cast<int64_t>(d) * nblocks + b;
      const uint32_t c = counts[at];
      counts[at] = r;
      r += c;
    }
  }
  if (threadIdx.x == 0) *ticket = 0u;
}

template <typename K>
__global__ void __launch_bounds__(kSortThreads)
    scatter_kernel(const K *__restrict__ kin, const uint32_t *__restrict__ vin, K *__restrict__ kout,
                   uint32_t *__restrict__ vout, int64_t n, int shift, int bits, const uint32_t *__restrict__ offsets,
                   int nblocks) {
  __shared__ uint32_t cnt[4][kMaxBins];
  const int bins = 1 << bits;
  const uint32_t mask = static_cast<uint32_t>(bins - 1);
  const int w = threadIdx.x >> 6;
  for (int x = threadIdx.x; x < 4 * bins; x += kSortThreads) cnt[x / bins][x % bins] = 0;
  __syncthreads();
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kSortTile + w * (kSortTile / 4);
  const uint64_t lt = hlr::lanemask_lt();
  K kk[kSortItems];
  uint32_t vv[kSortItems];
  uint32_t rk[kSortItems];
#pragma unroll
  for (int r = 0; r < kSortItems; ++r) {
    const int64_t idx = base + r * hlr::kWave + hlr::lane_id();
    const bool valid = idx < n;
    const K k = valid ? kin[idx] : K(0);
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
    vv[r] = valid ? vin[idx] : 0u;
    rk[r] = prev + rin;
  }
  __syncthreads();
  for (int d = threadIdx.x; d < bins; d += kSortThreads) {
    uint32_t run = offsets[static_cast<int64_t>(d) * nblocks + blockIdx.x];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t c = cnt[q][d];
      cnt[q][d] = run;
      run += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kSortItems; ++r) {
    const int64_t idx = base + r * hlr::kWave + hlr::lane_id();
    if (idx < n) {
      const uint32_t d = static_cast<uint32_t>(kk[r] >> shift) & mask;
      const uint32_t dst = cnt[w][d] + rk[r];
      kout[dst] = kk[r];
      vout[dst] = vv[r];
    }
  }
}

// Segment pass 1: number of segment heads per tile; the last tile turns the
// counts into exclusive tile offsets (bcount[nblocks + b]) and the total.
// Elements whose key equals `excluded` belong to no segment.
template <typename K>
__global__ void __launch_bounds__(kSortThreads)
    seg_count_kernel(const K *__restrict__ keys, int64_t n, K excluded, bool use_excluded, uint32_t *bcount,
                     int nblocks, uint32_t *ticket, int64_t *nseg) {
  __shared__ uint32_t sh[kSortThreads];
  __shared__ int is_last;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kSortTile + threadIdx.x * kSortItems;
  uint32_t c = 0;
  for (int i = 0; i < kSortItems; ++i) {
    const int64_t j = base + i;
    if (j < n) {
      const K k = keys[j];
      const bool ok = !(use_excluded && k == excluded);
      const bool head = ok && (j == 0 || keys[j - 1] != k);
      c += head ? 1u : 0u;
    }
  }
  uint32_t tot;
  block_exclusive_scan(c, sh, &tot);
  if (threadIdx.x == 0) bcount[blockIdx.x] = tot;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) is_last = (atomicAdd(ticket, 1u) == static_cast<uint32_t>(nblocks - 1));
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (int b = 0; b < nblocks; ++b) {
      const uint32_t x = bcount[b];
      bcount[nblocks + b] = run;
      run += x;
    }
    *nseg = run;
    *ticket = 0u;
  }
}

// Segment pass 2: per sorted element its segment index; heads and tails record
// the segment bounds.  The functor `emit(j, seg, head, tail, key, val)` adds
// mode-specific outputs (dedup: unique keys, last positions, inverse).
template <typename K, typename Emit>
__global__ void __launch_bounds__(kSortThreads)
    seg_index_kernel(const K *__restrict__ keys, const uint32_t *__restrict__ vals, int64_t n, K excluded,
                     bool use_excluded, const uint32_t *__restrict__ bcount, int nblocks, int32_t *segidx,
                     int32_t *seg_start, int32_t *seg_end, Emit emit) {
  __shared__ uint32_t sh[kSortThreads];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kSortTile + threadIdx.x * kSortItems;
  uint32_t c = 0;
  for (int i = 0; i < kSortItems; ++i) {
    const int64_t j = base + i;
    if (j < n) {
      const K k = keys[j];
      const bool ok = !(use_excluded && k == excluded);
      c += (ok && (j == 0 || keys[j - 1] != k)) ? 1u : 0u;
    }
  }
  uint32_t tot;
  uint32_t run = block_exclusive_scan(c, sh, &tot) + bcount[nblocks + blockIdx.x];
  for (int i = 0; i < kSortItems; ++i) {
    const int64_t j = base + i;
    if (j >= n) break;
    const K k = keys[j];
    const bool ok = !(use_excluded && k == excluded);
    if (!ok) {
      segidx[j] = -1;
      continue;
    }
    const bool head = (j == 0 || keys[j - 1] != k);
    const bool tail = (j == n - 1 || keys[j + 1] != k);
    if (head) ++run;
    const int32_t seg = static_cast<int32_t>(run) - 1;
    segidx[j] = seg;
    if (head) seg_start[seg] = static_cast<int32_t>(j);
    if (tail) seg_end[seg] = static_cast<int32_t>(j + 1);
    emit(j, seg, head, tail, k, vals[j]);
  }
}

struct NoEmit {
  template <typename K>
  __device__ void operator()(int64_t, int32_t, bool, bool, K, uint32_t) const {}
};

// Runs every radix pass; returns the index (0/1) of the buffer holding the result.
template <typename K>
inline int radix_sort_pairs(SegWork<K> &w, int total_bits, hipStream_t s) {
  const SortPlan plan = make_plan(total_bits);
  int cur = 0;
  for (int p = 0; p < plan.passes; ++p) {
    hist_kernel<K><<<w.nblocks, kSortThreads, 0, s>>>(w.k[cur], w.n, plan.shift[p], plan.bits[p], w.counts,
                                                       w.nblocks, w.ticket);
    scatter_kernel<K><<<w.nblocks, kSortThreads, 0, s>>>(w.k[cur], w.v[cur], w.k[cur ^ 1], w.v[cur ^ 1], w.n,
                                                          plan.shift[p], plan.bits[p], w.counts, w.nblocks);
    cur ^= 1;
  }
  return cur;
}

template <typename K, typename Emit>
inline void segment_sorted(SegWork<K> &w, int cur, K excluded, bool use_excluded, Emit emit, hipStream_t s) {
  seg_count_kernel<K><<<w.nblocks, kSortThreads, 0, s>>>(w.k[cur], w.n, excluded, use_excluded, w.bcount,
                                                          w.nblocks, w.ticket, w.nseg);
  seg_index_kernel<K, Emit><<<w.nblocks, kSortThreads, 0, s>>>(w.k[cur], w.v[cur], w.n, excluded, use_excluded,
                                                                w.bcount, w.nblocks, w.segidx, w.seg_start,
                                                                w.seg_end, emit);
}

}  // namespace

namespace {

// Sort keys for grouping a batch by row: row r for positions that take part
// (row in range, mask set), the sentinel num_rows (sorted last, excluded from
// every segment) for the others.
__global__ void __launch_bounds__(256)
    rowkey_init(const int64_t *__restrict__ rows, const uint8_t *__restrict__ mask, int64_t n, int64_t num_rows,
                uint32_t *__restrict__ k, uint32_t *__restrict__ v, uint32_t *ticket) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) {
    const int64_t r = rows[i];
    const bool ok = r >= 0 && r < num_rows && (mask == nullptr || mask[i] != 0);
    k[i] = ok ? static_cast<uint32_t>(r) : static_cast<uint32_t>(num_rows);
    v[i] = static_cast<uint32_t>(i);
  }
  if (i < 4) ticket[i] = 0u;
}

// Groups positions by row: returns the buffer index holding (row, position)
// sorted by row, positions ascending within a row, with the segment table
// (seg_start, seg_end, nseg) built.
inline int group_by_row(SegWork<uint32_t> &w, const int64_t *rows, const uint8_t *mask, int64_t num_rows,
                        hipStream_t s) {
  rowkey_init<<<hlr::grid_for(w.n, 256), 256, 0, s>>>(rows, mask, w.n, num_rows, w.k[0], w.v[0], w.ticket);
  const int bits = bit_width_u64(static_cast<uint64_t>(num_rows));
  const int cur = radix_sort_pairs<uint32_t>(w, bits, s);
  segment_sorted<uint32_t>(w, cur, static_cast<uint32_t>(num_rows), true, NoEmit{}, s);
  return cur;
}

}  // namespace
