// Decoupled, growable key store ("MTGR: Industrial-Scale Generative
// Recommendation Framework in Meituan", sec. 3.2): a light key store maps raw
// keys to rows of a separate value store (rows plus their metadata, here the
// last batch that touched each row); growing the key store copies keys only.
//
// Key store: open addressing over key_cap (a power of two) slots, linear
// probing from the SplitMix64 finaliser of the key; key -1 marks an empty slot.
// Value store: rows handed out in order (next_row, a device counter, at most
// max_rows).  One batch, two phases: keys already stored are hits; then the
// distinct missed keys, in order of first occurrence, take the next rows.
//   ks_init    clear the batch's miss table; copy next_row; zero the stats
//   ks_probe   thread per position: probe the key store; a miss registers its
//              key in the miss table (CAS) with its first position (atomicMin)
//   ks_count   per tile of 256 positions: first occurrences of missed keys
//   ks_assign  ranks of first occurrences (earlier tiles + wave ballots) give
//              the rows; the key is inserted (CAS on an empty slot) and the row
//              stamped and zero-filled; the last tile advances next_row
//   ks_resolve every missed position takes its key's row
//   ks_rehash  re-inserts every stored key into a larger key store
#include "hlr_common.hpp"

namespace {
using namespace hlr;

constexpr int kThreads = 256;
constexpr int32_t kNoPos = 0x7fffffff;

struct KSWork {
  int64_t *mkey;    // miss table: key (-1 free)
  int32_t *mfirst;  // first position of the key in the batch
  int64_t *mrow;    // row given to the key (-1: overflow)
  int32_t *pent;    // [n] miss-table entry of each position (-1: none)
  uint32_t *bcnt;   // [tiles] first occurrences per tile
  int64_t *base;    // [1] next_row at batch start
  uint64_t mcap;
  int tiles;
};

size_t ks_layout(int64_t n, KSWork *w, void *base) {
  Carver c(base);
  const uint64_t mcap = next_pow2(static_cast<uint64_t>(n > 32 ? 2 * n : 64));
  const int tiles = static_cast<int>((n + kThreads - 1) / kThreads);
  w->mkey = c.take<int64_t>(mcap);
  w->mfirst = c.take<int32_t>(mcap);
  w->mrow = c.take<int64_t>(mcap);
  w->pent = c.take<int32_t>(static_cast<size_t>(n > 0 ? n : 1));
  w->bcnt = c.take<uint32_t>(static_cast<size_t>(tiles > 0 ? tiles : 1));
  w->base = c.take<int64_t>(1);
  w->mcap = mcap;
  w->tiles = tiles;
  return c.off;
}

__device__ __forceinline__ void add_stat(unsigned long long *stats, int k, bool pred) {
  if (stats) wave_count(&stats[k], pred);
}

__global__ void __launch_bounds__(kThreads) ks_init(KSWork w, const int64_t *next_row, unsigned long long *stats) {
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kThreads;
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x; i < w.mcap; i += stride) {
    w.mkey[i] = -1;
    w.mfirst[i] = kNoPos;
    w.mrow[i] = -1;
  }
  if (blockIdx.x == 0 && threadIdx.x < 4 && stats) stats[threadIdx.x] = 0ull;
  if (blockIdx.x == 0 && threadIdx.x == 0) *w.base = *next_row;
}

__global__ void ks_zero_stats(unsigned long long *stats) {
  if (threadIdx.x < 4) stats[threadIdx.x] = 0ull;
}

__global__ void __launch_bounds__(kThreads)
    ks_probe(const int64_t *__restrict__ keys, const int64_t *__restrict__ krows, uint64_t key_cap,
             int64_t *stamps, int64_t max_rows, const int64_t *__restrict__ ids, int64_t n, int64_t now, int insert,
             int64_t *rows, int8_t *hit, KSWork w, unsigned long long *stats) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  bool is_hit = false, invalid = false;
  if (i < n) {
    const int64_t id = ids[i];
    int64_t row = -1;
    int32_t ent = -1;
    if (id == -1) {
      invalid = true;
    } else {
      const uint64_t mask = key_cap - 1;
      uint64_t s = mix64(static_cast<uint64_t>(id)) & mask;
      bool miss = false;
      for (uint64_t j = 0; j < key_cap; ++j) {
        const int64_t k = keys[s];
        if (k == id) {
          row = krows[s];
          break;
        }
        if (k == -1) {
          miss = true;
          break;
        }
        s = (s + 1) & mask;
      }
      if (row >= 0 && row < max_rows) {
        is_hit = true;
        if (insert) stamps[row] = now;
      } else {
        row = -1;
        if (insert && miss) {
          const uint64_t mm = w.mcap - 1;
          uint64_t e = (mix64(static_cast<uint64_t>(id)) >> 32) & mm;
          for (;;) {
            const int64_t prev = atomic_cas_i64(&w.mkey[e], -1, id);
            if (prev == -1 || prev == id) break;
            e = (e + 1) & mm;
          }
          atomicMin(&w.mfirst[e], static_cast<int32_t>(i));
          ent = static_cast<int32_t>(e);
        }
      }
    }
    rows[i] = row;
    hit[i] = is_hit ? 1 : 0;
    if (insert) w.pent[i] = ent;
  }
  add_stat(stats, 0, is_hit);
  add_stat(stats, 3, invalid);
}

__device__ __forceinline__ bool first_miss(const KSWork &w, int64_t i, int64_t n) {
  if (i >= n) return false;
  const int32_t e = w.pent[i];
  return e >= 0 && w.mfirst[e] == static_cast<int32_t>(i);
}

__global__ void __launch_bounds__(kThreads) ks_count(KSWork w, int64_t n) {
  __shared__ uint32_t wsum[kThreads / kWave];
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const uint32_t c = static_cast<uint32_t>(__popcll(ballot(first_miss(w, i, n))));
  if (lane_id() == 0) wsum[threadIdx.x / kWave] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int q = 0; q < kThreads / kWave; ++q) t += wsum[q];
    w.bcnt[blockIdx.x] = t;
  }
}

__global__ void __launch_bounds__(kThreads)
    ks_assign(int64_t *keys, int64_t *krows, uint64_t key_cap, int64_t *stamps, float4 *values, int64_t v4,
              int64_t max_rows, int64_t *next_row, const int64_t *__restrict__ ids, int64_t n, int64_t now, KSWork w,
              unsigned long long *stats) {
  __shared__ uint32_t red[kThreads];
  __shared__ uint32_t wcnt[kThreads / kWave];
  __shared__ uint32_t before_blk, total_all;
  // first occurrences in earlier tiles, and in all tiles
  uint32_t before = 0, total = 0;
  for (int b = threadIdx.x; b < w.tiles; b += kThreads) {
    const uint32_t v = w.bcnt[b];
    if (b < static_cast<int>(blockIdx.x)) before += v;
    total += v;
  }
  red[threadIdx.x] = before;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) before_blk = red[0];
  __syncthreads();
  red[threadIdx.x] = total;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) total_all = red[0];
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const bool first = first_miss(w, i, n);
  const uint64_t bal = ballot(first);
  const int wv = threadIdx.x / kWave;
  if (lane_id() == 0) wcnt[wv] = static_cast<uint32_t>(__popcll(bal));
  __syncthreads();
  uint32_t rank = before_blk + static_cast<uint32_t>(__popcll(bal & lanemask_lt()));
  for (int q = 0; q < wv; ++q) rank += wcnt[q];
  const int64_t base = *w.base;
  const int64_t avail = max_rows - base;
  int64_t row = -1;
  if (first) {
    const int64_t id = ids[i];
    const int32_t e = w.pent[i];
    if (static_cast<int64_t>(rank) < avail) {
      row = base + static_cast<int64_t>(rank);
      const uint64_t mask = key_cap - 1;
      uint64_t s = mix64(static_cast<uint64_t>(id)) & mask;
      for (uint64_t j = 0; j < key_cap; ++j) {
        if (atomic_cas_i64(&keys[s], -1, id) == -1) {
          krows[s] = row;
          break;
        }
        s = (s + 1) & mask;
      }
      stamps[row] = now;
    }
    w.mrow[e] = row;
  }
  // the wave zero-fills each new row with 16-byte stores
  if (values) {
    uint64_t m = ballot(row >= 0);
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    while (m) {
      const int l = __builtin_ctzll(m);
      m &= m - 1;
      float4 *dst = values + readlane_i64(row, l) * v4;
      for (int64_t c = lane_id(); c < v4; c += kWave) dst[c] = z;
    }
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) {
    const int64_t tot = static_cast<int64_t>(total_all);
    const int64_t ins = tot < avail ? tot : (avail > 0 ? avail : 0);
    *next_row = base + ins;
    if (stats) {
      stats[1] = static_cast<unsigned long long>(ins);
      stats[2] = static_cast<unsigned long long>(tot - ins);
    }
  }
}

__global__ void __launch_bounds__(kThreads) ks_resolve(KSWork w, int64_t n, int64_t *rows) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i < n) {
    const int32_t e = w.pent[i];
    if (e >= 0) rows[i] = w.mrow[e];
  }
}

__global__ void __launch_bounds__(kThreads)
    ks_rehash(const int64_t *__restrict__ keys, const int64_t *__restrict__ krows, uint64_t key_cap, int64_t *nkeys,
              int64_t *nkrows, uint64_t new_cap) {
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kThreads;
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x; i < key_cap; i += stride) {
    const int64_t id = keys[i];
    if (id == -1) continue;
    const uint64_t mask = new_cap - 1;
    uint64_t s = mix64(static_cast<uint64_t>(id)) & mask;
    for (uint64_t j = 0; j < new_cap; ++j) {
      if (atomic_cas_i64(&nkeys[s], -1, id) == -1) {
        nkrows[s] = krows[i];
        break;
      }
      s = (s + 1) & mask;
    }
  }
}

bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

}  // namespace

extern "C" size_t dks_workspace_size(int64_t n) {
  if (n < 0) return 0;
  KSWork w;
  return ks_layout(n, &w, nullptr);
}

extern "C" hlr_status dks_lookup_or_insert(int64_t *keys, int64_t *krows, int64_t key_cap, int64_t *stamps,
                                           float *values, int64_t dim, int64_t max_rows, int64_t *next_row,
                                           const int64_t *ids, int64_t n, int64_t now, int32_t insert,
                                           int64_t *out_rows, int8_t *out_hit, int64_t *out_stats, void *ws,
                                           size_t ws_bytes, hipStream_t stream) {
  if (n < 0 || n > kMaxN || !pow2(key_cap) || max_rows < 0 || (insert != 0 && insert != 1)) return HLR_INVALID_ARG;
  if (!keys || !krows || (insert && (!stamps || !next_row))) return HLR_INVALID_ARG;
  if (n > 0 && (!ids || !out_rows || !out_hit)) return HLR_INVALID_ARG;
  if (values && (dim <= 0 || dim % 4 != 0)) return HLR_UNSUPPORTED_DIM;
  if (!aligned(keys, 8) || !aligned(krows, 8) || (stamps && !aligned(stamps, 8)) ||
      (next_row && !aligned(next_row, 8)) || (ids && !aligned(ids, 8)) || (out_rows && !aligned(out_rows, 8)) ||
      (out_stats && !aligned(out_stats, 8)) || (values && !aligned(values, 16)))
    return HLR_MISALIGNED;
  unsigned long long *stats = reinterpret_cast<unsigned long long *>(out_stats);
  KSWork w{};
  if (insert) {
    const size_t need = ks_layout(n, &w, nullptr);
    if (!ws || ws_bytes < need) return HLR_WORKSPACE_TOO_SMALL;
    if (!aligned(ws, 256)) return HLR_MISALIGNED;
    ks_layout(n, &w, ws);
    int gi = grid_for(static_cast<int64_t>(w.mcap), kThreads);
    if (gi > 4096) gi = 4096;
    ks_init<<<gi, kThreads, 0, stream>>>(w, next_row, stats);
  } else if (stats) {
    ks_zero_stats<<<1, 64, 0, stream>>>(stats);
  }
  if (n == 0) return launch_status();
  const int g = grid_for(n, kThreads);
  ks_probe<<<g, kThreads, 0, stream>>>(keys, krows, static_cast<uint64_t>(key_cap), stamps, max_rows, ids, n, now,
                                       insert, out_rows, out_hit, w, stats);
  if (!insert) return launch_status();
  ks_count<<<g, kThreads, 0, stream>>>(w, n);
  ks_assign<<<g, kThreads, 0, stream>>>(keys, krows, static_cast<uint64_t>(key_cap), stamps,
                                        reinterpret_cast<float4 *>(values), values ? dim / 4 : 0, max_rows, next_row,
                                        ids, n, now, w, stats);
  ks_resolve<<<g, kThreads, 0, stream>>>(w, n, out_rows);
  return launch_status();
}

extern "C" hlr_status dks_rehash(const int64_t *keys, const int64_t *krows, int64_t key_cap, int64_t *new_keys,
                                 int64_t *new_krows, int64_t new_cap, hipStream_t stream) {
  if (!pow2(key_cap) || !pow2(new_cap) || new_cap < key_cap) return HLR_INVALID_ARG;
  if (!keys || !krows || !new_keys || !new_krows) return HLR_INVALID_ARG;
  if (!aligned(keys, 8) || !aligned(krows, 8) || !aligned(new_keys, 8) || !aligned(new_krows, 8))
    return HLR_MISALIGNED;
  hlr_fill(new_keys, new_cap, int64_t(-1), stream);
  int g = grid_for(key_cap, kThreads);
  if (g > 8192) g = 8192;
  ks_rehash<<<g, kThreads, 0, stream>>>(keys, krows, static_cast<uint64_t>(key_cap), new_keys, new_krows,
                                        static_cast<uint64_t>(new_cap));
  return launch_status();
}
