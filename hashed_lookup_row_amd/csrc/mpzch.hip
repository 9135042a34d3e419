// MPZCH lookup / insert with LRU eviction.
//
// "Memory Layer: Train the In-Model Cache for Recommendation Models", sec. 2:
// an identity tensor maps raw item IDs to rows with no collisions (one ID per
// row), capacity is bounded, rows are recycled least-recently-used, and the
// LRU metadata shares the row index.
//
// A batch is applied in two phases.  Phase 1 (probe): every ID resident at
// batch start hits and pins its slot (stamp = now).  Phase 2: the distinct
// missed IDs of each bucket, in order of first occurrence, take the bucket's
// slots in preference order — empty slots by probe index, then unpinned slots
// by (stamp, probe index) — one per ID; the rest overflow.  Taking the k-th
// preferred slot for the k-th new ID is exactly the serial
// first-empty-else-LRU rule, because every insert pins the slot it takes.
//
// GPU plan (all on one stream, no host sync):
//   mz_init    clear the transient miss table and bucket table
//   mz_probe   one lane per position: bucket probe, hit + pin, or register
//              the miss (hash table keyed by ID, atomicMin of first position);
//              the lane that creates an ID's entry links it into its bucket's
//              list (hash table keyed by bucket, atomicExch list push)
//   mz_assign  one lane per bucket with pending IDs: picks the IDs with the
//              smallest first positions, commits them with atomic CAS on the
//              identity slot (a failed CAS would mean a broken invariant and
//              is counted), stamps them, records the displaced ID
//   mz_resolve one lane per missed position: row of its ID; the first
//              occurrence reports the eviction and the wave zero-fills the
//              new row cooperatively (16-byte stores); an extra block folds the
//              per-block partial counts of probe and assign into the stats
// Counts are kept per block and folded once, never with same-address global
// atomics (those serialise at the memory side).
#include <mutex>

#include "hlr_common.hpp"
#include "mlwork.hpp"
#include "step_parts.hpp"

namespace {
using namespace hlr;

constexpr int kMaxProbes = 32;
constexpr int kThreads = 256;

struct MZWork {
  int64_t *mkey;   // miss table: ID (-1 = free)
  int32_t *mfpos;  // first occurrence of the ID in the batch
  int32_t *mnext;  // next entry of the same bucket (-1 = end)
  int64_t *mslot;  // slot given to the ID (-1 = overflow)
  int64_t *mevict; // ID displaced by the insert (-1 = slot was empty)
  int64_t *bkey;   // bucket table: bucket index (-1 = free)
  int32_t *bhead;  // first miss-table entry of the bucket's list
  int32_t *pent;   // per position: miss-table entry, -1 = hit / invalid
  uint32_t *part;  // per-block partial counts: probe blocks x 2, then assign blocks x 4
  uint32_t cap;    // entries of each hash table (power of two)
  uint32_t probe_blocks;
};

constexpr int kAssignMaxBlocks = 1024;

size_t mz_layout(int64_t n, MZWork *w, void *base) {
  Carver c(base);
  const uint64_t cap = next_pow2(static_cast<uint64_t>(n > 32 ? 2 * n : 64));
  w->mkey = c.take<int64_t>(cap);
  w->mfpos = c.take<int32_t>(cap);
  w->mnext = c.take<int32_t>(cap);
  w->mslot = c.take<int64_t>(cap);
  w->mevict = c.take<int64_t>(cap);
  w->bkey = c.take<int64_t>(cap);
  w->bhead = c.take<int32_t>(cap);
  w->pent = c.take<int32_t>(static_cast<size_t>(n > 0 ? n : 1));
  w->probe_blocks = static_cast<uint32_t>((n + kThreads - 1) / kThreads);
  w->part = c.take<uint32_t>(2 * static_cast<size_t>(w->probe_blocks) + 4 * kAssignMaxBlocks);
  w->cap = static_cast<uint32_t>(cap);
  return c.off;
}

__device__ __forceinline__ int64_t ld_relaxed(const int64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t bucket_of(uint64_t h, uint64_t nb, bool pow2) {
  return pow2 ? (h & (nb - 1)) : (h % nb);
}

__global__ void __launch_bounds__(kThreads) mz_init(MZWork w) {
  const uint32_t stride = kThreads * gridDim.x;
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < w.cap; i += stride) {
    w.mkey[i] = -1;
    w.mfpos[i] = 0x7fffffff;
    w.bkey[i] = -1;
    w.bhead[i] = -1;
  }
}

// Sum of one small count per thread over the block (LDS), visible to thread 0.
__device__ __forceinline__ uint32_t block_sum(uint32_t x, uint32_t *sh) {
  if (threadIdx.x == 0) *sh = 0u;
  __syncthreads();
  if (x) atomicAdd(sh, x);
  __syncthreads();
  return *sh;
}

__global__ void mz_zero_stats(unsigned long long *stats) {
  if (threadIdx.x < 6) stats[threadIdx.x] = 0ull;
}

template <int P>
__global__ void __launch_bounds__(kThreads)
    mz_probe(const int64_t *__restrict__ ids, int64_t n, const int64_t *__restrict__ identity, int64_t *stamps,
             uint64_t nb, bool nb_pow2, int probes_rt, int64_t now, int insert, int64_t *__restrict__ rows,
             int8_t *__restrict__ hit, int64_t *__restrict__ evicted, MZWork w, unsigned long long *stats) {
  const int probes = P > 0 ? P : probes_rt;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const bool valid = i < n;
  const int64_t id = valid ? ids[i] : HLR_EMPTY_ID;
  const bool invalid = valid && id == HLR_EMPTY_ID;
  int64_t row = -1;
  uint64_t h = 0, b = 0;
  if (valid && !invalid) {
    h = mix64(static_cast<uint64_t>(id));
    b = bucket_of(h, nb, nb_pow2);
    const int64_t base = static_cast<int64_t>(b) * probes;
    if (P == 8) {
      const longlong2 *q = reinterpret_cast<const longlong2 *>(identity + base);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const longlong2 v = q[j];
        if (v.x == id) row = base + 2 * j;
        if (v.y == id) row = base + 2 * j + 1;
      }
    } else {
      for (int j = 0; j < probes; ++j)
        if (identity[base + j] == id) row = base + j;
    }
  }
  const bool is_hit = row >= 0;
  const bool is_miss = valid && !invalid && !is_hit;
  if (valid) {
    rows[i] = row;
    hit[i] = is_hit ? 1 : 0;
    if (evicted) evicted[i] = HLR_EMPTY_ID;
    if (insert) {
      if (is_hit) stamps[row] = now;
      w.pent[i] = -1;
    }
  }
  if (stats) {
    __shared__ uint32_t sh_hit, sh_inv;
    const uint32_t h_blk = block_sum(is_hit ? 1u : 0u, &sh_hit);
    const uint32_t i_blk = block_sum(invalid ? 1u : 0u, &sh_inv);
    if (threadIdx.x == 0) {
      if (insert) {
        w.part[2 * blockIdx.x] = h_blk;
        w.part[2 * blockIdx.x + 1] = i_blk;
      } else {
        if (h_blk) atomicAdd(&stats[0], (unsigned long long)h_blk);
        if (i_blk) atomicAdd(&stats[4], (unsigned long long)i_blk);
      }
    }
  }
  if (!(insert && is_miss)) return;
  // Register the missed ID in the transient miss table (keyed by ID).
  const uint32_t mmask = w.cap - 1;
  uint32_t s = static_cast<uint32_t>(h >> 32) & mmask;
  bool created = false;
  for (;;) {
    const int64_t k = ld_relaxed(&w.mkey[s]);
    if (k == id) break;
    if (k == -1) {
      const int64_t prev = atomic_cas_i64(&w.mkey[s], -1, id);
      if (prev == -1) {
        created = true;
        break;
      }
      if (prev == id) break;
    }
    s = (s + 1) & mmask;
  }
  atomicMin(&w.mfpos[s], static_cast<int32_t>(i));
  w.pent[i] = static_cast<int32_t>(s);
  if (!created) return;
  // Push the new entry onto its bucket's list (bucket table keyed by bucket index).
  uint32_t t = static_cast<uint32_t>(mix64(b ^ 0x5851f42d4c957f2dULL) >> 32) & mmask;
  const int64_t bk = static_cast<int64_t>(b);
  for (;;) {
    const int64_t k = ld_relaxed(&w.bkey[t]);
    if (k == bk) break;
    if (k == -1) {
      const int64_t prev = atomic_cas_i64(&w.bkey[t], -1, bk);
      if (prev == -1 || prev == bk) break;
    }
    t = (t + 1) & mmask;
  }
  w.mnext[s] = atomicExch(&w.bhead[t], static_cast<int32_t>(s));
}

// One lane per bucket-table entry: the serial insert rule of one bucket.
template <int P>
__global__ void __launch_bounds__(kThreads)
    mz_assign(int64_t *identity, int64_t *stamps, int probes_rt, int64_t now, MZWork w,
              unsigned long long *stats) {
  constexpr int PM = P > 0 ? P : kMaxProbes;
  const int probes = P > 0 ? P : probes_rt;
  uint32_t ins = 0, evs = 0, ovf = 0, bad = 0;
  for (uint32_t t = blockIdx.x * kThreads + threadIdx.x; t < w.cap; t += kThreads * gridDim.x) {
  const int64_t bk = w.bkey[t];
  if (bk >= 0) {
    const int64_t base = bk * probes;
    int64_t idv[PM], stv[PM];
    int rank[PM];
#pragma unroll
    for (int j = 0; j < PM; ++j) {
      if (j < probes) {
        idv[j] = identity[base + j];
        stv[j] = stamps[base + j];
      }
    }
    int nempty = 0, nfree = 0;
#pragma unroll
    for (int j = 0; j < PM; ++j) {
      if (j < probes) {
        if (idv[j] == HLR_EMPTY_ID) ++nempty;
        else if (stv[j] < now) ++nfree;
      }
    }
    const int avail = nempty + nfree;
    // Preference rank of every slot: empties by probe index, then unpinned by (stamp, index).
#pragma unroll
    for (int j = 0; j < PM; ++j) {
      if (j >= probes) continue;
      int r = PM + 1;
      if (idv[j] == HLR_EMPTY_ID) {
        r = 0;
#pragma unroll
        for (int k = 0; k < PM; ++k)
          if (k < j && idv[k] == HLR_EMPTY_ID) ++r;
      } else if (stv[j] < now) {
        r = nempty;
#pragma unroll
        for (int k = 0; k < PM; ++k) {
          if (k < probes && idv[k] != HLR_EMPTY_ID && stv[k] < now &&
              (stv[k] < stv[j] || (stv[k] == stv[j] && k < j)))
            ++r;
        }
      }
      rank[j] = r;
    }
    // Walk the bucket's pending IDs, keeping the `avail` smallest first positions (sorted).
    int32_t sf[PM], se[PM];
    int cnt = 0, L = 0;
    int32_t lastf = 0;  // largest kept first position (valid once cnt == avail)
    for (int32_t e = w.bhead[t]; e != -1; e = w.mnext[e]) {
      const int32_t f = w.mfpos[e];
      w.mslot[e] = -1;  // overflow unless selected below
      ++L;
      int pos;
      if (cnt < avail) pos = cnt++;
      else if (cnt > 0 && f < lastf) pos = cnt - 1;
      else continue;
#pragma unroll
      for (int k = 0; k < PM; ++k)
        if (k == pos) {
          sf[k] = f;
          se[k] = e;
        }
#pragma unroll
      for (int k = PM - 1; k > 0; --k) {
        if (k <= pos && sf[k] < sf[k - 1]) {
          const int32_t tf = sf[k], te = se[k];
          sf[k] = sf[k - 1];
          se[k] = se[k - 1];
          sf[k - 1] = tf;
          se[k - 1] = te;
        }
      }
#pragma unroll
      for (int k = 0; k < PM; ++k)
        if (k == cnt - 1) lastf = sf[k];
    }
#pragma unroll
    for (int k = 0; k < PM; ++k) {
      if (k >= cnt) continue;
      int j = -1;
#pragma unroll
      for (int q = 0; q < PM; ++q)
        if (q < probes && rank[q] == k) j = q;
      const int64_t slot = base + j;
      const int64_t old = idv[j];
      const int64_t id = w.mkey[se[k]];
      const int64_t prev = atomic_cas_i64(&identity[slot], old, id);
      if (prev != old) ++bad;
      stamps[slot] = now;
      w.mslot[se[k]] = slot;
      w.mevict[se[k]] = old;
      ++ins;
      if (old != HLR_EMPTY_ID) ++evs;
    }
    ovf += L - cnt;
    w.bkey[t] = -1;  // the bucket-table entry is spent: leave it free for the next batch
    w.bhead[t] = -1;
  }
  }
  if (stats) {
    __shared__ uint32_t sh[4];
    const uint32_t a = block_sum(ins, &sh[0]);
    const uint32_t b = block_sum(evs, &sh[1]);
    const uint32_t c = block_sum(ovf, &sh[2]);
    const uint32_t d = block_sum(bad, &sh[3]);
    if (threadIdx.x == 0) {
      uint32_t *p = w.part + 2 * w.probe_blocks + 4 * blockIdx.x;
      p[0] = a;
      p[1] = b;
      p[2] = c;
      p[3] = d;
    }
  }
}

// The miss-table entry of an ID is spent once its positions know their row:
// the ID's first occurrence frees it for the next batch (the other positions
// of the ID read only mslot and mevict, and compare mfpos with their own
// position, which a cleared mfpos never equals).  With mz_assign freeing its
// bucket-table entries, a batch leaves both tables as mz_init makes them.
__device__ __forceinline__ void clear_miss_entry(const MZWork &w, int32_t e) {
  w.mkey[e] = -1;
  w.mfpos[e] = 0x7fffffff;
}

// Final stats from the per-block partial counts of mz_probe and mz_assign (no
// global atomics): the work of one extra block.
__device__ __forceinline__ void fold_stats(const MZWork &w, unsigned long long *stats, uint32_t assign_blocks) {
  if (!stats) return;
  __shared__ unsigned long long acc[6];
  if (threadIdx.x < 6) acc[threadIdx.x] = 0ull;
  __syncthreads();
  unsigned long long loc[6] = {0, 0, 0, 0, 0, 0};
  for (uint32_t b = threadIdx.x; b < w.probe_blocks; b += kThreads) {
    loc[0] += w.part[2 * b];
    loc[4] += w.part[2 * b + 1];
  }
  for (uint32_t b = threadIdx.x; b < assign_blocks; b += kThreads) {
    const uint32_t *p = w.part + 2 * w.probe_blocks + 4 * b;
    loc[1] += p[0];
    loc[2] += p[1];
    loc[3] += p[2];
    loc[5] += p[3];
  }
  for (int k = 0; k < 6; ++k)
    if (loc[k]) atomicAdd(&acc[k], loc[k]);
  __syncthreads();
  if (threadIdx.x < 6) stats[threadIdx.x] = acc[threadIdx.x];
}

__global__ void __launch_bounds__(kThreads)
    mz_resolve(int64_t n, float *values, int64_t dim, MZWork w, int64_t *__restrict__ rows,
               int64_t *__restrict__ evicted, unsigned long long *stats, uint32_t assign_blocks) {
  if (blockIdx.x == gridDim.x - 1) {  // the extra last block: stats; it has no positions
    fold_stats(w, stats, assign_blocks);
    return;
  }
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int32_t e = i < n ? w.pent[i] : -1;
  int64_t slot = -1;
  bool zero_fill = false;
  if (e >= 0) {
    slot = w.mslot[e];
    rows[i] = slot;
    const bool first = w.mfpos[e] == static_cast<int32_t>(i);
    if (first && slot >= 0) {
      if (evicted) evicted[i] = w.mevict[e];
      zero_fill = values != nullptr;
    }
    if (first) clear_miss_entry(w, e);
  }
  // The whole wave zero-fills each new row: 16-byte stores, lanes along the row.
  uint64_t m = ballot(zero_fill);
  const int64_t v4 = dim >> 2;
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  while (m) {
    const int l = __builtin_ctzll(m);
    m &= m - 1;
    const int64_t s = readlane_i64(slot, l);
    float4 *dst = reinterpret_cast<float4 *>(values) + s * v4;
    for (int64_t c = lane_id(); c < v4; c += kWave) dst[c] = z;
  }
}

// mz_resolve for the one-call Memory-Layer step (no zero-fill: the rows it
// inserts are read as zero by the row pass), fused with the grouping of the
// batch's positions by row (mlwork.hpp): a block resolves a tile of
// ml::kTile positions, then groups them.  A position's row is its hit row
// (from mz_probe) or the slot its missed ID took here; a row taken by a missed
// ID was inserted by this batch (fresh).
__global__ void __launch_bounds__(kThreads)
    mz_resolve_group(int64_t n, int64_t num_rows, MZWork w, int64_t *__restrict__ rows,
                     int64_t *__restrict__ evicted, unsigned long long *stats, uint32_t assign_blocks, ml::Work g) {
  if (blockIdx.x == gridDim.x - 1) {  // the extra last block: stats; it has no positions
    fold_stats(w, stats, assign_blocks);
    return;
  }
  __shared__ ml::Shared sh;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * ml::kTile;
  int32_t ent[ml::kItems];
  int64_t r[ml::kItems];
#pragma unroll
  for (int k = 0; k < ml::kItems; ++k) {  // every load first
    const int64_t i = base + k * kThreads + threadIdx.x;
    ent[k] = i < n ? w.pent[i] : -1;
    r[k] = i < n ? rows[i] : -1;
  }
  int32_t key[ml::kItems], pos[ml::kItems];
  bool fresh[ml::kItems];
#pragma unroll
  for (int k = 0; k < ml::kItems; ++k) {
    const int64_t i = base + k * kThreads + threadIdx.x;
    fresh[k] = false;
    if (ent[k] >= 0) {
      const int32_t e = ent[k];
      const int64_t slot = w.mslot[e];
      rows[i] = slot;
      const bool first = w.mfpos[e] == static_cast<int32_t>(i);
      if (slot >= 0 && evicted && first) evicted[i] = w.mevict[e];
      if (first) clear_miss_entry(w, e);
      r[k] = slot;
      fresh[k] = slot >= 0;
    }
    key[k] = (r[k] >= 0 && r[k] < num_rows) ? static_cast<int32_t>(r[k]) : -1;
    pos[k] = i < n ? static_cast<int32_t>(i) : -1;
  }
  ml::group_tile(sh, g, blockIdx.x, key, fresh, pos);
}

// Zero-fill of the rows a batch inserted (positions with hit 0 and a row),
// for callers that run the lookup without `values` on another stream and
// clear the new rows on the stream that reads and writes them.  One wave per
// 64 positions; the whole wave clears each selected row with 16-byte stores.
__global__ void __launch_bounds__(kThreads)
    mz_zero_inserted(float4 *values, int64_t num_rows, int64_t v4, const int64_t *__restrict__ rows,
                     const int8_t *__restrict__ hit, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  int64_t r = -1;
  if (i < n && hit[i] == 0) {
    r = rows[i];
    if (r >= num_rows) r = -1;
  }
  uint64_t m = ballot(r >= 0);
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  while (m) {
    const int l = __builtin_ctzll(m);
    m &= m - 1;
    float4 *dst = values + readlane_i64(r, l) * v4;
    for (int64_t c = lane_id(); c < v4; c += kWave) dst[c] = z;
  }
}

template <int P>
void mz_launch(int64_t *identity, int64_t *stamps, float *values, int64_t capacity, int probes, int64_t dim,
               const int64_t *ids, int64_t n, int64_t now, int insert, int64_t *rows, int8_t *hit,
               int64_t *evicted, unsigned long long *stats, MZWork &w, const ml::Work *group, hipStream_t s) {
  const uint64_t nb = static_cast<uint64_t>(capacity / probes);
  const bool pow2 = (nb & (nb - 1)) == 0;
  const int gpos = grid_for(n, kThreads);
  if (insert && !group) {  // the step (group) keeps its tables clear from batch to batch instead
    int gi = grid_for(w.cap, kThreads);
    if (gi > 4096) gi = 4096;
    mz_init<<<gi, kThreads, 0, s>>>(w);
  } else if (!insert && stats) {
    mz_zero_stats<<<1, 64, 0, s>>>(stats);
  }
  mz_probe<P><<<gpos, kThreads, 0, s>>>(ids, n, identity, stamps, nb, pow2, probes, now, insert, rows, hit, evicted,
                                         w, stats);
  if (!insert) return;
  int ga = grid_for(w.cap, kThreads);
  if (ga > kAssignMaxBlocks) ga = kAssignMaxBlocks;
  mz_assign<P><<<ga, kThreads, 0, s>>>(identity, stamps, probes, now, w, stats);
  if (group)
    mz_resolve_group<<<grid_for(n, ml::kTile) + 1, kThreads, 0, s>>>(n, capacity, w, rows, evicted, stats,
                                                                     static_cast<uint32_t>(ga), *group);
  else
    mz_resolve<<<gpos + 1, kThreads, 0, s>>>(n, values, dim, w, rows, evicted, stats, static_cast<uint32_t>(ga));
}

}  // namespace

extern "C" size_t mpzch_lookup_or_insert_workspace_size(int64_t n, int32_t insert) {
  if (!insert || n < 0) return 0;
  MZWork w;
  return mz_layout(n, &w, nullptr);
}

namespace {

// layout_n: the batch size the workspace's tables are laid out for (n, or for
// the step, whose tables stay clear from batch to batch, the largest batch
// the workspace was prepared for: the layout must not move between batches).
hlr_status mpzch_run(int64_t *identity, int64_t *stamps, float *values, int64_t capacity, int32_t probes,
                     int64_t dim, const int64_t *ids, int64_t n, int64_t now, int32_t insert, int64_t *out_rows,
                     int8_t *out_hit, int64_t *out_evicted, int64_t *out_stats, void *ws, size_t ws_bytes,
                     int64_t layout_n, const ml::Work *group, hipStream_t stream) {
  if (n < 0 || n > kMaxN || capacity <= 0 || probes < 1 || probes > kMaxProbes || capacity % probes != 0)
    return HLR_INVALID_ARG;
  if (insert != 0 && insert != 1) return HLR_INVALID_ARG;
  if (!identity || (insert && !stamps)) return HLR_INVALID_ARG;
  if (n > 0 && (!ids || !out_rows || !out_hit)) return HLR_INVALID_ARG;
  if (values && (dim <= 0 || dim % 4 != 0)) return HLR_UNSUPPORTED_DIM;
  if (!aligned(identity, 8) || (stamps && !aligned(stamps, 8)) || (ids && !aligned(ids, 8)) ||
      (out_rows && !aligned(out_rows, 8)) || (out_evicted && !aligned(out_evicted, 8)) ||
      (out_stats && !aligned(out_stats, 8)) || (values && !aligned(values, 16)))
    return HLR_MISALIGNED;
  // the aligned-bucket fast path reads a bucket as 16-byte pairs
  if (probes == 8 && !aligned(identity, 16)) return HLR_MISALIGNED;
  MZWork w{};
  if (insert) {
    if (layout_n < n) return HLR_INVALID_ARG;
    const size_t need = mz_layout(layout_n, &w, nullptr);
    if (!ws || ws_bytes < need) return HLR_WORKSPACE_TOO_SMALL;
    if (!aligned(ws, 256)) return HLR_MISALIGNED;
    mz_layout(layout_n, &w, ws);
    w.probe_blocks = static_cast<uint32_t>((n + kThreads - 1) / kThreads);  // this batch's probe blocks
  }
  unsigned long long *stats = reinterpret_cast<unsigned long long *>(out_stats);
  if (n == 0) {
    if (out_stats) mz_zero_stats<<<1, 64, 0, stream>>>(stats);
    return launch_status();
  }
  if (probes == 8)
    mz_launch<8>(identity, stamps, values, capacity, probes, dim, ids, n, now, insert, out_rows, out_hit, out_evicted,
                 stats, w, group, stream);
  else
    mz_launch<0>(identity, stamps, values, capacity, probes, dim, ids, n, now, insert, out_rows, out_hit,
                 out_evicted, stats, w, group, stream);
  return launch_status();
}

}  // namespace

extern "C" hlr_status mpzch_lookup_or_insert(int64_t *identity, int64_t *stamps, float *values, int64_t capacity,
                                             int32_t probes, int64_t dim, const int64_t *ids, int64_t n,
                                             int64_t now, int32_t insert, int64_t *out_rows, int8_t *out_hit,
                                             int64_t *out_evicted, int64_t *out_stats, void *ws, size_t ws_bytes,
                                             hipStream_t stream) {
  return mpzch_run(identity, stamps, values, capacity, probes, dim, ids, n, now, insert, out_rows, out_hit,
                   out_evicted, out_stats, ws, ws_bytes, n, nullptr, stream);
}

// ---------------------------------------------------------------------------
// The same call without a caller workspace, for callers that cannot allocate
// device memory (code under graph capture, serving loops, harnesses that
// forbid allocation): the scratch is this file-scope device array, one per
// GPU for the life of the process.  Host code must not pass `scratch` itself
// to a kernel (in host code it names a host-side stand-in): its device address
// comes from hipGetSymbolAddress, once per device, with that device current.
namespace {

constexpr int64_t kStaticMaxN = 262144;         // largest batch of the allocation-free call
constexpr size_t kStaticBytes = size_t(24) << 20;  // >= mpzch_lookup_or_insert_workspace_size(kStaticMaxN, 1)
constexpr int kStaticMaxDevices = 64;

static __device__ __align__(256) char scratch[kStaticBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kStaticMaxDevices];

// This device's address of `scratch` (nullptr on a HIP error).
void *scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kStaticMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int64_t mpzch_lookup_or_insert_static_max_n(void) { return kStaticMaxN; }

extern "C" hlr_status mpzch_lookup_or_insert_static(int64_t *identity, int64_t *stamps, float *values,
                                                    int64_t capacity, int32_t probes, int64_t dim,
                                                    const int64_t *ids, int64_t n, int64_t now, int32_t insert,
                                                    int64_t *out_rows, int8_t *out_hit, int64_t *out_evicted,
                                                    int64_t *out_stats, hipStream_t stream) {
  if (n < 0 || n > kStaticMaxN) return HLR_INVALID_ARG;  // beyond the array's batch size
  const size_t need = mpzch_lookup_or_insert_workspace_size(n, insert);
  if (need > kStaticBytes) return HLR_WORKSPACE_TOO_SMALL;
  void *ws = nullptr;
  if (need > 0) {
    ws = scratch_on_current_device();
    if (!ws) return HLR_HIP_ERROR;
  }
  // mz_init clears every table the batch uses first, so the last call's contents do not matter
  return mpzch_run(identity, stamps, values, capacity, probes, dim, ids, n, now, insert, out_rows, out_hit,
                   out_evicted, out_stats, ws, need > 0 ? kStaticBytes : 0, n, nullptr, stream);
}

extern "C" size_t memory_layer_step_workspace_size(int64_t n, int64_t capacity) {
  if (n < 0 || capacity < 0) return 0;
  ml::Work g;
  return ml::layout(n, capacity, &g, nullptr);
}

extern "C" hlr_status memory_layer_step_workspace_init(void *mz_ws, size_t mz_ws_bytes, void *wb_ws, size_t wb_ws_bytes,
                                                       int64_t n, int64_t capacity, hipStream_t stream) {
  if (n < 0 || n > kMaxN || capacity <= 0) return HLR_INVALID_ARG;
  if ((mz_ws && !aligned(mz_ws, 256)) || (wb_ws && !aligned(wb_ws, 256))) return HLR_MISALIGNED;
  if (mz_ws) {
    if (mz_ws_bytes < mpzch_lookup_or_insert_workspace_size(n, 1)) return HLR_WORKSPACE_TOO_SMALL;
    MZWork w{};
    mz_layout(n, &w, mz_ws);
    int gi = grid_for(w.cap, kThreads);
    if (gi > 4096) gi = 4096;
    mz_init<<<gi, kThreads, 0, stream>>>(w);
  }
  if (wb_ws) {
    if (wb_ws_bytes < memory_layer_step_workspace_size(n, capacity)) return HLR_WORKSPACE_TOO_SMALL;
    ml::Work g;
    ml::layout(n, capacity, &g, wb_ws);
    hlr_fill(reinterpret_cast<uint32_t *>(g.hrow), 4 * capacity, 0u, stream);
  }
  return launch_status();
}

hlr_status hlr::ml_plan(int64_t *identity, int64_t *stamps, int64_t capacity, int32_t probes, const int64_t *ids,
                        int64_t n, int64_t n_max, int64_t now, int64_t *out_rows, int8_t *out_hit,
                        int64_t *out_evicted, int64_t *out_stats, void *mz_ws, size_t mz_ws_bytes, void *ws,
                        hipStream_t stream) {
  ml::Work g;
  ml::layout(n_max, capacity, &g, ws);
  return mpzch_run(identity, stamps, nullptr, capacity, probes, 0, ids, n, now, 1, out_rows, out_hit, out_evicted,
                   out_stats, mz_ws, mz_ws_bytes, n_max, &g, stream);
}

extern "C" hlr_status mpzch_zero_inserted(float *values, int64_t capacity, int64_t dim, const int64_t *rows,
                                          const int8_t *hit, int64_t n, hipStream_t stream) {
  if (n < 0 || n > kMaxN || capacity <= 0) return HLR_INVALID_ARG;
  if (dim <= 0 || dim % 4 != 0) return HLR_UNSUPPORTED_DIM;
  if (n == 0) return HLR_OK;
  if (!values || !rows || !hit) return HLR_INVALID_ARG;
  if (!aligned(values, 16) || !aligned(rows, 8)) return HLR_MISALIGNED;
  mz_zero_inserted<<<grid_for(n, kThreads), kThreads, 0, stream>>>(reinterpret_cast<float4 *>(values), capacity,
                                                                   dim / 4, rows, hit, n);
  return launch_status();
}
