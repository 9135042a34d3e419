// The grouping of a Memory-Layer batch's positions by row, shared by the
// lookup's last kernel (which builds it: mpzch.hip) and the one-pass row
// traffic that reads it (mlstep.hip).  "Memory Layer: Train the In-Model Cache
// for Recommendation Models", sec. 2: every position reads its row M[i], and
// each distinct row of the batch takes one Writeback from its last
// occurrence.
//
// A tile of kTile consecutive positions is grouped by row in LDS: a group is
// (tile, row) with its positions listed contiguously in gpos and one
// descriptor in gdesc.  Across tiles a row's groups meet in one 16-byte entry
// per row, indexed by the row itself (position count, last position + 1,
// positions done: one cache line per row touched, not one per field), added
// to with global atomics that return nothing.  A group that
// holds all positions of its row ("whole") applies the Writeback on its own;
// the groups of a row spread over several tiles count their positions into
// the row's done counter, and the one that completes it applies the
// Writeback.  The row pass returns every row entry it used to zero, so the
// tables start each batch at zero (memory_layer_step_workspace_init clears
// them once, before the first batch).
#pragma once

#include "hlr_common.hpp"
#include "radix.hpp"

namespace {

namespace ml {

constexpr int kThreads = 256;
constexpr int kTile = 1024;               // positions per grouping block
constexpr int kItems = kTile / kThreads;  // positions per thread
constexpr int kLHash = 2 * kTile;         // LDS hash entries
constexpr int kLPer = kLHash / kThreads;  // LDS entries per thread after grouping
constexpr int32_t kLEmpty = INT32_MIN;    // free LDS entry (keys are rows or -1)

// descriptor word 3: flags, and the group's position count in the low 28 bits
constexpr uint32_t kFresh = 1u << 31;   // the row was inserted by this batch: read as zero
constexpr uint32_t kNoRow = 1u << 30;   // positions without a row: zero vector, no Writeback
constexpr uint32_t kCountMask = (1u << 28) - 1;

struct Work {
  uint4 *hrow;       // [rows] x: positions of the row in the batch,      } zero between batches
                     //        y: last position of the row + 1 (0: none), }
                     //        z: positions whose read of the row is done }
  uint32_t *ntile;   // [tiles] groups of each tile
  uint4 *gdesc;      // [tiles * kTile] group j of tile t at t * kTile + j: row, -, first index in gpos,
                     //                 count | flags
  int32_t *gpos;     // [n] positions, tile by tile, group by group
  int64_t tiles;
};

inline size_t layout(int64_t n, int64_t rows, Work *w, void *base) {
  hlr::Carver c(base);
  const size_t nr = static_cast<size_t>(rows > 0 ? rows : 1);
  w->hrow = c.take<uint4>(nr);
  w->tiles = (n + kTile - 1) / kTile;
  const size_t nt = static_cast<size_t>(w->tiles > 0 ? w->tiles : 1);
  w->ntile = c.take<uint32_t>(nt);
  w->gdesc = c.take<uint4>(nt * kTile);
  w->gpos = c.take<int32_t>(static_cast<size_t>(n > 0 ? n : 1));
  return c.off;
}

__device__ __forceinline__ uint32_t lhash(int32_t key) {
  return (static_cast<uint32_t>(key) * 2654435761u) >> (32 - 11);  // 11 bits: kLHash entries
}
static_assert(kLHash == 1 << 11, "lhash takes 11 bits");

// LDS of one grouping block.
struct Shared {
  int32_t key[kLHash];
  uint32_t cnt[kLHash];
  int32_t last[kLHash];
  uint32_t fresh[kLHash];
  uint32_t start[kLHash];
  uint32_t gid[kLHash];
  int32_t pos[kTile];
  uint32_t scan[kThreads + 1];
};

// Groups tile `tile` (positions from tile * kTile): key[k] (a row, or -1 for
// no row; ignored when pos[k] < 0) and fresh[k] of this thread's kItems
// positions pos[k].  Called by the whole block.
__device__ __forceinline__ void group_tile(Shared &sh, Work &w, int64_t tile, const int32_t (&key)[kItems],
                                           const bool (&fresh)[kItems], const int32_t (&pos)[kItems]) {
  for (int e = threadIdx.x; e < kLHash; e += kThreads) {
    sh.key[e] = kLEmpty;
    sh.cnt[e] = 0u;
    sh.last[e] = -1;
    sh.fresh[e] = 0u;
  }
  __syncthreads();
  int32_t ent[kItems];
  uint32_t rank[kItems];
#pragma unroll
  for (int k = 0; k < kItems; ++k) {
    ent[k] = -1;
    if (pos[k] < 0) continue;
    uint32_t e = lhash(key[k]);
    for (;;) {
      const int32_t prev = atomicCAS(&sh.key[e], kLEmpty, key[k]);
      if (prev == kLEmpty || prev == key[k]) break;
      e = (e + 1) & (kLHash - 1);
    }
    ent[k] = static_cast<int32_t>(e);
    rank[k] = atomicAdd(&sh.cnt[e], 1u);
    atomicMax(&sh.last[e], pos[k]);
    if (fresh[k]) sh.fresh[e] = 1u;
  }
  __syncthreads();
  // number the groups and place their position lists: one block scan of
  // (groups << 16 | positions) over each thread's kLPer entries
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < kLPer; ++j) {
    const int e = threadIdx.x * kLPer + j;
    if (sh.key[e] != kLEmpty) mine += (1u << 16) + sh.cnt[e];
  }
  uint32_t total;
  uint32_t pre = block_exclusive_scan(mine, sh.scan, &total);
#pragma unroll
  for (int j = 0; j < kLPer; ++j) {
    const int e = threadIdx.x * kLPer + j;
    if (sh.key[e] != kLEmpty) {
      sh.gid[e] = pre >> 16;
      sh.start[e] = pre & 0xffffu;
      pre += (1u << 16) + sh.cnt[e];
    }
  }
  if (threadIdx.x == 0) w.ntile[tile] = total >> 16;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kItems; ++k)
    if (ent[k] >= 0) sh.pos[sh.start[ent[k]] + rank[k]] = pos[k];
  __syncthreads();
  const int64_t base = tile * kTile;
  const uint32_t npos = total & 0xffffu;
  for (uint32_t k = threadIdx.x; k < npos; k += kThreads) w.gpos[base + k] = sh.pos[k];
  // descriptors; the row's count and last position go to the row's entries
  // (atomics without a return value: nothing waits for them)
#pragma unroll
  for (int j = 0; j < kLPer; ++j) {
    const int e = threadIdx.x * kLPer + j;
    const int32_t key = sh.key[e];
    if (key == kLEmpty) continue;
    const uint32_t cnt = sh.cnt[e];
    uint4 d = make_uint4(static_cast<uint32_t>(key), 0u, static_cast<uint32_t>(base) + sh.start[e], cnt);
    if (key < 0) {
      d.w |= kNoRow;
    } else {
      atomicAdd(&w.hrow[key].x, cnt);
      atomicMax(&w.hrow[key].y, static_cast<uint32_t>(sh.last[e]) + 1u);
      if (sh.fresh[e]) d.w |= kFresh;
    }
    w.gdesc[base + sh.gid[e]] = d;
  }
}

}  // namespace ml

}  // namespace
