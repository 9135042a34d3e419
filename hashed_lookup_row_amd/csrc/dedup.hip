// In-batch deduplication ("Memory Layer: Train the In-Model Cache for
// Recommendation Models", sec. 2: duplicate IDs of a batch are deduplicated so
// each row receives exactly one exact write).  The winner of a key is its last
// occurrence; distinct keys come out in ascending signed order.
//
// Plan: keys are mapped to unsigned order (sign bit flipped) and sorted with
// their positions as (key, position) pairs (msort.hpp: tile sort + merge
// path), so positions are ascending inside a key; the segment pass then
// writes, per distinct key, the key, its last position and, per position, the
// inverse index.
#include "msort.hpp"
#include "radix.hpp"

namespace {
using namespace hlr;

constexpr uint64_t kSign = 0x8000000000000000ull;

struct DedupEmit {
  int64_t *unique;
  int64_t *last_pos;
  int64_t *inverse;
  __device__ void operator()(int64_t, int32_t seg, bool head, bool tail, uint64_t k, uint32_t v) const {
    if (head) unique[seg] = static_cast<int64_t>(k ^ kSign);
    if (tail) last_pos[seg] = static_cast<int64_t>(v);
    if (inverse) inverse[v] = seg;
  }
};

// The sort's input: pair i is (keys[i] in unsigned order, i).
struct DedupLoad {
  const int64_t *keys;
  __device__ __forceinline__ void operator()(int64_t i, uint64_t *key, uint32_t *pos) const {
    *key = static_cast<uint64_t>(keys[i]) ^ kSign;
    *pos = static_cast<uint32_t>(i);
  }
};

}  // namespace

extern "C" size_t dedup_ids_workspace_size(int64_t n) {
  if (n < 0) return 0;
  SegWork<uint64_t> w;
  return segwork_layout<uint64_t>(n, &w, nullptr);
}

extern "C" hlr_status dedup_ids(const int64_t *keys, int64_t n, int64_t *out_unique, int64_t *out_last_pos,
                                int64_t *out_inverse, int64_t *out_num_unique, void *ws, size_t ws_bytes,
                                hipStream_t stream) {
  if (n < 0 || n > kMaxN || !out_num_unique) return HLR_INVALID_ARG;
  if (n > 0 && (!keys || !out_unique || !out_last_pos)) return HLR_INVALID_ARG;
  if ((keys && !aligned(keys, 8)) || (out_unique && !aligned(out_unique, 8)) ||
      (out_last_pos && !aligned(out_last_pos, 8)) || (out_inverse && !aligned(out_inverse, 8)) ||
      !aligned(out_num_unique, 8))
    return HLR_MISALIGNED;
  if (n == 0) {
    hlr_fill<int64_t>(out_num_unique, 1, 0, stream);
    return launch_status();
  }
  SegWork<uint64_t> w;
  const size_t need = segwork_layout<uint64_t>(n, &w, nullptr);
  if (!ws || ws_bytes < need) return HLR_WORKSPACE_TOO_SMALL;
  if (!aligned(ws, 256)) return HLR_MISALIGNED;
  segwork_layout<uint64_t>(n, &w, ws);
  w.nseg = out_num_unique;
  const int cur = merge_sort_pairs<uint64_t>(DedupLoad{keys}, w.k, w.v, n, nullptr, stream);
  segment_sorted<uint64_t>(w, cur, 0ull, false, nullptr, DedupEmit{out_unique, out_last_pos, out_inverse}, stream);
  return launch_status();
}
