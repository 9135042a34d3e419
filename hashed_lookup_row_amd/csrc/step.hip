// One Memory-Layer training batch ("Memory Layer: Train the In-Model Cache
// for Recommendation Models", sec. 2: MPZCH ID -> row, gather, Writeback with
// lr = 1) enqueued by a single host call in the two-stream schedule: the
// ID-side half (lookup/insert, then the grouping of the batch's positions by
// row) on a lookup stream, the row traffic (one pass over the distinct rows
// that gathers them and applies the Writeback, mlstep.hip) on a compute
// stream, ordered by events.  The overlap is the dispatch/compute stream
// split of "MTGR: Industrial-Scale Generative Recommendation Framework in
// Meituan", sec. 3.5.  The batch gives the same results as the library's
// lookup, gather and Writeback calls made one after another on one stream.
// The two halves can also be enqueued by separate calls, so that a caller
// enqueues the ID-side half of batch t+1 before the row traffic of batch t
// (lookahead): the lookup kernels then find the GPU ready while the previous
// batch's rows move.
#include <hip/hip_runtime.h>

#include "hlr.h"
#include "hlr_common.hpp"
#include "step_parts.hpp"

namespace {

inline hlr_status hip_ok(hipError_t e) { return e == hipSuccess ? HLR_OK : HLR_HIP_ERROR; }


}  // namespace

extern "C" hlr_status memory_layer_step(int64_t *identity, int64_t *stamps, float *values, int64_t capacity,
                                        int32_t probes, int64_t dim, const int64_t *ids, int64_t n, int64_t n_max,
                                        int64_t now,
                                        const float *e, int64_t *out_rows, int8_t *out_hit, int64_t *out_evicted,
                                        int64_t *out_stats, float *out, void *mz_ws, size_t mz_ws_bytes,
                                        void *wb_ws, size_t wb_ws_bytes, hipStream_t lookup, hipStream_t compute,
                                        hipEvent_t slot_free, hipEvent_t looked_up, hipEvent_t planned,
                                        hipEvent_t gather_begin, hipEvent_t gather_end, hipEvent_t slot_done,
                                        int32_t halves) {
  // everything host-checkable first, so that an error enqueues nothing
  if (n < 0 || n_max < n || n_max > hlr::kMaxN || capacity <= 0 || capacity >= 0x7fffffff || probes < 1 ||
      probes > 32 || capacity % probes != 0)
    return HLR_INVALID_ARG;
  if (dim <= 0 || dim % 4 != 0 || dim > 1024) return HLR_UNSUPPORTED_DIM;
  if (halves < 1 || halves > 3) return HLR_INVALID_ARG;
  const bool lk = halves & 1, cp = halves & 2;
  if (!values || !out_rows || !out_hit) return HLR_INVALID_ARG;
  if (lk && (!identity || !stamps || (n > 0 && !ids))) return HLR_INVALID_ARG;
  if (cp && n > 0 && (!e || !out)) return HLR_INVALID_ARG;
  if (!hlr::aligned(values, 16) || (e && !hlr::aligned(e, 16)) || (out && !hlr::aligned(out, 16)) ||
      (identity && !hlr::aligned(identity, probes == 8 ? 16 : 8)) || (stamps && !hlr::aligned(stamps, 8)) ||
      (ids && !hlr::aligned(ids, 8)) || !hlr::aligned(out_rows, 8) || (out_evicted && !hlr::aligned(out_evicted, 8)) ||
      (out_stats && !hlr::aligned(out_stats, 8)))
    return HLR_MISALIGNED;
  if (mz_ws_bytes < mpzch_lookup_or_insert_workspace_size(n_max, 1) ||
      wb_ws_bytes < memory_layer_step_workspace_size(n_max, capacity))
    return HLR_WORKSPACE_TOO_SMALL;
  if ((n > 0 && (!mz_ws || !wb_ws)) || (mz_ws && !hlr::aligned(mz_ws, 256)) || (wb_ws && !hlr::aligned(wb_ws, 256)))
    return mz_ws && wb_ws ? HLR_MISALIGNED : HLR_WORKSPACE_TOO_SMALL;
  hlr_status st;
  if (lk) {  // lookup stream: MPZCH lookup/insert, then the grouping of positions by row
    if (slot_free && (st = hip_ok(hipStreamWaitEvent(lookup, slot_free, 0))) != HLR_OK) return st;
    if ((st = hlr::ml_plan(identity, stamps, capacity, probes, ids, n, n_max, now, out_rows, out_hit, out_evicted,
                           out_stats, mz_ws, mz_ws_bytes, wb_ws, lookup)) != HLR_OK)
      return st;
    if (looked_up && (st = hip_ok(hipEventRecord(looked_up, lookup))) != HLR_OK) return st;
    if (planned && (st = hip_ok(hipEventRecord(planned, lookup))) != HLR_OK) return st;
  }
  if (!cp) return HLR_OK;
  // compute stream: one pass over the batch's rows (gather + Writeback)
  if (planned && (st = hip_ok(hipStreamWaitEvent(compute, planned, 0))) != HLR_OK) return st;
  if (gather_begin && (st = hip_ok(hipEventRecord(gather_begin, compute))) != HLR_OK) return st;
  if ((st = hlr::ml_apply(values, capacity, dim, e, n, n_max, out, wb_ws, compute)) != HLR_OK) return st;
  if (gather_end && (st = hip_ok(hipEventRecord(gather_end, compute))) != HLR_OK) return st;
  if (slot_done && (st = hip_ok(hipEventRecord(slot_done, compute))) != HLR_OK) return st;
  return HLR_OK;
}
