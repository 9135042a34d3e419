// One Memory-Layer training batch ("Memory Layer: Train the In-Model Cache
// for Recommendation Models", sec. 2: MPZCH ID -> row, gather, Writeback with
// lr = 1) enqueued by a single host call in the two-stream schedule: the
// ID-side half (lookup/insert, the Writeback plan) on a lookup stream, the row
// traffic (gather, Writeback apply) on a compute stream, ordered by events.  The overlap is the dispatch/compute stream split
// of "MTGR: Industrial-Scale Generative Recommendation Framework in Meituan",
// sec. 3.5.  The calls are the library's own entry points (the gather and
// the apply in the variants that take the lookup's hit mask in place of a
// zero-fill of the inserted rows), so the batch gives the same results as
// those calls made one after another on one stream; one host call instead of
// seven keeps the host ahead of the GPU.  The two halves
// can also be enqueued by separate calls, so that a caller enqueues the
// ID-side half of batch t+1 before the row traffic of batch t (lookahead): the
// lookup kernels then find the GPU ready while the previous batch's rows move.
#include <hip/hip_runtime.h>

#include "hlr.h"
#include "hlr_common.hpp"
#include "step_parts.hpp"

namespace {

inline hlr_status hip_ok(hipError_t e) { return e == hipSuccess ? HLR_OK : HLR_HIP_ERROR; }

}  // namespace

extern "C" hlr_status memory_layer_step(int64_t *identity, int64_t *stamps, float *values, int64_t capacity,
                                        int32_t probes, int64_t dim, const int64_t *ids, int64_t n, int64_t now,
                                        const float *e, int64_t *out_rows, int8_t *out_hit, int64_t *out_evicted,
                                        int64_t *out_stats, float *out, void *mz_ws, size_t mz_ws_bytes,
                                        void *wb_ws, size_t wb_ws_bytes, hipStream_t lookup, hipStream_t compute,
                                        hipEvent_t slot_free, hipEvent_t looked_up, hipEvent_t planned,
                                        hipEvent_t gather_begin, hipEvent_t gather_end, hipEvent_t slot_done,
                                        int32_t halves) {
  // everything host-checkable first, so that an error enqueues nothing
  if (n < 0 || n > hlr::kMaxN || capacity <= 0 || probes < 1 || probes > 32 || capacity % probes != 0)
    return HLR_INVALID_ARG;
  if (dim <= 0 || dim % 4 != 0) return HLR_UNSUPPORTED_DIM;
  if (halves < 1 || halves > 3) return HLR_INVALID_ARG;
  const bool lk = halves & 1, cp = halves & 2;
  if (!values || !out_rows || !out_hit || !looked_up || !planned) return HLR_INVALID_ARG;
  if (lk && (!identity || !stamps || (n > 0 && !ids))) return HLR_INVALID_ARG;
  if (cp && n > 0 && (!e || !out)) return HLR_INVALID_ARG;
  if (!hlr::aligned(values, 16) || (e && !hlr::aligned(e, 16)) || (out && !hlr::aligned(out, 16)) ||
      (identity && !hlr::aligned(identity, 8)) || (stamps && !hlr::aligned(stamps, 8)) ||
      (ids && !hlr::aligned(ids, 8)) || !hlr::aligned(out_rows, 8))
    return HLR_MISALIGNED;
  if (mz_ws_bytes < mpzch_lookup_or_insert_workspace_size(n, 1) ||
      wb_ws_bytes < writeback_rows_workspace_size(capacity, dim, n, HLR_WB_LAST_WINS))
    return HLR_WORKSPACE_TOO_SMALL;
  hlr_status st;
  if (lk) {  // lookup stream
    if (slot_free && (st = hip_ok(hipStreamWaitEvent(lookup, slot_free, 0))) != HLR_OK) return st;
    if ((st = mpzch_lookup_or_insert(identity, stamps, nullptr, capacity, probes, dim, ids, n, now, 1, out_rows,
                                     out_hit, out_evicted, out_stats, mz_ws, mz_ws_bytes, lookup)) != HLR_OK)
      return st;
    if ((st = hip_ok(hipEventRecord(looked_up, lookup))) != HLR_OK) return st;
    if ((st = writeback_plan(capacity, out_rows, n, HLR_WB_LAST_WINS, wb_ws, wb_ws_bytes, lookup)) != HLR_OK)
      return st;
    if ((st = hip_ok(hipEventRecord(planned, lookup))) != HLR_OK) return st;
  }
  if (!cp) return HLR_OK;
  // compute stream
  // The rows the lookup inserted are not cleared by a kernel of their own: only positions that missed
  // refer to them, so the gather reads zeros there and the apply takes them as zero (step_parts.hpp).
  // A compute half enqueued on its own (halves == 2) follows a lookup half enqueued earlier, so its plan is
  // normally long finished: one wait on `planned` (recorded after `looked_up` on the lookup stream) covers
  // both.  With both halves in one call the gather starts as soon as the lookup is done.
  const bool one_wait = halves == 2;
  if ((st = hip_ok(hipStreamWaitEvent(compute, one_wait ? planned : looked_up, 0))) != HLR_OK) return st;
  if (gather_begin && (st = hip_ok(hipEventRecord(gather_begin, compute))) != HLR_OK) return st;
  if ((st = hlr::gather_rows_fresh(values, capacity, dim, out_rows, out_hit, n, out, compute)) != HLR_OK) return st;
  if (gather_end && (st = hip_ok(hipEventRecord(gather_end, compute))) != HLR_OK) return st;
  if (!one_wait && (st = hip_ok(hipStreamWaitEvent(compute, planned, 0))) != HLR_OK) return st;
  if ((st = hlr::writeback_apply_last_fresh(values, capacity, dim, e, n, out_hit, wb_ws, wb_ws_bytes, compute)) !=
      HLR_OK)
    return st;
  if (slot_done && (st = hip_ok(hipEventRecord(slot_done, compute))) != HLR_OK) return st;
  return HLR_OK;
}
