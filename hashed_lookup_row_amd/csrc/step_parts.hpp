// Variants of two entry points for the one-call Memory-Layer step
// (memory_layer_step), shared between the library's translation units and
// not exported.  In that step the rows a batch's lookup inserts are not
// cleared by a kernel of their own: every position that refers to such a row
// missed (hit 0), since a row in use by the batch is never evicted, so the
// gather reads the zero vector for those positions and the Writeback apply
// takes the row as zero, which is what clearing it first would give.
#pragma once

#include <hip/hip_runtime.h>

#include "hlr.h"

namespace hlr {

// gather_rows, with positions whose hit[i] == 0 reading the zero vector.
__attribute__((visibility("hidden"))) hlr_status gather_rows_fresh(const float *table, int64_t num_rows,
                                                                   int64_t dim, const int64_t *rows,
                                                                   const int8_t *hit, int64_t n, float *out,
                                                                   hipStream_t stream);

// writeback_apply(LAST_WINS, lr = 1) through the plan in ws, with the row of a
// position whose hit == 0 taken as zero before the update.
__attribute__((visibility("hidden"))) hlr_status writeback_apply_last_fresh(float *table, int64_t num_rows,
                                                                            int64_t dim, const float *src,
                                                                            int64_t n, const int8_t *hit, void *ws,
                                                                            size_t ws_bytes, hipStream_t stream);

// The one-call step's ID-side half: the MPZCH lookup/insert (values = NULL)
// whose last kernel also groups the batch's positions by row into ws
// (memory_layer_step_workspace_size(n_max, capacity) bytes, 256-byte
// aligned).  Both workspaces are laid out for batches of up to n_max
// positions and must be as memory_layer_step_workspace_init(..., n_max, ...)
// leaves them; the batch's kernels leave them so again.
__attribute__((visibility("hidden"))) hlr_status ml_plan(int64_t *identity, int64_t *stamps, int64_t capacity,
                                                         int32_t probes, const int64_t *ids, int64_t n, int64_t n_max,
                                                         int64_t now, int64_t *out_rows, int8_t *out_hit,
                                                         int64_t *out_evicted, int64_t *out_stats, void *mz_ws,
                                                         size_t mz_ws_bytes, void *ws, hipStream_t stream);

// Its row half: the gather of every position into out and the Writeback
// (last occurrence wins, lr = 1) of every distinct row, one pass over the rows
// through the grouping in ws.
__attribute__((visibility("hidden"))) hlr_status ml_apply(float *values, int64_t num_rows, int64_t dim,
                                                          const float *e, int64_t n, int64_t n_max, float *out,
                                                          void *ws, hipStream_t stream);

}  // namespace hlr
