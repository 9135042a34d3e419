/*
 * hlr.h — C ABI of libhlr.so, the MI355X (gfx950) hot path of an in-model
 * embedding cache for recommendation models.
 *
 * The operations follow these pages (cited by title and section):
 *  [ML]   "Memory Layer: Train the In-Model Cache for Recommendation Models",
 *         sec. 2 (method) and sec. 5 (limitations);
 *  [CS3]  "CS3: Efficient Online Capability Synergy for Two-Tower
 *         Recommendation", sec. 2 (method: CTS and CMS);
 *  [DLRM] "DLRMv4: MLPerf recommendation training goes sequential", feature
 *         expansion paragraph (hashed tables, 512-d fp32 rows, per-token
 *         unpooled lookups);
 *  [MTGR] "MTGR: Industrial-Scale Generative Recommendation Framework in
 *         Meituan", sec. 3.2 (dynamic hash table) and sec. 3.5 (dispatch and
 *         compute streams).
 *
 * Conventions shared by every entry point
 *  - Array arguments are DEVICE pointers on the current HIP device, owned by
 *    the caller.  The library allocates nothing and keeps no state between
 *    calls; every launch is enqueued on `stream` and no call synchronises.
 *  - Rows are int64 indices into a table of `num_rows` rows of `dim` values,
 *    row-major; -1 means "no row" (a miss or an overflow) and reads as the
 *    zero vector.  Rows outside [-1, num_rows) are a caller error: kernels skip
 *    them (treat them like -1) so memory stays safe; results for them are
 *    unspecified.
 *  - float tables, value and output arrays must be 16-byte aligned and
 *    `dim % 4 == 0` (rows are moved as 16-byte vectors); int64 arrays must be
 *    8-byte aligned.  n counts positions; 0 <= n < 2^31.
 *  - Scratch: entry points that need device scratch take (ws, ws_bytes);
 *    `*_workspace_size(...)` gives the byte count for a given problem.  ws
 *    must be 256-byte aligned and may be NULL only when that size is 0.  The
 *    workspace is scratch only: its contents on entry do not matter and calls
 *    that share one workspace must be ordered on one stream.
 *  - Every entry point returns an hlr_status.  Host-checkable faults return
 *    an error before anything is enqueued.  Device-side data faults are never
 *    thrown; mpzch_lookup_or_insert counts them in out_stats.
 *  - Floating point: no contraction into FMA; each fp32 operation named
 *    below rounds on its own (IEEE round-to-nearest-even, denormals kept).
 */
#ifndef HLR_H
#define HLR_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t hlr_status;
#define HLR_OK 0
#define HLR_INVALID_ARG 1        /* bad size, NULL where not allowed, bad mode */
#define HLR_UNSUPPORTED_DIM 2    /* dim % 4 != 0 (dim % 16 != 0 for int8 rows) or dim <= 0 */
#define HLR_MISALIGNED 3         /* pointer not aligned as required */
#define HLR_WORKSPACE_TOO_SMALL 4
#define HLR_HIP_ERROR 5          /* a launch failed (hipGetLastError) */

#define HLR_EMPTY_ID (-1)        /* identity value of an empty slot; also an invalid input ID */

/* Human-readable name of a status code (static string, never NULL). */
const char *hlr_status_string(hlr_status status);

/* Library ABI version (major*100 + minor). */
int32_t hlr_version(void);

/* ------------------------------------------------------------------------
 * MPZCH lookup / insert with LRU eviction   [ML] sec. 2
 *
 * The identity tensor maps raw int64 item IDs to table rows with no
 * collisions (one ID per row).  Capacity is bounded and rows are recycled
 * least-recently-used; metadata (the LRU stamp) shares the row index.
 *
 *  identity[capacity]  int64, -1 = empty slot.  In/out (insert mode).
 *  stamps[capacity]    int64 LRU stamps (last batch that touched the slot;
 *                      -1 for never).  In/out (insert mode).
 *  values[capacity*dim] fp32 rows, nullable: when given, rows that receive a
 *                      new ID are zero-filled (a new ID never reads an
 *                      evicted ID's vector; a miss reads zero, [ML] sec. 2).
 *  capacity % probes == 0; probes in [1, 32].  Bucket of x =
 *  SplitMix64-finaliser(x) mod (capacity/probes); x probes the `probes`
 *  consecutive slots of its bucket in order.
 *  ids[n]              int64 item IDs; -1 is invalid (row -1, counted).
 *  now                 int64 step counter, strictly greater than every stamp
 *                      already stored (insert mode); not checked on device.
 *  insert              1 = training batch (lookup, pin, insert, evict);
 *                      0 = serving lookup (reads only, changes nothing).
 *  Semantics (two phases): every ID resident at batch start is a hit and its
 *  slot's stamp becomes `now` (pinned).  Then the distinct missed IDs, in
 *  order of first occurrence in `ids`, are inserted: each takes the first
 *  empty slot of its bucket, else the unpinned slot (stamp < now) with the
 *  smallest stamp (lowest probe index on ties), else it overflows (row -1).
 *  out_rows[n]         slot of each position's ID, or -1.
 *  out_hit[n]          int8, 1 iff the ID was resident at batch start.
 *  out_evicted[n]      nullable; the ID displaced by an insert, written at that
 *                      ID's first occurrence; -1 elsewhere.
 *  out_stats[6]        nullable, device int64: {hit positions, inserts,
 *                      evictions, overflows (distinct IDs), invalid positions,
 *                      internal consistency failures (always 0)}.
 *  Workspace: mpzch_lookup_or_insert_workspace_size(n, insert) bytes
 *  (0 in lookup-only mode).
 * --------------------------------------------------------------------- */
size_t mpzch_lookup_or_insert_workspace_size(int64_t n, int32_t insert);
hlr_status mpzch_lookup_or_insert(int64_t *identity, int64_t *stamps, float *values, int64_t capacity,
                                  int32_t probes, int64_t dim, const int64_t *ids, int64_t n, int64_t now,
                                  int32_t insert, int64_t *out_rows, int8_t *out_hit, int64_t *out_evicted,
                                  int64_t *out_stats, void *ws, size_t ws_bytes, hipStream_t stream);

/* mpzch_lookup_or_insert without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, semantics and
 * errors as mpzch_lookup_or_insert; the scratch is a device array inside the
 * library (24 MiB per GPU it runs on, held until the process ends), so the call
 * allocates nothing.  n must be at most mpzch_lookup_or_insert_static_max_n()
 * (262,144): larger batches return HLR_INVALID_ARG before anything is
 * enqueued.  Every call on one GPU shares that GPU's array: calls that may
 * overlap on one GPU (different streams, or different host threads) race and
 * must be ordered by the caller.  A HIP error while locating the array returns
 * HLR_HIP_ERROR. */
int64_t mpzch_lookup_or_insert_static_max_n(void);
hlr_status mpzch_lookup_or_insert_static(int64_t *identity, int64_t *stamps, float *values, int64_t capacity,
                                         int32_t probes, int64_t dim, const int64_t *ids, int64_t n, int64_t now,
                                         int32_t insert, int64_t *out_rows, int8_t *out_hit, int64_t *out_evicted,
                                         int64_t *out_stats, hipStream_t stream);

/* Zero-fill of the rows a batch inserted, split from the lookup: a lookup
 * run with values == NULL (for instance on its own stream, so it can overlap
 * the previous batch's row traffic) leaves the new rows as they were; this
 * call then writes zeros to rows[i] for every position with hit[i] == 0 and
 * rows[i] >= 0, which is exactly the set of slots the lookup inserted into.
 * Enqueue it after every earlier write to those rows and before any read
 * of them for this batch.  values[capacity*dim] fp32 (16-byte aligned,
 * dim % 4 == 0); rows[n], hit[n] from mpzch_lookup_or_insert. */
hlr_status mpzch_zero_inserted(float *values, int64_t capacity, int64_t dim, const int64_t *rows,
                               const int8_t *hit, int64_t n, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Row gather   [ML] sec. 2 (the model reads the cached row M[i])
 *  out[i][:] = table[rows[i]][:] for rows[i] >= 0, zeros for rows[i] == -1.
 *  table[num_rows*dim], out[n*dim] fp32, 16-byte aligned, dim % 4 == 0.
 * --------------------------------------------------------------------- */
hlr_status gather_rows(const float *table, int64_t num_rows, int64_t dim, const int64_t *rows, int64_t n,
                       float *out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * In-batch deduplication   [ML] sec. 2 (duplicate IDs of a batch are
 * deduplicated so each row gets one exact write)
 *  keys[n]             int64 keys (IDs or rows).
 *  out_unique[n]       distinct keys in ascending signed order (first u used).
 *  out_last_pos[n]     position of the LAST occurrence of each distinct key.
 *  out_inverse[n]      nullable; index into out_unique of each position's key.
 *  out_num_unique      device int64 scalar: u.
 *  Workspace: dedup_ids_workspace_size(n) bytes.
 * --------------------------------------------------------------------- */
size_t dedup_ids_workspace_size(int64_t n);
hlr_status dedup_ids(const int64_t *keys, int64_t n, int64_t *out_unique, int64_t *out_last_pos,
                     int64_t *out_inverse, int64_t *out_num_unique, void *ws, size_t ws_bytes,
                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * Row updates from a batch   [ML] sec. 2 (Writeback); [DLRM] (per-row SGD)
 *  table[num_rows*dim] fp32 in place; rows[n]; src[n*dim] fp32.
 *  mode HLR_WB_LAST_WINS: src holds the item-tower vectors e_i.  Every
 *    distinct row r >= 0 takes one exact write from its LAST occurrence p:
 *    g = fl(M[r] - e_p), M[r] = fl(M[r] - g)   (exact SGD at learning rate 1,
 *    so M[r] becomes e_p up to these two roundings).  lr must be 1.
 *  mode HLR_WB_SGD_SUM: src holds gradients g_i.  The gradients of each row
 *    are summed as one fp32 running sum per element in ascending batch
 *    order, starting from the first (s = g_1, s = fl(s + g_k)), then
 *    M[r] = fl(M[r] - fl(lr*s)).
 *  mode HLR_WB_L2_ALIGN: src holds targets e_i; the row is learned by SGD on
 *    ||M[r] - e_i||^2, the alternative to Writeback in [ML] sec. 2 and 3:
 *    each occurrence's gradient is fl(2*fl(M[r] - e_i)) with M[r] the row
 *    before the batch, summed and applied exactly as in HLR_WB_SGD_SUM.
 *  Rows not in the batch are untouched.
 *  Workspace: writeback_rows_workspace_size(num_rows, dim, n, mode) bytes.
 * --------------------------------------------------------------------- */
#define HLR_WB_LAST_WINS 0
#define HLR_WB_SGD_SUM 1
#define HLR_WB_L2_ALIGN 2
size_t writeback_rows_workspace_size(int64_t num_rows, int64_t dim, int64_t n, int32_t mode);
hlr_status writeback_rows(float *table, int64_t num_rows, int64_t dim, const int64_t *rows, const float *src,
                          int64_t n, int32_t mode, float lr, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * writeback_rows in two halves, so the half that needs only `rows` can run on
 * another stream ahead of the values (the lookup/dispatch stream beside the
 * compute stream of "MTGR: Industrial-Scale Generative Recommendation
 * Framework in Meituan", sec. 3.5).  writeback_plan followed by
 * writeback_apply with the same workspace, n, num_rows and mode equals
 * writeback_rows bit for bit.
 *  writeback_plan: groups the positions of rows[n] by row (LAST_WINS: the
 *    last position of every distinct row; SGD_SUM and L2_ALIGN: positions in
 *    batch order per row) into ws.  `rows` is not read after the plan.
 *  writeback_apply: applies src[n*dim] to table through the plan in ws.
 *  ws: writeback_rows_workspace_size(num_rows, dim, n, mode) bytes, sized for
 *    the apply's dim.  It holds the plan between the two calls: each plan
 *    serves exactly one apply, and nothing else may use ws in between (order
 *    the two calls with an event when they run on different streams).
 * --------------------------------------------------------------------- */
hlr_status writeback_plan(int64_t num_rows, const int64_t *rows, int64_t n, int32_t mode, void *ws,
                          size_t ws_bytes, hipStream_t stream);
hlr_status writeback_apply(float *table, int64_t num_rows, int64_t dim, const float *src, int64_t n,
                           int32_t mode, float lr, void *ws, size_t ws_bytes, hipStream_t stream);

/* Several independent SGD_SUM or L2_ALIGN updates applied by one launch (the
 * hashed tables of [DLRM] take one update per table per step).  Each update
 * is writeback_apply(table, num_rows, dim, src, n, mode, lr, ws, ws_bytes)
 * with its plan in ws (writeback_plan with the same mode); the results equal
 * those calls made one after another.  The duplicate runs of all updates
 * start together and their other rows stream beside them (two kernel
 * launches for the whole batch).
 *  count in [0, 8]; updates[count] is a host array; mode HLR_WB_SGD_SUM or
 *  HLR_WB_L2_ALIGN for all.  Every update must have the same dim; tables and
 *  workspaces must not overlap between updates (HLR_INVALID_ARG).  Updates
 *  with n == 0 or num_rows == 0 are skipped.  Other errors as
 *  writeback_apply, checked for every update before anything is enqueued. */
typedef struct {
  float *table;
  int64_t num_rows;
  int64_t dim;
  const float *src;
  int64_t n;
  float lr;
  void *ws;
  size_t ws_bytes;
} hlr_wb_apply;
hlr_status writeback_apply_batch(int32_t count, const hlr_wb_apply *updates, int32_t mode, hipStream_t stream);

/* The distinct rows a LAST_WINS plan covers (the rows the batch writes), for
 * publishing them after the apply (Raw Embedding Streaming, [ML] sec. 2).
 *  ws: a workspace holding a writeback_plan(..., HLR_WB_LAST_WINS) for the
 *  same num_rows and n, not yet reused.  out_rows[n] receives the distinct
 *  rows in an unspecified order (the first *out_count entries);
 *  out_count: device int64 scalar. */
hlr_status writeback_plan_rows(int64_t num_rows, int64_t n, const void *ws, size_t ws_bytes, int64_t *out_rows,
                               int64_t *out_count, hipStream_t stream);

/* ------------------------------------------------------------------------
 * EMA row updates   [CS3] sec. 2 (CTS: c <- a*c + (1-a)*v on positive
 * interactions; CMS: s <- b*s + (1-b)*h on every interaction)
 *  For every position i in batch order with 0 <= rows[i] < num_rows and
 *  mask[i] != 0 (mask NULL = every position; other rows take no part):
 *  T[r] = fl(fl(a*T[r]) + fl(b*vals[i])),
 *  element-wise; duplicates of a row are applied in batch order, so the
 *  result equals the sequential loop bit for bit.  a and b are passed
 *  separately (b is not recomputed as 1-a).
 *  table[num_rows*dim] fp32 in place; vals[n*dim] fp32; mask[n] uint8.
 *  Workspace: ema_update_rows_workspace_size(num_rows, dim, n) bytes.
 * --------------------------------------------------------------------- */
size_t ema_update_rows_workspace_size(int64_t num_rows, int64_t dim, int64_t n);
hlr_status ema_update_rows(float *table, int64_t num_rows, int64_t dim, const int64_t *rows, const float *vals,
                           const uint8_t *mask, int64_t n, float a, float b, void *ws, size_t ws_bytes,
                           hipStream_t stream);

/* ema_update_rows in two halves, as writeback_plan / writeback_apply:
 * ema_update_plan groups the positions (rows[n], mask[n] or NULL) by row into
 * ws; ema_update_apply applies vals[n*dim] with (a, b) through that plan.
 * Together they equal ema_update_rows bit for bit.  ws:
 * ema_update_rows_workspace_size(num_rows, dim, n) bytes, sized for the
 * apply's dim; each plan serves exactly one apply. */
hlr_status ema_update_plan(int64_t num_rows, const int64_t *rows, const uint8_t *mask, int64_t n, void *ws,
                           size_t ws_bytes, hipStream_t stream);
hlr_status ema_update_apply(float *table, int64_t num_rows, int64_t dim, const float *vals, int64_t n, float a,
                            float b, void *ws, size_t ws_bytes, hipStream_t stream);

/* Several independent EMA updates applied by one launch ([CS3] sec. 2 keeps
 * four caches per batch: CTS and CMS for users and for items).  Each update
 * is ema_update_apply(table, num_rows, dim, vals, n, a, b, ws, ws_bytes) with
 * its plan in ws; the results equal those calls made one after another.  The
 * heavy rows of all updates start together and their light rows stream
 * beside them (two kernel launches for the whole batch).
 *  count in [0, 4]; updates[count] is a host array.  Every update must have
 *  the same dim (HLR_INVALID_ARG otherwise); tables and workspaces must not
 *  overlap between updates (HLR_INVALID_ARG).  Updates with n == 0 or
 *  num_rows == 0 are skipped.  Other errors as ema_update_apply, checked
 *  for every update before anything is enqueued. */
typedef struct {
  float *table;
  int64_t num_rows;
  int64_t dim;
  const float *vals;
  int64_t n;
  float a;
  float b;
  void *ws;
  size_t ws_bytes;
} hlr_ema_apply;
hlr_status ema_update_apply_batch(int32_t count, const hlr_ema_apply *updates, hipStream_t stream);

/* Two EMA updates keyed by different rows, planned by one sort and applied as
 * one ([CS3] sec. 2: each batch updates a user-keyed and an item-keyed cache
 * with the same rule, CTS on the positives and CMS on every pair).
 *  Update 0: table0[num_rows0*dim] with rows0[n], values vals0[n*dim];
 *  update 1: table1[num_rows1*dim] with rows1[n], values vals1[n*dim];
 *  both with the same mask[n] (NULL = every position) and the same (a, b).
 *  The result equals ema_update_rows on each table, bit for bit (the two
 *  tables are independent).  ema_update_plan_pair groups the 2n pairs by
 *  (table, row) into ws; ema_update_apply_pairs applies up to four such pairs
 *  in one launch, under the rules of ema_update_apply_batch (one dim; no
 *  table or workspace shared between or within pairs).  The plan of a subset
 *  of a pair plan's positions comes from ema_update_plan_subset given
 *  num_rows0 + num_rows1 as num_rows and 2n as n (its mask is still mask[n]).
 *  ws: ema_update_pair_workspace_size(num_rows0, num_rows1, dim, n) bytes
 *  (0 for sizes out of range: num_rows0 + num_rows1 must stay below 2^31 - 1
 *  and 2n within the batch limit).  Errors: HLR_INVALID_ARG for sizes out of
 *  range, NULL pointers or overlaps, HLR_MISALIGNED, HLR_UNSUPPORTED_DIM,
 *  HLR_WORKSPACE_TOO_SMALL; nothing is enqueued then. */
size_t ema_update_pair_workspace_size(int64_t num_rows0, int64_t num_rows1, int64_t dim, int64_t n);
hlr_status ema_update_plan_pair(int64_t num_rows0, const int64_t *rows0, int64_t num_rows1, const int64_t *rows1,
                                const uint8_t *mask, int64_t n, void *ws, size_t ws_bytes, hipStream_t stream);
typedef struct {
  float *table0;
  int64_t num_rows0;
  const float *vals0;
  float *table1;
  int64_t num_rows1;
  const float *vals1;
  int64_t dim;
  int64_t n;
  float a;
  float b;
  void *ws;
  size_t ws_bytes;
} hlr_ema_apply_pair;
hlr_status ema_update_apply_pairs(int32_t count, const hlr_ema_apply_pair *pairs, hipStream_t stream);

/* The plan of a subset of another plan's positions, without sorting again
 * ([CS3] sec. 2: CTS updates on the positive interactions, a subset of the
 * pairs CMS updates on, keyed by the same user and item IDs).
 *  src_ws: a workspace holding an ema_update_plan (or ema_update_plan_subset)
 *    result for rows[n] and num_rows; only read, so it can still be applied.
 *  mask[n] uint8: the positions to keep.  ws receives the plan that
 *    ema_update_plan(num_rows, rows, src_mask AND mask, n) would make, and
 *    applying it gives the same result bit for bit.
 *  Both workspaces are ema_update_rows_workspace_size(num_rows, dim, n)
 *  bytes, distinct and not overlapping (HLR_INVALID_ARG otherwise); mask must
 *  not be NULL (HLR_INVALID_ARG).  The src plan must be complete when this
 *  runs (same stream, or ordered by an event). */
hlr_status ema_update_plan_subset(int64_t num_rows, const uint8_t *mask, int64_t n, const void *src_ws,
                                  size_t src_ws_bytes, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Serving score: int8 row dequantisation fused with a dot product
 *   [ML] sec. 1 (O(1K) candidates scored per request) and sec. 5 (serving
 *   reads int8 rows); miss -> zero vector [ML] sec. 2.
 *  qtable[num_rows*dim] int8 (16-byte aligned, dim % 16 == 0);
 *  scale[num_rows], bias[num_rows] fp32: x_d = q_d*scale + bias.
 *  rows[num_requests*cands_per_request] (from a lookup-only MPZCH call);
 *  user_vecs[num_requests*dim] fp32.
 *  out_scores[r*cands + c] = sum_d x_d * user[r][d], evaluated in fp64 as
 *  scale*sum_d q_d*u_d + bias*sum_d u_d (the same sum up to fp64 rounding
 *  order) and rounded once to fp32; a row of -1, or any row outside
 *  [0, num_rows), scores 0.0f and is not read.  num_rows = 0: all 0.0f.
 * --------------------------------------------------------------------- */
hlr_status gather_dequant_score(const int8_t *qtable, const float *scale, const float *bias, int64_t num_rows,
                                int64_t dim, const int64_t *rows, int64_t num_requests,
                                int64_t cands_per_request, const float *user_vecs, float *out_scores,
                                hipStream_t stream);

/* ------------------------------------------------------------------------
 * Serving lookup and score in one launch   [ML] sec. 2 (MPZCH identity
 *   tensor) and sec. 1, 5 (candidates scored against int8 rows)
 *  The lookup-only MPZCH rule of mpzch_lookup_or_insert (insert 0: the slot
 *  of bucket(id) holding the ID, else -1; an ID of -1 never has a row;
 *  nothing changes) followed by gather_dequant_score, in one launch:
 *  identity[capacity] (16-byte aligned when probes == 8), probes,
 *  ids[num_requests*cands_per_request]; qtable/scale/bias hold one row per
 *  identity slot (num_rows = capacity); other arguments and out_scores as
 *  gather_dequant_score.  out_rows (int64) and out_hit (int8), nullable,
 *  receive the lookup's rows and hit mask.
 * --------------------------------------------------------------------- */
hlr_status mpzch_score(const int64_t *identity, int64_t capacity, int32_t probes, const int64_t *ids,
                       const int8_t *qtable, const float *scale, const float *bias, int64_t dim,
                       int64_t num_requests, int64_t cands_per_request, const float *user_vecs, float *out_scores,
                       int64_t *out_rows, int8_t *out_hit, hipStream_t stream);

/* ------------------------------------------------------------------------
 * int8 row quantisation for publishing   [ML] sec. 2 (Raw Embedding
 * Streaming quantises the rows a step touched before pushing them to
 * serving) and sec. 5 (serving reads int8 rows)
 *  For each i < m, m = min(n, *count) (count NULL: m = n), row r = rows[i]:
 *    scale = fl(fl(max - min) / 255), or 1 when max == min;
 *    bias  = fl(min + fl(128 * scale));
 *    q_d   = clamp(rne(fl(fl(x_d - bias) / scale)), -128, 127)
 *  over the row's fp32 values x (min, max over the row; fp32 throughout).
 *  scatter 0: written at index i (out_q[m*dim], out_scale[m], out_bias[m]);
 *    a row of -1 gives q = 0, scale = 0, bias = 0.
 *  scatter 1: written at index r (arrays of num_rows entries, for example
 *    the serving table of gather_dequant_score); rows of -1 are skipped.
 *  table fp32 (16-byte aligned, dim % 4 == 0, dim <= 1024); out_q 4-byte
 *  aligned.  q*scale + bias dequantises to within about scale/2.
 * --------------------------------------------------------------------- */
hlr_status quantize_rows_int8(const float *table, int64_t num_rows, int64_t dim, const int64_t *rows, int64_t n,
                              const int64_t *count, int32_t scatter, int8_t *out_q, float *out_scale,
                              float *out_bias, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Written-row set between publishes   [ML] sec. 2 (Raw Embedding Streaming
 * deduplicates the rows training wrote and pushes them at intervals)
 *  mark_rows: for i < min(n, *count) (count NULL: n) with 0 <= rows[i] <
 *    num_rows, the row is appended to list[] (and *list_count incremented)
 *    unless flags[row] is already set; then flags[row] is set.  Duplicates
 *    across calls are listed once; list order is unspecified.
 *    flags[num_rows] uint32 (zero before first use); list[num_rows] int64;
 *    list_count device int64 scalar (zero before first use).
 *  clear_marks: unflags the first *list_count rows of list and sets
 *    *list_count = 0, leaving flags all zero again.
 * --------------------------------------------------------------------- */
hlr_status mark_rows(const int64_t *rows, int64_t n, const int64_t *count, int64_t num_rows, uint32_t *flags,
                     int64_t *list, int64_t *list_count, hipStream_t stream);
hlr_status clear_marks(const int64_t *list, int64_t *list_count, int64_t num_rows, uint32_t *flags,
                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * Decoupled, growable key store   "MTGR: Industrial-Scale Generative
 * Recommendation Framework in Meituan", sec. 3.2 (a light key store maps a key
 * to a row of a separate value store, which holds the embedding with counters
 * and timestamps for eviction; growing copies the light key store only)
 *  keys[key_cap], krows[key_cap] int64: the key store, open addressing with
 *    linear probing from SplitMix64-finaliser(key) mod key_cap; key_cap a
 *    power of two; key -1 = empty slot.  Keep at least n empty slots before a
 *    batch (grow with dks_rehash); otherwise results are unspecified.
 *  Value store: chunks of 2^chunk_shift rows (4 <= chunk_shift <= 24), each
 *    one device allocation of dks_chunk_bytes(chunk_shift, dim) bytes (16-byte
 *    aligned) laid out as the rows' vectors fp32[2^chunk_shift][dim], then
 *    their stamps int64[2^chunk_shift] (last batch that touched the row; -1
 *    never), then their counts uint32[2^chunk_shift] (lookups that reached the
 *    row); chunks[num_chunks] is a device array of the chunks' addresses, and
 *    row r lives at row r mod 2^chunk_shift of chunks[r >> chunk_shift].  The
 *    store holds num_chunks << chunk_shift rows and grows by appending chunks
 *    (prepared with dks_chunk_init); no row ever moves.  dim % 4 == 0.
 *    next_row: device int64, rows in use (in/out).
 *  Semantics (insert 1): keys already stored are hits (row; the row's stamp =
 *    now); then the distinct missed keys, in order of first occurrence in ids,
 *    take rows next_row, next_row + 1, ... (vector zero-filled, stamped) while
 *    the store holds rows; later ones overflow (row -1, not stored).  Every
 *    position whose key has a row after the batch adds one to that row's
 *    count (a hit, or any occurrence of a key the batch inserted).  insert 0
 *    only looks up and changes nothing.  ids of -1 are invalid (row -1,
 *    counted).
 *  out_rows[n], out_hit[n] int8; out_stats[4] nullable, device int64:
 *    {hit positions, inserted keys, overflowed keys, invalid positions}.
 *  Workspace: dks_workspace_size(n) bytes (insert mode only).
 * dks_chunk_bytes: bytes of one chunk (0 for an invalid shift or dim).
 * dks_chunk_init: clears a chunk before it joins the store (vectors and
 *  counts 0, stamps -1); enqueued on stream.
 * dks_gather_rows: out[n][dim] fp32 = the vector of row rows[i], or zeros for
 *  rows[i] < 0 or beyond the rows the store holds.
 * dks_rehash: copies every stored key with its row into an empty key store of
 *  new_cap >= key_cap slots (filled with -1 by the call); the value store is
 *  not touched.
 * --------------------------------------------------------------------- */
size_t dks_workspace_size(int64_t n);
int64_t dks_chunk_bytes(int32_t chunk_shift, int64_t dim);
hlr_status dks_chunk_init(void *chunk, int32_t chunk_shift, int64_t dim, hipStream_t stream);
hlr_status dks_lookup_or_insert(int64_t *keys, int64_t *krows, int64_t key_cap, const uint64_t *chunks,
                                int32_t chunk_shift, int64_t num_chunks, int64_t dim, int64_t *next_row,
                                const int64_t *ids, int64_t n, int64_t now, int32_t insert, int64_t *out_rows,
                                int8_t *out_hit, int64_t *out_stats, void *ws, size_t ws_bytes, hipStream_t stream);
hlr_status dks_gather_rows(const uint64_t *chunks, int32_t chunk_shift, int64_t num_chunks, int64_t dim,
                           const int64_t *rows, int64_t n, float *out, hipStream_t stream);
hlr_status dks_rehash(const int64_t *keys, const int64_t *krows, int64_t key_cap, int64_t *new_keys,
                      int64_t *new_krows, int64_t new_cap, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Hashed-table row mapping   [DLRM] feature expansion (hashed tables)
 *  out_rows[i] = SplitMix64-finaliser(ids[i]) mod num_rows (collisions
 *  allowed; no identity tensor).  num_rows >= 1.
 * --------------------------------------------------------------------- */
hlr_status hashed_rows(const int64_t *ids, int64_t n, int64_t num_rows, int64_t *out_rows, hipStream_t stream);

/* ------------------------------------------------------------------------
 * One Memory-Layer training batch in one host call   [ML] sec. 2 (lookup,
 * gather, Writeback with lr = 1); two-stream overlap as the dispatch and
 * compute streams of [MTGR] sec. 3.5.
 *  Enqueues, in this order:
 *   lookup stream:  wait slot_free (if given);
 *                   MPZCH lookup/insert (as mpzch_lookup_or_insert with
 *                   values = NULL, insert = 1), then the grouping of the
 *                   batch's positions by row into wb_ws;
 *                   record looked_up (if given); record planned (if given).
 *   compute stream: wait planned (if given);
 *                   record gather_begin (if given);
 *                   one pass over the batch's distinct rows: each row is read
 *                   once, written to out at every position that holds it
 *                   (the gather), then takes its Writeback from its last
 *                   position;
 *                   record gather_end (if given); record slot_done (if given).
 *  The rows the lookup inserts are not zero-filled in memory first: a row the
 *  batch inserted is read as the zero vector (a new ID never reads an evicted
 *  ID's vector) and is then written by its Writeback.
 *  The results equal mpzch_lookup_or_insert, gather_rows and
 *  writeback_rows(LAST_WINS) made one after another on one stream:
 *  identity/stamps/values updated, out_rows/out_hit/out_evicted/out_stats as
 *  mpzch_lookup_or_insert, out[n*dim] the gathered rows (read before the
 *  Writeback), values[r] <- fl(M - fl(M - e[last position of r])).
 *  Arguments as the calls above; capacity = the table's row count, below
 *  2^31 - 1; dim <= 1024.  Events are the caller's (hipEventCreateWithFlags;
 *  timing needed only for the gather pair), each nullable.  A compute half
 *  without planned does not wait for its lookup half: give NULL only when the
 *  caller orders the two halves itself (the same stream for both, or a wait
 *  the caller enqueued on the compute stream for an event recorded after this
 *  batch's lookup half, e.g. once for a group of batches).  n_max >= n: the
 *  largest batch the
 *  workspaces serve (the same for every batch that uses them).  mz_ws: a
 *  workspace of mpzch_lookup_or_insert_workspace_size(n_max, 1) bytes; wb_ws:
 *  one of memory_layer_step_workspace_size(n_max, capacity) bytes (both
 *  256-byte aligned).  Unlike the other entry points' scratch, these two keep
 *  their tables clear from batch to batch (no clearing kernel per batch):
 *  prepare each with memory_layer_step_workspace_init(..., n_max, capacity,
 *  ...) before its first batch; a batch whose two halves both ran leaves them
 *  prepared.  out_rows, out_hit and wb_ws
 *  stay in use until slot_done.
 *  halves: 1 = the lookup-stream half only, 2 = the compute-stream half
 *  only, 3 = both.  A batch's lookup half must be enqueued before its compute
 *  half (the compute half waits on planned, if given, as recorded by the most
 *  recent lookup half); enqueueing the lookup half of batch t+1 before the compute
 *  half of batch t (lookahead) is allowed and gives the same results, since
 *  the compute stream keeps the row traffic in batch order, provided each
 *  batch in flight has its own out_rows, out_hit, wb_ws and events.
 *  Pointers a half does not use may be NULL there (the lookup half does not
 *  read e or out, the compute half does not read identity, stamps or ids);
 *  the buffers of a batch (out_rows, out_hit, wb_ws) and its events must be
 *  the same in both calls.
 *  Host-checkable errors return before anything is enqueued; a HIP error
 *  from a later call returns HLR_HIP_ERROR with the batch partly enqueued.
 * --------------------------------------------------------------------- */
size_t memory_layer_step_workspace_size(int64_t n, int64_t capacity);

/* Puts a pair of workspaces for memory_layer_step into the state every batch
 * expects on entry and leaves behind (its tables clear), laid out for batches
 * of up to n positions (memory_layer_step's n_max): mz_ws of
 * mpzch_lookup_or_insert_workspace_size(n, 1) bytes and wb_ws of
 * memory_layer_step_workspace_size(n, capacity) bytes, either nullable.  Call
 * it once for every workspace before its first batch, and again after a batch
 * whose halves were not both enqueued or that returned an error.  Enqueued on
 * stream. */
hlr_status memory_layer_step_workspace_init(void *mz_ws, size_t mz_ws_bytes, void *wb_ws, size_t wb_ws_bytes,
                                            int64_t n, int64_t capacity, hipStream_t stream);
/* The rows a memory_layer_step batch wrote, added to a written-row set for
 * RES publishing ([ML] sec. 2, Raw Embedding Streaming: the rows training
 * updated since the last push): every row the batch's compute half applied
 * a Writeback to sets flags[row] (flags[capacity] uint32) and, if the flag was
 * clear, is appended to list (int64) at *list_count (int64, advanced), as
 * mark_rows does; a row already in the set is not listed again.  Reads the
 * batch's row grouping from wb_ws (memory_layer_step_workspace_size(n_max,
 * capacity) bytes, 256-byte aligned), so enqueue it on the compute stream
 * after the batch's compute half and before a later batch's lookup half
 * reuses wb_ws (record the slot's done event after this call).  n: the
 * batch's positions.  Errors: HLR_INVALID_ARG (n out of [0, n_max], NULL
 * pointers), HLR_MISALIGNED, HLR_WORKSPACE_TOO_SMALL; nothing is enqueued
 * then. */
hlr_status memory_layer_step_mark_written(const void *wb_ws, size_t wb_ws_bytes, int64_t n, int64_t n_max,
                                          int64_t capacity, uint32_t *flags, int64_t *list, int64_t *list_count,
                                          hipStream_t stream);
hlr_status memory_layer_step(int64_t *identity, int64_t *stamps, float *values, int64_t capacity, int32_t probes,
                             int64_t dim, const int64_t *ids, int64_t n, int64_t n_max, int64_t now, const float *e,
                             int64_t *out_rows, int8_t *out_hit, int64_t *out_evicted, int64_t *out_stats,
                             float *out, void *mz_ws, size_t mz_ws_bytes, void *wb_ws, size_t wb_ws_bytes,
                             hipStream_t lookup, hipStream_t compute, hipEvent_t slot_free, hipEvent_t looked_up,
                             hipEvent_t planned, hipEvent_t gather_begin, hipEvent_t gather_end,
                             hipEvent_t slot_done, int32_t halves);

#ifdef __cplusplus
}
#endif

#endif /* HLR_H */
