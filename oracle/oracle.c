/*
 * CPU oracle for the in-model embedding cache — TEST INFRASTRUCTURE ONLY.
 *
 * Plain, single-threaded, deliberately slow C.  Only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load this library; the
 * product path (libhlr.so) never does and shares no code with it.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC
 * (no FMA contraction: every float operation below rounds on its own, in the
 * order written).
 *
 * Sources (cited by page title and section; no line numbers):
 *  [ML]   "Memory Layer: Train the In-Model Cache for Recommendation Models",
 *         sec. 2 (method): MPZCH identity tensor maps raw IDs to rows with no
 *         collisions, 512-d rows, metadata shares the row index, bounded
 *         capacity with LRU eviction; Writeback gradient g = M[i] - e_i applied
 *         by exact SGD at learning rate 1 so M[i] becomes e_i; duplicate IDs of
 *         a batch are deduplicated so each row receives one exact write; a
 *         cache miss zeroes the cached branch.  Sec. 5 (limitations): serving
 *         reads int8-quantised rows.
 *  [CS3]  "CS3: Efficient Online Capability Synergy for Two-Tower
 *         Recommendation", sec. 2 (method): CTS keeps c <- a*c + (1-a)*v,
 *         updated only on positive interactions; CMS keeps s <- b*s + (1-b)*h
 *         for every interaction.
 *  [DLRM] "DLRMv4: MLPerf recommendation training goes sequential", feature
 *         expansion paragraph: native sparse tables plus cross-product hashed
 *         tables, 512-d fp32 rows, per-token (unpooled) lookups.
 *  [SM64] SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 *         generators", OOPSLA 2014): 64-bit finaliser with the variant-13
 *         shift/multiply constants.
 *
 * Readings of points the pages leave open (each is listed in the design doc):
 *  - hash: SplitMix64 finaliser; bucket(x) = mix(x) mod (capacity/probes);
 *  - probes of x are the aligned bucket slots bucket(x)*P + j, j = 0..P-1;
 *  - identity == -1 is an empty slot, an input ID of -1 is invalid;
 *  - a batch is applied in two phases: every ID resident at batch start is a
 *    hit and its slot is pinned (stamp = now); then the distinct missed IDs are
 *    inserted in order of first occurrence, each taking the first empty slot of
 *    its bucket, else the unpinned slot (stamp < now) with the smallest stamp
 *    (lowest probe index on ties), else it overflows (row -1, zero vector);
 *  - an inserted row is zero-filled, evicted IDs are reported at the first
 *    occurrence of the ID that replaced them;
 *  - dedup keeps the last occurrence, unique keys ascending;
 *  - Writeback arithmetic is fp32: M' = fl(M - fl(M - e));
 *  - duplicate gradients of a row are summed as one fp32 running sum in
 *    ascending batch position, starting from the first gradient, then
 *    M' = fl(M - fl(lr * s));
 *  - EMA arithmetic is fp32 per step: T' = fl(fl(a*T) + fl(b*v)), positions in
 *    batch order;
 *  - dequant-score is evaluated in fp64: x_d = q_d*scale + bias,
 *    score = sum_d x_d*u_d, rounded once to fp32; a miss scores exactly 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL 1
#define ORC_ENOMEM 2
#define ORC_ESTAMP 3

#define ORC_EMPTY (-1)

/* [SM64] finaliser. */
uint64_t orc_mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

/* Bucket of an ID: the ID's two's-complement bits hashed, reduced modulo the bucket count. */
int64_t orc_bucket(int64_t id, int64_t num_buckets) {
    return (int64_t)(orc_mix64((uint64_t)id) % (uint64_t)num_buckets);
}

/* ------------------------------------------------------------ sort helpers */
typedef struct { int64_t key; int64_t pos; } orc_pair;

static int cmp_pair(const void *a, const void *b) {
    const orc_pair *x = (const orc_pair *)a, *y = (const orc_pair *)b;
    if (x->key != y->key) return x->key < y->key ? -1 : 1;
    if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;
    return 0;
}

static int cmp_pos_first(const void *a, const void *b) {
    const orc_pair *x = (const orc_pair *)a, *y = (const orc_pair *)b;
    if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;
    return 0;
}

/* ----------------------------------------------------------- MPZCH step [ML] */
/*
 * One batch against the MPZCH table.
 * identity[C], stamps[C]: table state, updated in place (insert mode only).
 * values[C*dim]: may be NULL; inserted rows are zero-filled when given.
 * Outputs per position: rows (slot or -1), hit (1 = resident at batch start),
 * evicted (the ID an insert displaced, at that insert's first occurrence; -1
 * elsewhere).  stats[5] = {hit positions, inserts, evictions, overflows,
 * invalid positions}.
 */
int orc_mpzch_step(int64_t *identity, int64_t *stamps, float *values, int64_t capacity, int32_t probes,
                   int64_t dim, const int64_t *ids, int64_t n, int64_t now, int32_t insert,
                   int64_t *rows, int8_t *hit, int64_t *evicted, int64_t *stats) {
    if (capacity <= 0 || probes <= 0 || capacity % probes != 0 || n < 0 || dim <= 0) return ORC_EINVAL;
    const int64_t nb = capacity / probes;
    int64_t st[5] = {0, 0, 0, 0, 0};
    if (insert) {
        for (int64_t s = 0; s < capacity; ++s)
            if (stamps[s] >= now) return ORC_ESTAMP;
    }
    /* Phase 1: IDs resident at batch start are hits and pin their slot. */
    for (int64_t i = 0; i < n; ++i) {
        rows[i] = -1;
        hit[i] = 0;
        evicted[i] = ORC_EMPTY;
        if (ids[i] == ORC_EMPTY) { st[4]++; continue; }
        const int64_t base = orc_bucket(ids[i], nb) * probes;
        for (int32_t j = 0; j < probes; ++j) {
            if (identity[base + j] == ids[i]) {
                rows[i] = base + j;
                hit[i] = 1;
                st[0]++;
                if (insert) stamps[base + j] = now;
                break;
            }
        }
    }
    if (insert) {
        /* Phase 2: distinct missed IDs in order of first occurrence. */
        int64_t m = 0;
        for (int64_t i = 0; i < n; ++i)
            if (!hit[i] && ids[i] != ORC_EMPTY) m++;
        orc_pair *miss = (orc_pair *)malloc((size_t)(m ? m : 1) * sizeof(orc_pair));
        orc_pair *first = (orc_pair *)malloc((size_t)(m ? m : 1) * sizeof(orc_pair));
        if (!miss || !first) { free(miss); free(first); return ORC_ENOMEM; }
        m = 0;
        for (int64_t i = 0; i < n; ++i)
            if (!hit[i] && ids[i] != ORC_EMPTY) { miss[m].key = ids[i]; miss[m].pos = i; m++; }
        qsort(miss, (size_t)m, sizeof(orc_pair), cmp_pair);
        int64_t f = 0;
        for (int64_t k = 0; k < m; ++k)
            if (k == 0 || miss[k].key != miss[k - 1].key) first[f++] = miss[k];
        qsort(first, (size_t)f, sizeof(orc_pair), cmp_pos_first);
        for (int64_t k = 0; k < f; ++k) {
            const int64_t id = first[k].key;
            const int64_t base = orc_bucket(id, nb) * probes;
            int32_t best = -1;
            for (int32_t j = 0; j < probes; ++j)
                if (identity[base + j] == ORC_EMPTY) { best = j; break; }
            if (best < 0) {
                for (int32_t j = 0; j < probes; ++j)
                    if (stamps[base + j] < now && (best < 0 || stamps[base + j] < stamps[base + best])) best = j;
            }
            if (best < 0) { st[3]++; continue; } /* overflow: every slot pinned by this batch */
            const int64_t s = base + best;
            const int64_t old = identity[s];
            if (old != ORC_EMPTY) st[2]++;
            st[1]++;
            identity[s] = id;
            stamps[s] = now;
            if (values) memset(values + s * dim, 0, (size_t)dim * sizeof(float));
            evicted[first[k].pos] = old;
        }
        /* Every missed position takes the slot its ID now occupies (or -1 on overflow). */
        for (int64_t k = 0; k < m; ++k) {
            const int64_t id = miss[k].key, i = miss[k].pos;
            const int64_t base = orc_bucket(id, nb) * probes;
            for (int32_t j = 0; j < probes; ++j)
                if (identity[base + j] == id) { rows[i] = base + j; break; }
        }
        free(miss);
        free(first);
    }
    if (stats) memcpy(stats, st, sizeof(st));
    return ORC_OK;
}

/* ------------------------------------------------------------- gather [ML] */
/* out[i] = table[rows[i]]; a row of -1 (miss or overflow) reads as the zero vector. */
int orc_gather(const float *table, int64_t num_rows, int64_t dim, const int64_t *rows, int64_t n, float *out) {
    for (int64_t i = 0; i < n; ++i) {
        if (rows[i] < -1 || rows[i] >= num_rows) return ORC_EINVAL;
        for (int64_t d = 0; d < dim; ++d) out[i * dim + d] = rows[i] < 0 ? 0.0f : table[rows[i] * dim + d];
    }
    return ORC_OK;
}

/* --------------------------------------------------------------- dedup [ML] */
/*
 * Distinct keys in ascending order, the last position of each, and for every
 * position the index of its key.  Returns the number of distinct keys (or -1).
 */
int64_t orc_dedup(const int64_t *keys, int64_t n, int64_t *unique, int64_t *last_pos, int64_t *inverse) {
    orc_pair *p = (orc_pair *)malloc((size_t)(n ? n : 1) * sizeof(orc_pair));
    if (!p) return -1;
    for (int64_t i = 0; i < n; ++i) { p[i].key = keys[i]; p[i].pos = i; }
    qsort(p, (size_t)n, sizeof(orc_pair), cmp_pair);
    int64_t u = -1;
    for (int64_t k = 0; k < n; ++k) {
        if (k == 0 || p[k].key != p[k - 1].key) { ++u; unique[u] = p[k].key; }
        last_pos[u] = p[k].pos; /* positions ascend within a key: the final one is the last occurrence */
        if (inverse) inverse[p[k].pos] = u;
    }
    free(p);
    return u + 1;
}

/* Positions grouped by row (rows >= 0 only), each group in ascending position. */
static orc_pair *group_rows(const int64_t *rows, const uint8_t *mask, int64_t n, int64_t num_rows, int64_t *m_out,
                            int *err) {
    int64_t m = 0;
    *err = ORC_OK;
    for (int64_t i = 0; i < n; ++i) {
        if (rows[i] < -1 || rows[i] >= num_rows) { *err = ORC_EINVAL; return NULL; }
        if (rows[i] >= 0 && (!mask || mask[i])) m++;
    }
    orc_pair *p = (orc_pair *)malloc((size_t)(m ? m : 1) * sizeof(orc_pair));
    if (!p) { *err = ORC_ENOMEM; return NULL; }
    m = 0;
    for (int64_t i = 0; i < n; ++i)
        if (rows[i] >= 0 && (!mask || mask[i])) { p[m].key = rows[i]; p[m].pos = i; m++; }
    qsort(p, (size_t)m, sizeof(orc_pair), cmp_pair);
    *m_out = m;
    return p;
}

/* ------------------------------------------------------ Writeback [ML] sec.2 */
/*
 * Each distinct row r >= 0 of the batch takes one exact write from its last
 * occurrence p: g = fl(M[r] - e[p]); M[r] = fl(M[r] - g)  (learning rate 1).
 */
int orc_writeback_last(float *table, int64_t num_rows, int64_t dim, const int64_t *rows, const float *e, int64_t n) {
    int64_t m = 0;
    int err;
    orc_pair *p = group_rows(rows, NULL, n, num_rows, &m, &err);
    if (!p) return err;
    for (int64_t k = 0; k < m; ++k) {
        if (k + 1 < m && p[k + 1].key == p[k].key) continue; /* not the last occurrence */
        float *w = table + p[k].key * dim;
        const float *src = e + p[k].pos * dim;
        for (int64_t d = 0; d < dim; ++d) {
            const float g = w[d] - src[d];
            w[d] = w[d] - g;
        }
    }
    free(p);
    return ORC_OK;
}

/* --------------------------------------------- SGD with summed duplicates */
/*
 * Duplicate gradients of a row are summed, then applied once ([DLRM] hashed
 * tables take a per-row SGD step; [ML] sec. 2 deduplicates a batch so a row is
 * written once).  For each element the sum is one fp32 running sum over the
 * row's positions in ascending batch order, starting from the first gradient
 * (s = g[p1], then s = fl(s + g[pk])); then M[r] = fl(M[r] - fl(lr*s)).
 */
int orc_sgd_sum(float *table, int64_t num_rows, int64_t dim, const int64_t *rows, const float *g, int64_t n,
                float lr) {
    int64_t m = 0;
    int err;
    orc_pair *p = group_rows(rows, NULL, n, num_rows, &m, &err);
    if (!p) return err;
    int64_t k0 = 0;
    while (k0 < m) {
        int64_t k1 = k0;
        while (k1 < m && p[k1].key == p[k0].key) k1++;
        float *w = table + p[k0].key * dim;
        for (int64_t d = 0; d < dim; ++d) {
            float s = g[p[k0].pos * dim + d];
            for (int64_t k = k0 + 1; k < k1; ++k) s = s + g[p[k].pos * dim + d];
            const float step = lr * s;
            w[d] = w[d] - step;
        }
        k0 = k1;
    }
    free(p);
    return ORC_OK;
}

/* ------------------------------ decoupled, growable key store [MTGR] sec. 3.2 */
/*
 * Key store and value store are separate ([MTGR] sec. 3.2): the key store maps
 * a raw key to a row of the value store; the value store holds the rows with
 * the metadata an eviction policy uses (counters and timestamps: here the last
 * batch that touched the row and the number of lookups that reached it);
 * growing the key store copies keys only.  Readings: the key store is an
 * open-addressing table of `key_cap` slots (keys[], krows[]; key -1 = empty),
 * linear probing from mix(key) mod key_cap; the value store hands out rows in
 * order (next_row, below max_rows = the rows the store holds during this
 * batch; the caller grows it between batches).  One batch, two phases as for
 * MPZCH: keys already stored are hits (row, stamp = now); then the distinct
 * missed keys, in order of first occurrence, take rows next_row, next_row + 1,
 * ... (zero-filled when values is given, stamp = now) until max_rows, after
 * which they overflow (row -1, nothing stored).  Every position whose key has
 * a row after the batch adds one to that row's count (counts nullable).
 * insert == 0 only looks up.  The table must keep at least one empty slot.
 * stats: {hit positions, inserted keys, overflowed keys, invalid positions}.
 */
static int64_t orc_dks_find(const int64_t *keys, int64_t key_cap, int64_t key, int64_t *slot) {
    int64_t s = (int64_t)(orc_mix64((uint64_t)key) % (uint64_t)key_cap);
    for (int64_t j = 0; j < key_cap; ++j) {
        if (keys[s] == key) { *slot = s; return 1; }
        if (keys[s] == ORC_EMPTY) { *slot = s; return 0; }
        s = (s + 1) % key_cap;
    }
    *slot = -1;
    return 0;
}

int orc_dks_step(int64_t *keys, int64_t *krows, int64_t key_cap, int64_t *stamps, uint32_t *counts, float *values,
                 int64_t dim, int64_t max_rows, int64_t *next_row, const int64_t *ids, int64_t n, int64_t now,
                 int32_t insert, int64_t *rows, int8_t *hit, int64_t *stats) {
    if (key_cap <= 0 || n < 0 || max_rows < 0 || *next_row < 0 || *next_row > max_rows) return ORC_EINVAL;
    int64_t st[4] = {0, 0, 0, 0};
    /* Phase 1: keys already stored. */
    for (int64_t i = 0; i < n; ++i) {
        rows[i] = -1;
        hit[i] = 0;
        if (ids[i] == ORC_EMPTY) { st[3]++; continue; }
        int64_t slot;
        if (orc_dks_find(keys, key_cap, ids[i], &slot)) {
            rows[i] = krows[slot];
            hit[i] = 1;
            st[0]++;
            if (insert) stamps[rows[i]] = now;
        }
    }
    if (insert) {
        /* Phase 2: distinct missed keys in order of first occurrence take the next rows. */
        for (int64_t i = 0; i < n; ++i) {
            if (ids[i] == ORC_EMPTY || hit[i]) continue;
            int64_t slot;
            if (orc_dks_find(keys, key_cap, ids[i], &slot)) {  /* inserted earlier in this batch */
                rows[i] = krows[slot];
                continue;
            }
            int64_t first = 1;
            for (int64_t k = 0; k < i && first; ++k)
                if (ids[k] == ids[i]) first = 0;
            if (!first) continue;  /* an earlier occurrence overflowed */
            if (*next_row >= max_rows || slot < 0) { st[2]++; continue; }
            const int64_t r = (*next_row)++;
            keys[slot] = ids[i];
            krows[slot] = r;
            stamps[r] = now;
            if (values) memset(values + r * dim, 0, (size_t)dim * sizeof(float));
            rows[i] = r;
            st[1]++;
        }
        if (counts)  /* one lookup per position that reached a row */
            for (int64_t i = 0; i < n; ++i)
                if (rows[i] >= 0) counts[rows[i]]++;
    }
    for (int k = 0; k < 4; ++k) stats[k] = st[k];
    return ORC_OK;
}

/* ------------------------------------------------ L2 alignment [ML] sec. 2 */
/*
 * The plain alternative to Writeback that [ML] sec. 2 and sec. 3 compare with
 * it: learn the cache row by SGD on the squared distance ||M[r] - sg(e_i)||^2.
 * Each occurrence i of row r contributes the gradient 2 (M[r] - e_i), taken at
 * the row's value before the batch: g_i = fl(2 * fl(M[r] - e_i)) (the doubling
 * is exact).  A row's gradients are summed as in orc_sgd_sum (one running sum
 * in ascending batch order, from the first) and applied once:
 * M[r] = fl(M[r] - fl(lr * s)).
 */
int orc_l2_align(float *table, int64_t num_rows, int64_t dim, const int64_t *rows, const float *e, int64_t n,
                 float lr) {
    int64_t m = 0;
    int err;
    orc_pair *p = group_rows(rows, NULL, n, num_rows, &m, &err);
    if (!p) return err;
    int64_t k0 = 0;
    while (k0 < m) {
        int64_t k1 = k0;
        while (k1 < m && p[k1].key == p[k0].key) k1++;
        float *w = table + p[k0].key * dim;
        for (int64_t d = 0; d < dim; ++d) {
            const float before = w[d];
            float diff = before - e[p[k0].pos * dim + d];
            float s = 2.0f * diff;
            for (int64_t k = k0 + 1; k < k1; ++k) {
                diff = before - e[p[k].pos * dim + d];
                s = s + 2.0f * diff;
            }
            const float step = lr * s;
            w[d] = before - step;
        }
        k0 = k1;
    }
    free(p);
    return ORC_OK;
}

/* --------------------------------------------------------------- EMA [CS3] */
/*
 * In batch order, for every position i with rows[i] >= 0 and mask[i] != 0 (mask
 * NULL = all): T[r] = fl(fl(a*T[r]) + fl(b*v_i)), element-wise.
 */
int orc_ema(float *table, int64_t num_rows, int64_t dim, const int64_t *rows, const float *vals,
            const uint8_t *mask, int64_t n, float a, float b) {
    for (int64_t i = 0; i < n; ++i)
        if (rows[i] < -1 || rows[i] >= num_rows) return ORC_EINVAL;
    for (int64_t i = 0; i < n; ++i) {
        if (rows[i] < 0 || (mask && !mask[i])) continue;
        float *t = table + rows[i] * dim;
        const float *v = vals + i * dim;
        for (int64_t d = 0; d < dim; ++d) {
            const float x = a * t[d];
            const float y = b * v[d];
            t[d] = x + y;
        }
    }
    return ORC_OK;
}

/* ------------------------------------- int8 row quantisation [ML] sec. 2, 5 */
/*
 * Raw Embedding Streaming quantises the rows a step touched before they are
 * published to serving, and serving reads int8 rows ([ML] sec. 2 and sec. 5).
 * Per row, asymmetric min-max over the row's fp32 values, each operation
 * rounded in fp32:
 *   scale = fl(fl(max - min) / 255), or 1 when max == min;
 *   bias  = fl(min + fl(128 * scale));
 *   q_d   = clamp(rne(fl(fl(x_d - bias) / scale)), -128, 127),
 * so q_d * scale + bias dequantises back to within about scale / 2.
 * Output i receives row rows[i] (scatter == 0: out index i; scatter == 1: out
 * index rows[i]).  rows[i] == -1 writes q = 0, scale = 0, bias = 0 in the
 * compact form and nothing in the scatter form.  Only the first min(n, count)
 * entries are used (count < 0: n).
 */
int orc_quantize_rows(const float *table, int64_t num_rows, int64_t dim, const int64_t *rows, int64_t n,
                      int64_t count, int32_t scatter, int8_t *out_q, float *out_scale, float *out_bias) {
    const int64_t m = (count >= 0 && count < n) ? count : n;
    for (int64_t i = 0; i < m; ++i)
        if (rows[i] < -1 || rows[i] >= num_rows) return ORC_EINVAL;
    for (int64_t i = 0; i < m; ++i) {
        const int64_t r = rows[i];
        if (r < 0) {
            if (!scatter) {
                memset(out_q + i * dim, 0, (size_t)dim);
                out_scale[i] = 0.0f;
                out_bias[i] = 0.0f;
            }
            continue;
        }
        const int64_t o = scatter ? r : i;
        const float *x = table + r * dim;
        float lo = x[0], hi = x[0];
        for (int64_t d = 1; d < dim; ++d) {
            if (x[d] < lo) lo = x[d];
            if (x[d] > hi) hi = x[d];
        }
        const float range = hi - lo;
        const float scale = (range == 0.0f) ? 1.0f : range / 255.0f;
        const float offset = 128.0f * scale;
        const float bias = lo + offset;
        for (int64_t d = 0; d < dim; ++d) {
            const float centred = x[d] - bias;
            const float v = rintf(centred / scale);
            out_q[o * dim + d] = (int8_t)(v < -128.0f ? -128.0f : (v > 127.0f ? 127.0f : v));
        }
        out_scale[o] = scale;
        out_bias[o] = bias;
    }
    return ORC_OK;
}

/* -------------------------------------------- int8 dequant + dot [ML] sec.5 */
/*
 * scores[q][c] = sum_d (qtable[row][d]*scale[row] + bias[row]) * user[q][d]
 * in fp64, rounded to fp32; row = rows[q*cands + c]; row -1 (miss) scores 0.
 */
int orc_dequant_score(const int8_t *qtable, const float *scale, const float *bias, int64_t num_rows, int64_t dim,
                      const int64_t *rows, int64_t num_requests, int64_t cands, const float *user, float *out) {
    for (int64_t r = 0; r < num_requests; ++r) {
        for (int64_t c = 0; c < cands; ++c) {
            const int64_t row = rows[r * cands + c];
            if (row < -1 || row >= num_rows) return ORC_EINVAL;
            if (row < 0) { out[r * cands + c] = 0.0f; continue; }
            double acc = 0.0;
            for (int64_t d = 0; d < dim; ++d) {
                const double x = (double)qtable[row * dim + d] * (double)scale[row] + (double)bias[row];
                acc += x * (double)user[r * dim + d];
            }
            out[r * cands + c] = (float)acc;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------ hashing trick [DLRM] */
/* rows[i] = mix(ids[i]) mod num_rows: collisions allowed, no identity tensor. */
int orc_hashed_rows(const int64_t *ids, int64_t n, int64_t num_rows, int64_t *rows) {
    if (num_rows <= 0) return ORC_EINVAL;
    for (int64_t i = 0; i < n; ++i) rows[i] = (int64_t)(orc_mix64((uint64_t)ids[i]) % (uint64_t)num_rows);
    return ORC_OK;
}
