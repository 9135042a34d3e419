"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks an oracle function against something the pages or the
mathematics fix: published SplitMix64 outputs, textbook LRU caches (batch of one
ID = set-associative LRU; one bucket = fully associative LRU), library routines
(numpy take / unique / cumsum / matmul), exact rational arithmetic, closed forms
and invariants stated on the pages.  A plausible mistake in the oracle (wrong
probe index, wrong victim order, dropped term, wrong sign, transposed operand,
first- instead of last-occurrence) fails at least one of them.
"""
import collections
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U32 = 2.0 ** -24


def f32_from_hex(h):
    return np.frombuffer(struct.pack("<I", int(h, 16)), dtype=np.float32)[0]


# ----------------------------------------------------------------- hashing
def test_mix64_matches_published_splitmix64_outputs():
    want = [int(l.split()[0], 16) for l in open(os.path.join(GOLDEN, "splitmix64_seed0.txt")) if l.startswith("0x")]
    state, got = 0, []
    for _ in want:
        state = (state + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
        got.append(oracle.mix64(state))
    assert got == want


def _golden_splitmix64():
    """(state, output) pairs of the published SplitMix64 sequence for seed 0: state k = k * gamma mod 2^64."""
    want = [int(l.split()[0], 16) for l in open(os.path.join(GOLDEN, "splitmix64_seed0.txt")) if l.startswith("0x")]
    gamma = 0x9E3779B97F4A7C15
    return [((k + 1) * gamma) & 0xFFFFFFFFFFFFFFFF for k in range(len(want))], want


def _as_i64(u):
    return u - (1 << 64) if u >= (1 << 63) else u


def test_bucket_of_published_states_is_published_output_mod_bucket_count():
    """bucket(x, nb) reduces the published hash of x's two's-complement bits: for the SplitMix64 states
    (most of them negative as int64) the bucket is the published output mod nb, for power-of-two and
    other bucket counts."""
    states, outs = _golden_splitmix64()
    for x, h in zip(states, outs):
        for nb in [1, 2, 512, 1 << 19, 7, 524_287, 25_165_824 // 8]:
            assert oracle.bucket(_as_i64(x), nb) == h % nb, (hex(x), nb)


def test_hashed_rows_of_published_states_is_published_output_mod_rows():
    states, outs = _golden_splitmix64()
    ids = np.array([_as_i64(x) for x in states], np.int64)
    for num_rows in [1, 4 << 20, 25_165_824, 5 << 20, 1_000_003]:
        rows = oracle.hashed_rows(ids, num_rows)
        assert rows.tolist() == [h % num_rows for h in outs], num_rows


# ------------------------------------------------------------ textbook LRU
class TextbookSetAssocLRU:
    """Classic set-associative LRU cache: per set an LRU-ordered list of (id, way)."""

    def __init__(self, sets, ways, set_of):
        self.ways, self.set_of = ways, set_of
        self.sets = [collections.OrderedDict() for _ in range(sets)]

    def access(self, x):
        """Returns (hit, way, evicted_id or -1)."""
        s = self.sets[self.set_of(x)]
        if x in s:
            s.move_to_end(x)
            return True, s[x], -1
        used = set(s.values())
        if len(s) < self.ways:
            way = min(w for w in range(self.ways) if w not in used)
            s[x] = way
            return False, way, -1
        victim, way = s.popitem(last=False)
        s[x] = way
        return False, way, victim


@pytest.mark.parametrize("capacity,universe,steps", [(64, 200, 3000), (4096, 10_000, 6000)])
def test_batch_of_one_is_textbook_set_associative_lru(capacity, universe, steps):
    P = 8
    nb = capacity // P
    t = oracle.MPZCHTable(capacity, P, 4)
    g = synth.rng(77, capacity)
    keys = synth.universe_keys(universe, 77)
    stream = keys[synth.zipf_ranks(g, universe, 1.1, steps)]
    ref = TextbookSetAssocLRU(nb, P, lambda x: oracle.bucket(int(x), nb))
    for now, x in enumerate(stream, start=1):
        rows, hit, ev, st = t.step(np.array([x]), now)
        h, way, victim = ref.access(int(x))
        assert bool(hit[0]) == h
        assert rows[0] == oracle.bucket(int(x), nb) * P + way
        assert ev[0] == victim
    resident = {int(x) for x in t.identity if x != -1}
    assert resident == {k for s in ref.sets for k in s}


def test_one_bucket_is_fully_associative_lru():
    """capacity == probes: no hashing is involved at all."""
    P = 8
    t = oracle.MPZCHTable(P, P, 2)
    seq = [5, 6, 7, 5, 8, 9, 10, 11, 12, 13, 5, 14, 6, 15, 7, 5, 16]
    lru = collections.OrderedDict()
    for now, x in enumerate(seq, start=1):
        rows, hit, ev, _ = t.step(np.array([x]), now)
        if x in lru:
            lru.move_to_end(x)
            assert hit[0] == 1 and ev[0] == -1
        else:
            victim = -1
            if len(lru) == P:
                victim, _ = lru.popitem(last=False)
            lru[x] = None
            assert hit[0] == 0 and ev[0] == victim
    assert set(t.identity.tolist()) == set(lru)


# ------------------------------------------------- batch-level invariants
def _bucket_members(ids, nb):
    return [oracle.bucket(int(x), nb) for x in ids]


def _check_batch(tab, ids, now, rows, hit, ev, st, before_id, before_st):
    P, C = tab.probes, tab.capacity
    nb = C // P
    resident0 = {int(x): s for s, x in enumerate(before_id) if x != -1}
    # zero collisions: the identity map stays injective and every ID sits in its own bucket
    live = tab.identity[tab.identity != -1]
    assert np.unique(live).size == live.size
    for s in np.nonzero(tab.identity != -1)[0]:
        assert oracle.bucket(int(tab.identity[s]), nb) == s // P
    seen_row = {}
    for i, x in enumerate(ids):
        x = int(x)
        if x == -1:
            assert rows[i] == -1 and hit[i] == 0
            continue
        # hit mask = membership at batch start (plain set)
        assert bool(hit[i]) == (x in resident0)
        if rows[i] >= 0:
            assert tab.identity[rows[i]] == x
            assert tab.stamps[rows[i]] == now
        # all positions of one ID share one row
        assert seen_row.setdefault(x, rows[i]) == rows[i]
    # rows of hits never move within the batch
    for i, x in enumerate(ids):
        if hit[i]:
            assert rows[i] == resident0[int(x)]
    # evicted IDs: were resident, not in this batch, and LRU among the bucket's unpinned slots
    batch = {int(x) for x in ids}
    evicted = [int(e) for e in ev if e != -1]
    assert len(evicted) == st[2] and len(set(evicted)) == len(evicted)
    for e in evicted:
        assert e in resident0 and e not in batch
        s = resident0[e]
        b = s // P
        survivors = [before_st[q] for q in range(b * P, b * P + P)
                     if before_id[q] != -1 and tab.identity[q] == before_id[q] and tab.stamps[q] != now]
        assert all(before_st[s] <= v for v in survivors)
    # an eviction only happens in a bucket that had no empty slot left
    for e in evicted:
        b = resident0[e] // P
        assert not np.any(tab.identity[b * P:(b + 1) * P] == -1)
    # overflow only when every slot of the bucket is pinned by this batch
    for i, x in enumerate(ids):
        if x != -1 and rows[i] == -1:
            b = oracle.bucket(int(x), nb)
            assert np.all(tab.stamps[b * P:(b + 1) * P] == now)
    # inserted rows are zero vectors (a new ID never reads an evicted vector)
    if tab.values is not None:
        for i in range(len(ids)):
            if rows[i] >= 0 and not hit[i]:
                assert not np.any(tab.values[rows[i]])
    assert st[0] == int(np.sum(hit)) and st[4] == int(np.sum(np.asarray(ids) == -1))


def test_invariants_on_tiny_config_stream():
    cfg = synth.TINY
    tab = oracle.MPZCHTable(cfg.capacity, cfg.probes, cfg.dim)
    for t, ids in enumerate(synth.mpzch_stream(cfg, 30), start=1):
        ids = ids.copy()
        ids[::97] = -1  # sprinkle invalid IDs
        bid, bst = tab.identity.copy(), tab.stamps.copy()
        tab.values[:] = 1.0  # so zero-fill is observable
        rows, hit, ev, st = tab.step(ids, t)
        _check_batch(tab, ids, t, rows, hit, ev, st, bid, bst)


def _ids_in_bucket(target, nb, count, start=1):
    out, x = [], start
    while len(out) < count:
        if oracle.bucket(x, nb) == target:
            out.append(x)
        x += 1
    return out


def test_crafted_bucket_overflow_empty_first_lru_and_ties():
    P, C = 8, 64
    nb = C // P
    ids = _ids_in_bucket(3, nb, 24)
    t = oracle.MPZCHTable(C, P, 4)
    # 1) 11 new IDs in one empty bucket: first 8 by first occurrence take slots 0..7 in probe order, 3 overflow
    batch = np.array(ids[:11][::-1] + [ids[10]], np.int64)  # reversed, plus a duplicate of the first one
    rows, hit, ev, st = t.step(batch, 10)
    assert rows[:8].tolist() == [3 * P + j for j in range(8)]
    assert rows[8:11].tolist() == [-1, -1, -1] and rows[11] == rows[0]
    assert st.tolist() == [0, 8, 0, 3, 0]
    # 2) later batch, 2 new IDs: victims are the two smallest stamps; equal stamps -> lowest probe index
    t.stamps[3 * P:3 * P + 8] = [50, 20, 20, 40, 30, 60, 70, 80]
    resid = t.identity[3 * P:3 * P + 8].copy()
    rows, hit, ev, st = t.step(np.array([ids[20], ids[21]], np.int64), 100)
    assert rows.tolist() == [3 * P + 1, 3 * P + 2]
    assert ev.tolist() == [resid[1], resid[2]]
    # 3) a resident hit in the batch is pinned and can't be chosen as victim
    t.stamps[3 * P:3 * P + 8] = [5, 6, 7, 8, 9, 10, 11, 12]
    hot = int(t.identity[3 * P])
    rows, hit, ev, st = t.step(np.array([ids[22], hot], np.int64), 200)
    assert hit.tolist() == [0, 1] and rows[0] == 3 * P + 1 and rows[1] == 3 * P


def test_lookup_only_changes_nothing():
    t = oracle.MPZCHTable(64, 8, 4)
    t.step(np.arange(1, 40, dtype=np.int64), 1)
    ident, stamps, vals = t.identity.copy(), t.stamps.copy(), t.values.copy()
    ids = np.arange(20, 60, dtype=np.int64)
    rows, hit, ev, st = t.step(ids, 2, insert=False)
    assert np.array_equal(ident, t.identity) and np.array_equal(stamps, t.stamps) and np.array_equal(vals, t.values)
    for i, x in enumerate(ids):
        if hit[i]:
            assert ident[rows[i]] == x
        else:
            assert rows[i] == -1 and x not in set(ident.tolist())


def test_non_increasing_now_is_rejected():
    t = oracle.MPZCHTable(64, 8, 4)
    t.step(np.array([1, 2], np.int64), 5)
    with pytest.raises(ValueError):
        t.step(np.array([3], np.int64), 5)


# ------------------------------------------------------------------ gather
def test_gather_matches_numpy_take_and_zero_for_misses():
    g = np.random.default_rng(1)
    table = g.standard_normal((100, 12)).astype(np.float32)
    rows = g.integers(-1, 100, size=777)
    out = oracle.gather(table, rows)
    ref = np.where((rows >= 0)[:, None], np.take(table, np.maximum(rows, 0), axis=0), 0.0)
    assert np.array_equal(out, ref.astype(np.float32))


# ------------------------------------------------------------------- dedup
@pytest.mark.parametrize("n", [0, 1, 5, 1000, 4099])
def test_dedup_matches_numpy_unique_and_last_occurrence(n):
    g = np.random.default_rng(n)
    keys = g.integers(-50, 50, size=n).astype(np.int64) * (1 << 40) + g.integers(0, 3, size=n)
    uq, lp, inv = oracle.dedup(keys)
    ref_u, ref_inv = np.unique(keys, return_inverse=True)
    assert np.array_equal(uq, ref_u)
    assert np.array_equal(inv, ref_inv.reshape(-1))
    last = {}
    for i, k in enumerate(keys.tolist()):
        last[k] = i
    assert lp.tolist() == [last[k] for k in ref_u.tolist()]


# --------------------------------------------------------------- Writeback
def test_writeback_golden_fp32_cases():
    for line in open(os.path.join(GOLDEN, "writeback_fp32_cases.txt")):
        if not line.startswith("0x"):
            continue
        m, e, want = [f32_from_hex(h) for h in line.split()[:3]]
        table = np.array([[m, 7.0]], np.float32)
        oracle.writeback_last(table, np.array([0]), np.array([[e, 7.0]], np.float32))
        assert table[0, 0].tobytes() == np.float32(want).tobytes(), line


def test_writeback_closed_form_bound_last_wins_untouched():
    g = np.random.default_rng(5)
    C, D, n = 300, 16, 2000
    table = (g.standard_normal((C, D)) * g.choice([1e-3, 1.0, 1e3], size=(C, 1))).astype(np.float32)
    table[:40] = 0.0  # fresh rows
    rows = g.integers(-1, 200, size=n)
    e = g.standard_normal((n, D)).astype(np.float32)
    before = table.copy()
    oracle.writeback_last(table, rows, e)
    last = {}
    for i, r in enumerate(rows.tolist()):
        if r >= 0:
            last[r] = i
    for r in range(C):
        if r not in last:
            assert np.array_equal(table[r], before[r])  # untouched rows are bit-identical
            continue
        ev = e[last[r]]
        for d in range(D):
            v, ee, out = Fraction(float(before[r, d])), Fraction(float(ev[d])), Fraction(float(table[r, d]))
            if v == 0 or (ee / 2 <= v <= 2 * ee) or (2 * ee <= v <= ee / 2):
                assert out == ee  # exact: 0-(0-e) and Sterbenz
            bound = Fraction(U32) * (abs(v - ee) + abs(ee)) * (1 + Fraction(U32))
            assert abs(out - ee) <= bound


# ------------------------------------------------------------ SGD-sum
def _exact_update(w, gs, lr):
    return Fraction(float(w)) - Fraction(float(lr)) * sum(Fraction(float(x)) for x in gs)


def test_sgd_sum_every_segment_length_equals_sequential_cumsum():
    """Each row's sum is numpy's float32 cumsum (np.add.accumulate: strictly sequential) over the row's
    gradients in batch order, for segments of every length from 1 to a few thousand."""
    g = np.random.default_rng(9)
    C, D = 60, 8
    lens = np.concatenate([np.arange(1, 41), [63, 64, 65, 255, 256, 257, 511, 512, 513, 1000, 2049, 4100]])
    rows = np.concatenate([np.full(k, r, np.int64) for r, k in enumerate(lens)] + [np.full(50, -1, np.int64)])
    g.shuffle(rows)
    n = rows.size
    table = g.standard_normal((C, D)).astype(np.float32)
    grads = (g.standard_normal((n, D)) * 1e-3).astype(np.float32)
    before = table.copy()
    oracle.sgd_sum(table, rows, grads, 0.01)
    for r in range(C):
        pos = np.nonzero(rows == r)[0]
        if pos.size == 0:
            assert np.array_equal(table[r], before[r])
            continue
        assert pos.size == lens[r]
        s = np.cumsum(grads[pos], axis=0, dtype=np.float32)[-1]
        want = before[r] - (np.float32(0.01) * s).astype(np.float32)
        assert np.array_equal(table[r], want.astype(np.float32)), r


def test_sgd_sum_long_segment_within_exact_bound():
    """The running sum of k terms is within (k-1) 2^-24 sum|g| of the exact rational sum, and the update
    adds two more roundings."""
    g = np.random.default_rng(11)
    D, k = 4, 3000
    rows = np.zeros(k, np.int64)
    grads = (g.standard_normal((k, D)) * 1e-3).astype(np.float32)
    table = np.ones((1, D), np.float32)
    oracle.sgd_sum(table, rows, grads, 1.0)
    for d in range(D):
        exact = _exact_update(1.0, grads[:, d], 1.0)
        err_bound = Fraction(k + 2) * Fraction(U32) * (sum(abs(Fraction(float(x))) for x in grads[:, d]) + 1)
        assert abs(Fraction(float(table[0, d])) - exact) <= err_bound


def test_sgd_sum_order_is_ascending_batch_position():
    """Three gradients whose fp32 sum depends on the order: 1 + 2^-24 + 2^-24 rounds to 1 left to right
    (each tiny term is lost) but to 1 + 2^-23 when the tiny terms come first.  The row's result tells the
    order: batch order must give exactly M - 1."""
    tiny = np.float32(2.0 ** -24)
    grads = np.array([[1.0], [tiny], [tiny]], np.float32)
    t = np.zeros((1, 1), np.float32)
    oracle.sgd_sum(t, np.zeros(3, np.int64), grads, 1.0)
    assert t[0, 0] == np.float32(-1.0)
    t = np.zeros((1, 1), np.float32)
    oracle.sgd_sum(t, np.zeros(3, np.int64), grads[::-1].copy(), 1.0)
    assert t[0, 0] == -(np.float32(1.0) + np.float32(2.0 ** -23))


def test_sgd_sum_learning_rate_scales_the_row_sum_once():
    """lr multiplies the row's finished sum once (R11: M' = fl(M - fl(lr s))), not every gradient: with
    gradients 1 and 2^-24 and lr = 3, the batch-order sum is fl(1 + 2^-24) = 1 (a tie, to even), so a zero
    row becomes -3 exactly, while scaling each term first would give 3 + 3 2^-24, which rounds to
    3 + 2^-22.  On zero rows (where the final subtraction loses nothing) random rows also equal
    -fl(lr * s) with s the sequential float32 sum."""
    t = np.zeros((1, 1), np.float32)
    oracle.sgd_sum(t, np.zeros(2, np.int64), np.array([[1.0], [2.0 ** -24]], np.float32), 3.0)
    assert t[0, 0] == np.float32(-3.0)
    g = np.random.default_rng(21)
    C, D, n = 8, 16, 400
    rows = g.integers(0, C, size=n)
    grads = (g.standard_normal((n, D)) * 1e-3).astype(np.float32)
    t = np.zeros((C, D), np.float32)
    oracle.sgd_sum(t, rows, grads, 0.01)
    for r in range(C):
        s = np.cumsum(grads[rows == r], axis=0, dtype=np.float32)[-1]
        assert np.array_equal(t[r], -(np.float32(0.01) * s).astype(np.float32))


def test_sgd_sum_integer_gradients_are_exact():
    g = np.random.default_rng(3)
    rows = g.integers(0, 5, size=2000)
    grads = g.integers(-8, 9, size=(2000, 3)).astype(np.float32)
    table = np.zeros((5, 3), np.float32)
    oracle.sgd_sum(table, rows, grads, 0.5)
    for r in range(5):
        assert np.array_equal(table[r], -0.5 * grads[rows == r].sum(axis=0))


# ------------------------------------------------ decoupled key store (MTGR)
def _dict_store(stream, max_rows):
    """Reference key -> row map: a Python dict, rows handed out in order of first appearance.
    max_rows: the rows the store holds, one number or one per batch (a growing value store)."""
    d, out = {}, []
    caps = max_rows if isinstance(max_rows, (list, tuple)) else [max_rows] * len(stream)
    for ids, max_rows in zip(stream, caps):
        rows, hit = [], []
        pending = {}
        for k in ids.tolist():
            if k == -1:
                rows.append(-1), hit.append(0)
            elif k in d:
                rows.append(d[k]), hit.append(1)
            else:
                rows.append(None), hit.append(0)
        for i, k in enumerate(ids.tolist()):  # misses in order of first occurrence
            if rows[i] is None:
                if k not in pending:
                    pending[k] = len(d) + len(pending) if len(d) + len(pending) < max_rows else -1
                rows[i] = pending[k]
        for k, r in pending.items():
            if r >= 0:
                d[k] = r
        inserted = sum(1 for r in pending.values() if r >= 0)
        out.append((np.array(rows), np.array(hit, np.int8), inserted, len(pending) - inserted))
    return d, out


def test_key_store_matches_dict_reference_and_table_invariants():
    g = np.random.default_rng(41)
    stream = [np.where(g.random(300) < 0.02, -1, g.zipf(1.3, size=300) * 7919 - 50).astype(np.int64)
              for _ in range(12)]
    for key_cap, max_rows in [(1024, 700), (512, 200), (256, 255)]:
        ks = oracle.KeyStore(key_cap, max_rows, 4)
        ks.values[:] = 1.0
        d, ref = _dict_store(stream, max_rows)
        for t, ids in enumerate(stream):
            rows, hit, st = ks.step(ids, t + 1)
            assert np.array_equal(rows, ref[t][0]) and np.array_equal(hit, ref[t][1]), (key_cap, t)
            assert st[3] == np.count_nonzero(ids == -1) and st[0] == hit.sum()
            assert (st[1], st[2]) == (ref[t][2], ref[t][3]), (key_cap, t)  # inserted and overflowed keys
        assert ks.mapping() == d and ks.next_row[0] == len(d)
        used = ks.keys != -1
        for s in np.nonzero(used)[0]:  # every key reachable from its home slot without crossing an empty slot
            home = oracle.mix64(int(ks.keys[s])) % key_cap
            j = home
            while j != s:
                assert ks.keys[j] >= 0
                j = (j + 1) % key_cap
        new_rows = np.arange(len(d))
        assert np.all(ks.values[new_rows] == 0) and np.all(ks.values[len(d):] == 1)  # only new rows zeroed


def test_key_store_counts_and_growing_value_store_match_dict_reference():
    """The value store grows between batches (the rows it holds per batch rise in steps, and stay below
    the keys offered for a while, so keys overflow and later batches insert them): rows, hits and the
    key -> row map equal the dict reference, and each row's count is the number of positions, over all
    batches, whose key had that row (a Counter over the reference's rows), never counting overflowed
    or invalid positions."""
    g = np.random.default_rng(43)
    stream = [np.where(g.random(400) < 0.02, -1, g.zipf(1.2, size=400) * 104729 - 7).astype(np.int64)
              for _ in range(14)]
    caps = [16, 16, 48, 48, 48, 112, 112, 240, 240, 240, 496, 496, 496, 1008]
    ks = oracle.KeyStore(2048, 1008, 4)
    d, ref = _dict_store(stream, caps)
    want = np.zeros(1008, np.int64)
    for t, ids in enumerate(stream):
        rows, hit, st = ks.step(ids, t + 1, capacity=caps[t])
        assert np.array_equal(rows, ref[t][0]) and np.array_equal(hit, ref[t][1]), t
        assert (st[1], st[2]) == (ref[t][2], ref[t][3]), t
        assert ks.next_row[0] <= caps[t]
        for r in ref[t][0].tolist():
            if r >= 0:
                want[r] += 1
    assert ks.mapping() == d
    assert np.array_equal(ks.counts.astype(np.int64), want)
    assert want[:ks.next_row[0]].min() >= 1 and not want[ks.next_row[0]:].any()
    # a lookup-only batch counts nothing
    before = ks.counts.copy()
    ks.step(stream[0], 99, insert=False, capacity=caps[-1])
    assert np.array_equal(ks.counts, before)


def test_key_store_lookup_only_changes_nothing_and_stamps():
    ks = oracle.KeyStore(64, 32, 2)
    ks.step(np.array([3, 4, 3, 5], np.int64), 1)
    before = (ks.keys.copy(), ks.krows.copy(), ks.stamps.copy(), ks.next_row.copy())
    rows, hit, st = ks.step(np.array([4, 9, 3], np.int64), 2, insert=False)
    assert rows.tolist() == [1, -1, 0] and hit.tolist() == [1, 0, 1] and st[1] == 0
    assert all(np.array_equal(a, b) for a, b in zip(before, (ks.keys, ks.krows, ks.stamps, ks.next_row)))
    ks.step(np.array([5, 6], np.int64), 3)
    assert ks.stamps[:4].tolist() == [1, 1, 3, 3]  # rows of 3, 4 last touched in batch 1; 5 and new 6 in batch 3


# ------------------------------------------------------------ L2 alignment
def test_l2_align_single_occurrence_half_rate_is_writeback():
    """lr = 0.5, one occurrence per row: M - 0.5 * 2 (M - e) is the Writeback assignment
    fl(M - fl(M - e)) exactly (the doubling and the halving are exact)."""
    g = np.random.default_rng(21)
    C, D = 40, 16
    rows = g.permutation(C)[:25].astype(np.int64)
    e = g.standard_normal((25, D)).astype(np.float32)
    table = g.standard_normal((C, D)).astype(np.float32)
    before = table.copy()
    oracle.l2_align(table, rows, e, 0.5)
    want = before.copy()
    want[rows] = before[rows] - (before[rows] - e)  # numpy float32: each operation rounded
    assert np.array_equal(table, want)


def test_l2_align_duplicates_exact_on_short_dyadics():
    """Values on a coarse dyadic grid make every partial sum exact, so the result must be the exact
    M - lr * sum_i 2 (M - e_i) with M the row before the batch (catches a dropped factor 2, a
    flipped sign, or a gradient taken at the partly updated row)."""
    g = np.random.default_rng(22)
    C, D, n = 6, 4, 900
    rows = g.integers(-1, C, size=n).astype(np.int64)
    rows[:300] = 2  # one row with 300+ occurrences
    e = (g.integers(-64, 65, size=(n, D)) / 16.0).astype(np.float32)
    table = (g.integers(-64, 65, size=(C, D)) / 16.0).astype(np.float32)
    before = table.copy()
    lr = 2.0 ** -12
    oracle.l2_align(table, rows, e, lr)
    for r in range(C):
        pos = np.nonzero(rows == r)[0]
        for d in range(D):
            m = Fraction(float(before[r, d]))
            exact = m - Fraction(lr) * sum(2 * (m - Fraction(float(e[i, d]))) for i in pos)
            assert Fraction(float(table[r, d])) == exact, (r, d)


def test_l2_align_duplicates_at_matching_rate_assign_e():
    """k copies of the same target with lr = 1 / (2k) move the row onto the target exactly."""
    for k in (1, 2, 8, 64):
        e = np.array([[1.5, -0.25, 3.0, 0.0]], np.float32)
        table = np.array([[0.5, 2.0, -1.0, 7.0], [9.0, 9.0, 9.0, 9.0]], np.float32)
        oracle.l2_align(table, np.zeros(k, np.int64), np.repeat(e, k, axis=0), 1.0 / (2 * k))
        assert np.array_equal(table[0], e[0]) and np.array_equal(table[1], np.full(4, 9.0, np.float32))


# ------------------------------------------------------- int8 quantisation
def test_quantize_integer_grid_is_exact():
    """min 0 and max 255 give scale 1 and bias 128, so integer values map to x - 128 exactly; scaling
    the row by a power of two scales scale and bias by it and leaves the codes unchanged."""
    g = np.random.default_rng(31)
    vals = g.integers(0, 256, size=(3, 40)).astype(np.float32)
    vals[:, 0], vals[:, 1] = 0.0, 255.0
    for k in (0, 3, -5):
        t = (vals * np.float32(2.0 ** k)).astype(np.float32)
        q, sc, bi = oracle.quantize_rows(t, np.arange(3))
        assert np.array_equal(q.astype(np.int64), vals.astype(np.int64) - 128)
        assert np.all(sc == np.float32(2.0 ** k)) and np.all(bi == np.float32(128 * 2.0 ** k))


def test_quantize_constant_row_and_ties_to_even():
    t = np.full((1, 8), -3.25, np.float32)
    q, sc, bi = oracle.quantize_rows(t, np.array([0]))
    assert sc[0] == 1.0 and bi[0] == np.float32(-3.25 + 128) and np.all(q == -128)
    assert q[0, 0] * sc[0] + bi[0] == np.float32(-3.25)  # dequantises exactly
    # scale 1, bias 128: x = 3.5 -> -124.5 -> -124 (even); 4.5 -> -123.5 -> -124; 5.5 -> -122.5 -> -122
    row = np.array([[0.0, 255.0, 3.5, 4.5, 5.5, 6.5]], np.float32)
    q, _, _ = oracle.quantize_rows(row, np.array([0]))
    assert q[0].tolist() == [-128, 127, -124, -124, -122, -122]


def test_quantize_round_trip_bound_and_layouts():
    """|q*scale + bias - x| <= scale/2 up to a few ulps for every value; codes span [-128, 127]; the
    scatter form writes row r's codes at index r; rows of -1 and the count limit are honoured."""
    g = np.random.default_rng(32)
    t = (g.standard_normal((50, 64)) * g.uniform(0.01, 10, size=(50, 1))).astype(np.float32)
    rows = np.array([7, 3, -1, 49, 7, 0], np.int64)
    q, sc, bi = oracle.quantize_rows(t, rows)
    for i, r in enumerate(rows):
        if r < 0:
            assert not q[i].any() and sc[i] == 0 and bi[i] == 0
            continue
        deq = q[i].astype(np.float64) * sc[i] + bi[i]
        assert np.all(np.abs(deq - t[r]) <= 0.5 * sc[i] * (1 + 1e-5) + 4 * np.spacing(np.abs(t[r]).max()))
        assert q[i].min() == -128 and q[i].max() == 127
    out = (np.zeros((50, 64), np.int8), np.zeros(50, np.float32), np.zeros(50, np.float32))
    oracle.quantize_rows(t, rows, scatter=True, out=out)
    for i, r in enumerate(rows):
        if r >= 0:
            assert np.array_equal(out[0][r], q[i]) and out[1][r] == sc[i] and out[2][r] == bi[i]
    assert not out[0][1].any()  # untouched rows stay as they were
    q2, _, _ = oracle.quantize_rows(t, rows, count=2)
    assert np.array_equal(q2[:2], q[:2]) and not q2[2:].any()


# -------------------------------------------------------------------- EMA
def test_ema_special_cases():
    g = np.random.default_rng(2)
    C, D, n = 20, 5, 400
    rows = g.integers(-1, C, size=n)
    vals = g.standard_normal((n, D)).astype(np.float32)
    mask = (g.random(n) < 0.3).astype(np.uint8)
    t0 = g.standard_normal((C, D)).astype(np.float32)
    # a=0, b=1: the row ends as the last masked value exactly
    t = t0.copy()
    oracle.ema(t, rows, vals, mask, 0.0, 1.0)
    for r in range(C):
        pos = [i for i in range(n) if rows[i] == r and mask[i]]
        assert np.array_equal(t[r], vals[pos[-1]] if pos else t0[r])
    # a=1, b=0: unchanged; empty mask: unchanged
    t = t0.copy()
    oracle.ema(t, rows, vals, None, 1.0, 0.0)
    assert np.array_equal(t, t0)
    t = t0.copy()
    oracle.ema(t, rows, vals, np.zeros(n, np.uint8), 0.99, 0.01)
    assert np.array_equal(t, t0)


def test_ema_rounds_each_product_before_the_sum():
    """R15: T' = fl(fl(a T) + fl(b v)).  Each float32 product is exact in float64 (24 + 24 bits) and the sum
    of two float32 values is exact in float64 here, so rounding those float64 values to float32 gives the
    IEEE float32 result of each operation.  The cases are the seeded ones where that differs from rounding
    the exact a T + b v once; the oracle must give the per-operation result."""
    g = np.random.default_rng(31)
    a, b = np.float32(0.95), np.float32(0.05)
    T = g.standard_normal(20000).astype(np.float32)
    v = g.standard_normal(20000).astype(np.float32)
    x = np.float32(np.float64(a) * np.float64(T))
    y = np.float32(np.float64(b) * np.float64(v))
    per_op = np.float32(np.float64(x) + np.float64(y))
    exact = [Fraction(float(a)) * Fraction(float(t)) + Fraction(float(b)) * Fraction(float(w)) for t, w in zip(T, v)]
    once = np.array([np.float32(float(e)) for e in exact], np.float32)
    pick = np.nonzero(per_op != once)[0][:200]
    assert pick.size >= 20  # the readings differ often enough to tell them apart
    t = T[pick].reshape(-1, 1).copy()
    oracle.ema(t, np.arange(pick.size), v[pick].reshape(-1, 1), None, float(a), float(b))
    assert np.array_equal(t[:, 0], per_op[pick])


def test_ema_rejects_rows_outside_the_table():
    t = np.zeros((4, 2), np.float32)
    vals = np.ones((2, 2), np.float32)
    for bad in ([0, 4], [-2, 1]):
        with pytest.raises(ValueError):
            oracle.ema(t, np.array(bad, np.int64), vals, None, 0.5, 0.5)
    assert not t.any()


def test_ema_dyadic_values_are_exact_rationals():
    """Small dyadic inputs with a=1/2, b=1/4: no rounding occurs, result = exact recurrence."""
    g = np.random.default_rng(4)
    C, D, n = 6, 3, 40
    rows = g.integers(0, C, size=n)
    vals = g.integers(-16, 17, size=(n, D)).astype(np.float32)
    t = g.integers(-16, 17, size=(C, D)).astype(np.float32)
    exact = [[Fraction(float(x)) for x in row] for row in t]
    oracle.ema(t, rows, vals, None, 0.5, 0.25)
    for i in range(n):
        r = rows[i]
        exact[r] = [Fraction(1, 2) * exact[r][d] + Fraction(1, 4) * Fraction(float(vals[i, d])) for d in range(D)]
    for r in range(C):
        assert [Fraction(float(x)) for x in t[r]] == exact[r]


def test_ema_within_fp64_closed_form():
    g = np.random.default_rng(6)
    D, k = 16, 3000
    vals = g.standard_normal((k, D)).astype(np.float32)
    t0 = g.standard_normal((1, D)).astype(np.float32)
    for a, b in [(0.99, 0.01), (0.95, 0.05)]:
        t = t0.copy()
        oracle.ema(t, np.zeros(k, np.int64), vals, None, a, b)
        af, bf = float(np.float32(a)), float(np.float32(b))
        w = af ** np.arange(k - 1, -1, -1, dtype=np.float64)
        closed = af ** k * t0[0].astype(np.float64) + bf * (w[:, None] * vals.astype(np.float64)).sum(axis=0)
        m = af ** k * np.abs(t0[0]) + bf * (w[:, None] * np.abs(vals)).sum(axis=0)
        # sequential fp32 rounding: at most ~2 roundings per step, damped by a
        assert np.all(np.abs(t[0] - closed) <= 2.5 * U32 / (1 - af) * m + 1e-30)


# ---------------------------------------------------------- dequant-score
def test_dequant_score_special_cases_and_library_matmul():
    g = np.random.default_rng(8)
    C, D, R, K = 50, 32, 4, 20
    q = g.integers(-128, 128, size=(C, D)).astype(np.int8)
    scale = (g.random(C) * 0.01 + 1e-3).astype(np.float32)
    bias = (g.standard_normal(C) * 0.01).astype(np.float32)
    rows = g.integers(-1, C, size=R * K)
    user = g.standard_normal((R, D)).astype(np.float32)
    out = oracle.dequant_score(q, scale, bias, rows, user, K)
    x = q.astype(np.float64) * scale[:, None].astype(np.float64) + bias[:, None].astype(np.float64)
    ref = np.einsum("rkd,rd->rk", x[np.maximum(rows, 0)].reshape(R, K, D), user.astype(np.float64))
    ref[rows.reshape(R, K) < 0] = 0.0
    scale_ = np.einsum("rkd,rd->rk", np.abs(x[np.maximum(rows, 0)].reshape(R, K, D)), np.abs(user.astype(np.float64)))
    assert np.all(np.abs(out - ref) <= 1e-7 * scale_ + 1e-30)
    assert np.all(out[rows.reshape(R, K) < 0] == 0.0)
    # one-hot user vector picks x_d; all-zero codes give bias * sum(u)
    onehot = np.zeros((1, D), np.float32)
    onehot[0, 5] = 1.0
    r1 = np.arange(C, dtype=np.int64)
    s1 = oracle.dequant_score(q, scale, bias, r1, onehot, C)
    assert np.array_equal(s1[0], x[:, 5].astype(np.float32))
    s0 = oracle.dequant_score(np.zeros_like(q), scale, bias, r1, user[:1], C)
    assert np.allclose(s0[0], bias.astype(np.float64) * user[0].astype(np.float64).sum(), rtol=1e-6, atol=0)


# -------------------------------------------------------------- generators
def test_zipf_sampler_matches_pmf_chi2():
    g = synth.rng(123, 0)
    n_univ, s, draws = 1000, 1.1, 200_000
    r = synth.zipf_ranks(g, n_univ, s, draws)
    p = synth.zipf_pmf(n_univ, s)
    obs = np.bincount(r, minlength=n_univ)[:50].astype(np.float64)
    exp = p[:50] * draws
    chi2 = float(np.sum((obs - exp) ** 2 / exp))
    assert chi2 < 100.0  # 49 dof: p(chi2 > 100) ~ 2e-5


def test_tiny_config_distinct_count_near_expectation():
    cfg = synth.TINY
    e_u = synth.expected_distinct(cfg.universe, cfg.zipf_s, cfg.batch)
    assert 380 < e_u < 440
    us = [np.unique(ids).size for ids in synth.mpzch_stream(cfg, 20)]
    assert abs(np.mean(us) - e_u) < 15
