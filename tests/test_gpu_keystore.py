"""GPU parity of the decoupled, growable key store (dks_lookup_or_insert, dks_rehash) and its chunked
value store (dks_chunk_init, dks_gather_rows) against the oracle's KeyStore: every position's row and
hit, the stats, the value store (new rows zeroed, the rest untouched), stamps, lookup counts and
next_row bit-exact; the key -> row map compared as a map (the slot a key lands in depends on the order
of concurrent inserts, so only the map is unique)."""
import numpy as np
import pytest
import torch

import hashed_lookup_row_amd as hlr
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hlr.load_library()
    return torch.device("cuda:0")


def to_np(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def bits_equal(a, b):
    return a.shape == b.shape and np.ascontiguousarray(a).tobytes() == np.ascontiguousarray(b).tobytes()


class GpuStore:
    """The raw calls on a value store of fixed size (all its chunks added up front)."""

    def __init__(self, dev, key_cap, max_rows, dim, init_values, shift=6):
        from hashed_lookup_row_amd.keystore import ChunkedValues
        self.dev = dev
        self.keys = torch.full((key_cap,), -1, dtype=torch.int64, device=dev)
        self.krows = torch.full((key_cap,), -1, dtype=torch.int64, device=dev)
        self.v = ChunkedValues(dim, max_rows, dev, chunk_shift=shift)
        assert self.v.max_rows == max_rows  # the tests use whole chunks
        self.v.grow_to(max_rows)
        R = self.v.rows_per_chunk
        for k in range(len(self.v.chunks)):
            self.v._part(k, "vectors").copy_(torch.from_numpy(init_values[k * R:(k + 1) * R]))
        self.next_row = torch.zeros(1, dtype=torch.int64, device=dev)
        self.max_rows = max_rows
        self.stats = torch.zeros(4, dtype=torch.int64, device=dev)
        self.rehashes = 0

    def grow_for(self, n):
        """Keeps the load at most 1/2 after the next batch: rehash into a larger key store (keys only)."""
        used = int(to_np(self.next_row)[0])
        cap = self.keys.numel()
        while used + n > cap // 2:
            cap *= 2
        if cap != self.keys.numel():
            self.keys, self.krows = hlr.dks_rehash(self.keys, self.krows, cap)
            self.rehashes += 1

    def step(self, ids, now, insert=True):
        v = self.v
        rows, hit, st = hlr.dks_lookup_or_insert(self.keys, self.krows, v.table, v.shift, len(v.chunks), v.dim,
                                                 self.next_row, torch.from_numpy(ids).to(self.dev), now, insert,
                                                 out_stats=self.stats)
        return to_np(rows), to_np(hit), to_np(st).copy()

    def dump(self):
        vec, st, ct = self.v.dump()
        return to_np(vec), to_np(st), to_np(ct)

    def mapping(self):
        k, r = to_np(self.keys), to_np(self.krows)
        m = k != -1
        return dict(zip(k[m].tolist(), r[m].tolist()))


def zipf_keys(g, n, s, universe, fresh=0.01):
    ranks = np.minimum(g.zipf(s, size=n), universe) - 1
    keys = ranks.astype(np.int64) * 2654435761 + 12345
    f = g.random(n) < fresh
    keys[f] = -2 - g.integers(0, 1 << 40, size=int(f.sum()))
    keys[g.random(n) < 0.002] = -1
    return keys


@pytest.mark.parametrize("n,steps,dim,max_rows", [(4096, 12, 64, 20_480), (20_000, 6, 128, 30_720),
                                                  (777, 20, 8, 3072)])
def test_key_store_matches_oracle_with_growth(dev, n, steps, dim, max_rows):
    g = np.random.default_rng(n + dim)
    init = g.standard_normal((max_rows, dim)).astype(np.float32)
    gpu = GpuStore(dev, 1024, max_rows, dim, init)
    ora = oracle.KeyStore(1 << 17, max_rows, dim)
    ora.values[:] = init
    for t in range(1, steps + 1):
        ids = zipf_keys(g, n, 1.15, 200_000)
        gpu.grow_for(n)
        rows, hit, st = gpu.step(ids, t)
        orows, ohit, ost = ora.step(ids, t)
        assert np.array_equal(rows, orows), f"rows step {t}"
        assert np.array_equal(hit, ohit), f"hit step {t}"
        assert np.array_equal(st, ost), (t, st, ost)
        assert int(to_np(gpu.next_row)[0]) == int(ora.next_row[0])
    assert gpu.rehashes > 0 or n * steps < 1024
    assert gpu.mapping() == ora.mapping()
    vec, st_, ct = gpu.dump()
    assert np.array_equal(st_, ora.stamps)
    assert np.array_equal(ct, ora.counts.astype(np.int64))
    assert bits_equal(vec, ora.values)
    # lookup-only: same rows for stored keys, nothing changes
    ids = zipf_keys(g, n, 1.15, 200_000)
    before = (to_np(gpu.keys).copy(), gpu.dump(), to_np(gpu.next_row).copy())
    rows, hit, st = gpu.step(ids, steps + 1, insert=False)
    orows, ohit, ost = ora.step(ids, steps + 1, insert=False)
    assert np.array_equal(rows, orows) and np.array_equal(hit, ohit) and np.array_equal(st, ost)
    after = (to_np(gpu.keys), gpu.dump(), to_np(gpu.next_row))
    assert np.array_equal(before[0], after[0]) and np.array_equal(before[2], after[2])
    assert all(np.array_equal(x, y) for x, y in zip(before[1], after[1]))


def test_key_store_overflow(dev):
    """The value store fills up mid-batch: later new keys overflow (row -1, not stored)."""
    g = np.random.default_rng(9)
    dim, max_rows = 16, 512
    init = np.ones((max_rows, dim), np.float32)
    gpu = GpuStore(dev, 4096, max_rows, dim, init)
    ora = oracle.KeyStore(8192, max_rows, dim)
    ora.values[:] = init
    for t in range(1, 5):
        ids = g.integers(0, 5000, size=400).astype(np.int64)
        rows, hit, st = gpu.step(ids, t)
        orows, ohit, ost = ora.step(ids, t)
        assert np.array_equal(rows, orows) and np.array_equal(hit, ohit) and np.array_equal(st, ost), t
    assert int(to_np(gpu.next_row)[0]) == max_rows and ost[2] > 0
    assert gpu.mapping() == ora.mapping()
    vec, st_, ct = gpu.dump()
    assert bits_equal(vec, ora.values) and np.array_equal(ct, ora.counts.astype(np.int64))


def test_rehash_keeps_the_map(dev):
    g = np.random.default_rng(10)
    gpu = GpuStore(dev, 1 << 12, 1536, 4, np.zeros((1536, 4), np.float32))
    gpu.step(g.integers(0, 1 << 50, size=1500).astype(np.int64), 1)
    m = gpu.mapping()
    for cap in (1 << 12, 1 << 13, 1 << 16):
        k, r = hlr.dks_rehash(gpu.keys, gpu.krows, cap)
        kk, rr = to_np(k), to_np(r)
        sel = kk != -1
        assert dict(zip(kk[sel].tolist(), rr[sel].tolist())) == m


@pytest.mark.parametrize("side", [False, True])
def test_dynamic_key_store_grows_without_waiting(dev, side):
    """DynamicKeyStore: batches enqueued back to back (no synchronisation), growth decided from
    completed copies of the row count; every batch's rows equal the oracle's.  With side=True the store
    runs on a stream of its own: its first batch must follow the tables' fill on the current stream, and
    the tables each rehash replaces must stay allocated until that stream is done with them."""
    from hashed_lookup_row_amd.keystore import DynamicKeyStore
    g = np.random.default_rng(12)
    dim, max_rows, n = 32, 60_000, 3000
    store = DynamicKeyStore(dim, max_rows, dev, key_cap=1024, chunk_shift=10,
                            stream=torch.cuda.Stream(dev) if side else None)
    ora = oracle.KeyStore(1 << 18, store.max_rows, dim)
    batches = [zipf_keys(g, n, 1.1, 500_000) for _ in range(15)]
    dev_b = [torch.from_numpy(b).to(dev) for b in batches]
    outs = [torch.empty(n, dtype=torch.int64, device=dev) for _ in batches]
    torch.cuda.synchronize()
    for t, b in enumerate(dev_b):
        store.step(b, t + 1, out_rows=outs[t])
    for t, b in enumerate(batches):
        orows, _, _ = ora.step(b, t + 1, capacity=store.capacity_history[t])
        assert np.array_equal(to_np(outs[t]), orows), t
    assert store.rehashes >= 3
    k, r = to_np(store.keys), to_np(store.krows)
    assert dict(zip(k[k != -1].tolist(), r[k != -1].tolist())) == ora.mapping()
    assert (k != -1).sum() <= store.keys.numel() // 2
    # the value store grew by chunks as rows filled, and every row it holds matches the oracle
    assert len(store.values.chunks) >= 2 and store.capacity_history[0] < store.capacity_history[-1]
    vec, st_, ct = (to_np(x) for x in store.values.dump())
    cap = store.values.capacity
    assert np.array_equal(st_, ora.stamps[:cap]) and np.array_equal(ct, ora.counts[:cap].astype(np.int64))
    assert bits_equal(vec, ora.values[:cap])


def test_value_store_rows_never_move_and_gather(dev):
    """Rows written into the value store keep their place while it grows by chunks (a chunk of 64 rows
    at a time) and the key store is rehashed; dks_gather_rows returns each row's vector, zeros for a
    missing row; lookup-only calls return the stored rows and change no stamp or count."""
    from hashed_lookup_row_amd.keystore import DynamicKeyStore
    g = np.random.default_rng(13)
    dim, n = 12, 300
    store = DynamicKeyStore(dim, 4096, dev, key_cap=256, chunk_shift=6)
    ora = oracle.KeyStore(1 << 14, 4096, dim)
    marked = {}
    for t in range(1, 13):
        ids = g.integers(0, 3000, size=n).astype(np.int64)
        rows, hit = store.step(torch.from_numpy(ids).to(dev), t)
        orows, ohit, _ = ora.step(ids, t, capacity=store.capacity_history[-1])
        assert np.array_equal(to_np(rows), orows) and np.array_equal(to_np(hit), ohit), t
        # write a recognisable vector into every row this batch inserted (the oracle does the same)
        new = np.unique(orows[(orows >= 0) & (ohit == 0)])
        for r in new.tolist():
            v = (np.arange(dim, dtype=np.float32) + 1000.0 * r + 0.25).astype(np.float32)
            ora.values[r] = v
            marked[r] = v
        torch.cuda.synchronize()
        vec = store.values
        for r in new.tolist():
            vec._part(r >> vec.shift, "vectors")[r & (vec.rows_per_chunk - 1)].copy_(torch.from_numpy(marked[r]))
    assert len(store.values.chunks) > 2
    q = np.concatenate([np.array(sorted(marked), np.int64), np.array([-1, 5000], np.int64)])
    got = to_np(store.gather(torch.from_numpy(q).to(dev)))
    want = np.zeros((q.size, dim), np.float32)
    for i, r in enumerate(q.tolist()):
        if 0 <= r < store.values.capacity:
            want[i] = ora.values[r]
    assert bits_equal(got, want)
    before = tuple(to_np(x).copy() for x in store.values.dump())
    ids = g.integers(0, 4000, size=n).astype(np.int64)
    rows, hit = store.lookup(torch.from_numpy(ids).to(dev))
    orows, ohit, _ = ora.step(ids, 99, insert=False, capacity=store.values.capacity)
    assert np.array_equal(to_np(rows), orows) and np.array_equal(to_np(hit), ohit)
    assert all(np.array_equal(a, to_np(b)) for a, b in zip(before, store.values.dump()))
