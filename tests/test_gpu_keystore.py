"""GPU parity of the decoupled, growable key store (dks_lookup_or_insert, dks_rehash) against the
oracle's KeyStore: every position's row and hit, the stats, the value store (new rows zeroed, the
rest untouched), stamps and next_row bit-exact; the key -> row map compared as a map (the slot a
key lands in depends on the order of concurrent inserts, so only the map is unique)."""
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
    def __init__(self, dev, key_cap, max_rows, dim, init_values):
        self.dev = dev
        self.keys = torch.full((key_cap,), -1, dtype=torch.int64, device=dev)
        self.krows = torch.full((key_cap,), -1, dtype=torch.int64, device=dev)
        self.stamps = torch.full((max_rows,), -1, dtype=torch.int64, device=dev)
        self.values = torch.from_numpy(init_values.copy()).to(dev)
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
        rows, hit, st = hlr.dks_lookup_or_insert(self.keys, self.krows, self.stamps, self.values, self.max_rows,
                                                 self.next_row, torch.from_numpy(ids).to(self.dev), now, insert,
                                                 out_stats=self.stats)
        return to_np(rows), to_np(hit), to_np(st).copy()

    def mapping(self):
        k, r = to_np(self.keys), to_np(self.krows)
        m = k >= 0
        return dict(zip(k[m].tolist(), r[m].tolist()))


def zipf_keys(g, n, s, universe, fresh=0.01):
    ranks = np.minimum(g.zipf(s, size=n), universe) - 1
    keys = ranks.astype(np.int64) * 2654435761 + 12345
    f = g.random(n) < fresh
    keys[f] = -2 - g.integers(0, 1 << 40, size=int(f.sum()))
    keys[g.random(n) < 0.002] = -1
    return keys


@pytest.mark.parametrize("n,steps,dim,max_rows", [(4096, 12, 64, 20_000), (20_000, 6, 128, 30_000),
                                                  (777, 20, 8, 3000)])
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
    assert np.array_equal(to_np(gpu.stamps), ora.stamps)
    assert bits_equal(to_np(gpu.values), ora.values)
    # lookup-only: same rows for stored keys, nothing changes
    ids = zipf_keys(g, n, 1.15, 200_000)
    before = (to_np(gpu.keys).copy(), to_np(gpu.stamps).copy(), to_np(gpu.next_row).copy())
    rows, hit, st = gpu.step(ids, steps + 1, insert=False)
    orows, ohit, ost = ora.step(ids, steps + 1, insert=False)
    assert np.array_equal(rows, orows) and np.array_equal(hit, ohit) and np.array_equal(st, ost)
    assert all(np.array_equal(a, b) for a, b in zip(before, (to_np(gpu.keys), to_np(gpu.stamps),
                                                            to_np(gpu.next_row))))


def test_key_store_overflow(dev):
    """The value store fills up mid-batch: later new keys overflow (row -1, not stored)."""
    g = np.random.default_rng(9)
    dim, max_rows = 16, 500
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
    assert bits_equal(to_np(gpu.values), ora.values)


def test_rehash_keeps_the_map(dev):
    g = np.random.default_rng(10)
    gpu = GpuStore(dev, 1 << 12, 1500, 4, np.zeros((1500, 4), np.float32))
    gpu.step(g.integers(0, 1 << 50, size=1500).astype(np.int64), 1)
    m = gpu.mapping()
    for cap in (1 << 12, 1 << 13, 1 << 16):
        k, r = hlr.dks_rehash(gpu.keys, gpu.krows, cap)
        kk, rr = to_np(k), to_np(r)
        sel = kk >= 0
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
    values = torch.zeros((max_rows, dim), dtype=torch.float32, device=dev)
    store = DynamicKeyStore(values, max_rows, key_cap=1024, stream=torch.cuda.Stream(dev) if side else None)
    ora = oracle.KeyStore(1 << 18, max_rows, dim)
    batches = [zipf_keys(g, n, 1.1, 500_000) for _ in range(15)]
    dev_b = [torch.from_numpy(b).to(dev) for b in batches]
    outs = [torch.empty(n, dtype=torch.int64, device=dev) for _ in batches]
    torch.cuda.synchronize()
    for t, b in enumerate(dev_b):
        store.step(b, t + 1, out_rows=outs[t])
    for t, b in enumerate(batches):
        orows, _, _ = ora.step(b, t + 1)
        assert np.array_equal(to_np(outs[t]), orows), t
    assert store.rehashes >= 3
    k, r = to_np(store.keys), to_np(store.krows)
    assert dict(zip(k[k >= 0].tolist(), r[k >= 0].tolist())) == ora.mapping()
    assert (k >= 0).sum() <= store.keys.numel() // 2
