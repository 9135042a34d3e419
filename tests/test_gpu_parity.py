"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Sizes here span several tiles plus a ragged tail and finish in seconds on the
oracle.  Bit-exact: MPZCH rows / hit / evicted / stats / identity / stamps,
gathered rows, dedup outputs, Writeback and SGD-sum rows, EMA rows.  Scores:
|gpu - oracle| <= 1e-6 * |oracle| + 1e-12 * sum_d |x_d * u_d| (1e-6 relative,
with a floor far below one fp32 ulp of the terms for scores that cancel; both
sides sum in fp64 and round once).
"""
import numpy as np
import pytest
import torch

import hashed_lookup_row_amd as hlr
import oracle
import synth

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
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    return a.shape == b.shape and a.tobytes() == b.tobytes()


class GpuCache:
    def __init__(self, dev, capacity, probes, dim):
        self.identity = torch.full((capacity,), -1, dtype=torch.int64, device=dev)
        self.stamps = torch.full((capacity,), -1, dtype=torch.int64, device=dev)
        self.values = torch.zeros((capacity, dim), dtype=torch.float32, device=dev)
        self.probes = probes

    def step(self, ids, now, insert=True, values=True):
        n = ids.numel()
        ev = torch.empty(n, dtype=torch.int64, device=ids.device)
        st = torch.zeros(6, dtype=torch.int64, device=ids.device)
        rows, hit, ev, st = hlr.mpzch_lookup_or_insert(self.identity, self.stamps, self.values if values else None,
                                                       self.probes, ids, now, insert=insert, out_evicted=ev,
                                                       out_stats=st)
        return rows, hit, ev, st


def run_mpzch_pair(dev, cfg, streams, check_every=1, e_std=1.0, seed_cfg=1):
    """Runs lookup+gather+writeback on GPU and oracle; compares everything bit-exactly."""
    C, P, D = cfg
    g = GpuCache(dev, C, P, D)
    o = oracle.MPZCHTable(C, P, D)
    for t, ids_np in enumerate(streams, start=1):
        e_np = synth.normal_rows_np(ids_np.size, D, e_std, seed_cfg, t)
        ids = torch.from_numpy(ids_np).to(dev)
        e = torch.from_numpy(e_np).to(dev)
        rows, hit, ev, st = g.step(ids, t)
        out = hlr.gather_rows(g.values, rows)
        hlr.writeback_rows(g.values, rows, e)
        orows, ohit, oev, ost = o.step(ids_np, t)
        oout = o.gather(orows)
        o.writeback(orows, e_np)
        if t % check_every == 0 or t == len(streams):
            assert np.array_equal(to_np(rows), orows), f"rows step {t}"
            assert np.array_equal(to_np(hit), ohit), f"hit step {t}"
            assert np.array_equal(to_np(ev), oev), f"evicted step {t}"
            s = to_np(st)
            assert np.array_equal(s[:5], ost) and s[5] == 0, (t, s, ost)
            assert np.array_equal(to_np(g.identity), o.identity), f"identity step {t}"
            assert np.array_equal(to_np(g.stamps), o.stamps), f"stamps step {t}"
            assert bits_equal(to_np(out), oout), f"gather step {t}"
            assert bits_equal(to_np(g.values), o.values), f"values step {t}"
    return g, o


def test_tiny_config_full_state_every_step(dev):
    cfg = synth.TINY
    streams = synth.mpzch_stream(cfg, cfg.steps)
    run_mpzch_pair(dev, (cfg.capacity, cfg.probes, cfg.dim), streams, e_std=cfg.e_std)


def test_scaled_memory_layer_with_prefill(dev):
    cfg = synth.scaled_memory_layer(capacity=32_768, universe=200_000, batch=8_192, steps=4)
    C, P, D = cfg.capacity, cfg.probes, cfg.dim
    g = GpuCache(dev, C, P, D)
    o = oracle.MPZCHTable(C, P, D, with_values=False)
    # prefill without values (all slots end up inserted), then both tables start at zero
    for k, batch in enumerate(synth.prefill_batches(cfg), start=1):
        ids = torch.from_numpy(batch).to(dev)
        g.step(ids, k, values=False)
        o.step(batch, k)
    assert np.array_equal(to_np(g.identity), o.identity)
    assert np.array_equal(to_np(g.stamps), o.stamps)
    o.values = np.zeros((C, D), np.float32)
    base = len(synth.prefill_batches(cfg))
    for t, ids_np in enumerate(synth.mpzch_stream(cfg, cfg.steps), start=1):
        now = base + t
        e_np = synth.normal_rows_np(ids_np.size, D, cfg.e_std, 2, t)
        ids = torch.from_numpy(ids_np).to(dev)
        rows, hit, ev, st = g.step(ids, now)
        out = hlr.gather_rows(g.values, rows)
        hlr.writeback_rows(g.values, rows, torch.from_numpy(e_np).to(dev))
        orows, ohit, oev, ost = o.step(ids_np, now)
        oout = o.gather(orows)
        o.writeback(orows, e_np)
        assert np.array_equal(to_np(rows), orows)
        assert np.array_equal(to_np(hit), ohit)
        assert np.array_equal(to_np(ev), oev)
        assert np.array_equal(to_np(st)[:5], ost)
        assert bits_equal(to_np(out), oout)
    assert np.array_equal(to_np(g.identity), o.identity)
    assert np.array_equal(to_np(g.stamps), o.stamps)
    assert bits_equal(to_np(g.values), o.values)


@pytest.mark.parametrize("C,P", [(64, 8), (96, 4), (600, 12), (4096, 16), (8, 8), (7 * 8, 8)])
def test_mpzch_other_geometries(dev, C, P):
    g = np.random.default_rng(C + P)
    streams = []
    for t in range(12):
        n = int(g.integers(1, 700))
        ids = g.integers(0, 3 * C, size=n).astype(np.int64)
        ids[g.random(n) < 0.02] = -1
        streams.append(ids)
    run_mpzch_pair(dev, (C, P, 8), streams)


def _ids_in_bucket(target, nb, count, start=1):
    out, x = [], start
    while len(out) < count:
        if oracle.bucket(x, nb) == target:
            out.append(x)
        x += 1
    return out


def test_mpzch_crafted_overflow_ties_and_pins(dev):
    C, P = 64, 8
    nb = C // P
    ids = _ids_in_bucket(3, nb, 30)
    g = GpuCache(dev, C, P, 4)
    o = oracle.MPZCHTable(C, P, 4)

    def both(batch, now, stamps=None):
        if stamps is not None:
            g.stamps[3 * P:3 * P + 8] = torch.tensor(stamps, dtype=torch.int64, device=dev)
            o.stamps[3 * P:3 * P + 8] = stamps
        b = np.array(batch, np.int64)
        r = g.step(torch.from_numpy(b).to(dev), now)
        orr = o.step(b, now)
        for x, y in zip(r[:3], orr[:3]):
            assert np.array_equal(to_np(x), y)
        assert np.array_equal(to_np(r[3])[:5], orr[3])
        assert np.array_equal(to_np(g.identity), o.identity)
        assert np.array_equal(to_np(g.stamps), o.stamps)

    both(ids[:13][::-1] + [ids[12], ids[0]], 10)             # 13 new IDs -> 8 inserted, 5 overflow
    both([ids[20], ids[21], ids[22]], 100, [50, 20, 20, 40, 30, 60, 70, 80])   # stamp ties
    hot = int(o.identity[3 * P])
    both([ids[23], hot, ids[24]], 200, [5, 6, 7, 8, 9, 10, 11, 12])          # pinned hit never evicted
    both([-1, ids[25], -1], 300)                                              # invalid IDs counted


def test_mpzch_lookup_only_changes_nothing(dev):
    C, P, D = 4096, 8, 16
    g = GpuCache(dev, C, P, D)
    o = oracle.MPZCHTable(C, P, D)
    first = np.arange(1, 3000, dtype=np.int64) * 7919
    g.step(torch.from_numpy(first).to(dev), 1)
    o.step(first, 1)
    ident, stamps = to_np(g.identity).copy(), to_np(g.stamps).copy()
    q = np.concatenate([first[::3], np.arange(10 ** 9, 10 ** 9 + 500, dtype=np.int64), [-1, -1]])
    rows, hit, ev, st = g.step(torch.from_numpy(q).to(dev), 2, insert=False)
    orows, ohit, oev, ost = o.step(q, 2, insert=False)
    assert np.array_equal(to_np(rows), orows) and np.array_equal(to_np(hit), ohit)
    assert np.array_equal(to_np(st)[:5], ost)
    assert np.array_equal(to_np(g.identity), ident) and np.array_equal(to_np(g.stamps), stamps)


@pytest.mark.parametrize("n,D", [(0, 64), (1, 4), (1023, 64), (5000, 100), (4097, 128), (3001, 512)])
def test_gather_ragged(dev, n, D):
    g = np.random.default_rng(n + D)
    C = 777
    table = g.standard_normal((C, D)).astype(np.float32)
    rows = g.integers(-1, C, size=n).astype(np.int64)
    out = hlr.gather_rows(torch.from_numpy(table).to(dev), torch.from_numpy(rows).to(dev))
    assert bits_equal(to_np(out), oracle.gather(table, rows))


@pytest.mark.parametrize("n", [1, 2, 4095, 4096, 4097, 8191, 8192, 8193, 16_385, 20_000, 70_001, 262_145])
def test_dedup_matches_oracle(dev, n):
    g = np.random.default_rng(n)
    pool = np.concatenate([g.integers(-(1 << 62), 1 << 62, size=max(1, n // 3)), [0, -1, 1, -(1 << 63), (1 << 63) - 1]])
    keys = pool[g.integers(0, pool.size, size=n)].astype(np.int64)
    uq, lp, inv, nu = hlr.dedup_ids(torch.from_numpy(keys).to(dev))
    u = int(to_np(nu)[0])
    ouq, olp, oinv = oracle.dedup(keys)
    assert u == ouq.size
    assert np.array_equal(to_np(uq)[:u], ouq)
    assert np.array_equal(to_np(lp)[:u], olp)
    assert np.array_equal(to_np(inv), oinv)


@pytest.mark.parametrize("n,distinct", [(30_000, 1), (30_000, 2), (50_000, 7)])
def test_dedup_few_keys(dev, n, distinct):
    """Long runs of equal keys: the sort orders them by position alone, across tiles and merge rounds."""
    g = np.random.default_rng(n + distinct)
    pool = g.integers(-(1 << 62), 1 << 62, size=distinct)
    keys = pool[g.integers(0, distinct, size=n)].astype(np.int64)
    uq, lp, inv, nu = hlr.dedup_ids(torch.from_numpy(keys).to(dev))
    u = int(to_np(nu)[0])
    ouq, olp, oinv = oracle.dedup(keys)
    assert u == ouq.size
    assert np.array_equal(to_np(uq)[:u], ouq) and np.array_equal(to_np(lp)[:u], olp)
    assert np.array_equal(to_np(inv), oinv)


def test_dedup_empty(dev):
    uq, lp, inv, nu = hlr.dedup_ids(torch.empty(0, dtype=torch.int64, device=dev))
    assert int(to_np(nu)[0]) == 0


@pytest.mark.parametrize("n,C,D", [(5000, 300, 64), (65_536, 40_000, 512), (9000, 5, 8)])
def test_writeback_last_wins(dev, n, C, D):
    g = np.random.default_rng(n + C)
    table = (g.standard_normal((C, D)) * g.choice([1e-3, 1.0, 1e4], size=(C, 1))).astype(np.float32)
    table[: C // 4] = 0.0
    rows = g.integers(-1, C, size=n).astype(np.int64)
    e = g.standard_normal((n, D)).astype(np.float32)
    t = torch.from_numpy(table).to(dev)
    hlr.writeback_rows(t, torch.from_numpy(rows).to(dev), torch.from_numpy(e).to(dev))
    oracle.writeback_last(table, rows, e)
    assert bits_equal(to_np(t), table)


def _zipf_rows(g, n, C, s):
    return np.minimum(synth.zipf_ranks(g, C, s, n), C - 1).astype(np.int64)


@pytest.mark.parametrize("n,C,D,s", [(20_000, 3000, 512, 1.2), (3000, 2, 64, 1.0), (131_072, 60_000, 128, 1.2),
                                     (777, 50, 4, 1.1)])
def test_sgd_sum_matches_oracle(dev, n, C, D, s):
    g = np.random.default_rng(n + D)
    table = (g.standard_normal((C, D)) * 0.01).astype(np.float32)
    rows = _zipf_rows(g, n, C, s)
    rows[g.random(n) < 0.01] = -1
    grads = (g.standard_normal((n, D)) * 1e-3).astype(np.float32)
    t = torch.from_numpy(table).to(dev)
    hlr.writeback_rows(t, torch.from_numpy(rows).to(dev), torch.from_numpy(grads).to(dev), mode=hlr.WB_SGD_SUM,
                       lr=0.01)
    oracle.sgd_sum(table, rows, grads, 0.01)
    assert bits_equal(to_np(t), table)
    assert np.bincount(rows[rows >= 0]).max() >= 64 or n < 5000  # a heavy (chained) row is exercised


@pytest.mark.parametrize("n,C,D,s,lr", [(20_000, 3000, 512, 1.2, 0.05), (3000, 2, 64, 1.0, 0.5),
                                        (65_536, 30_000, 512, 1.05, 0.01), (777, 50, 4, 1.1, 0.25),
                                        (30_000, 12, 128, 2.0, 0.001)])
def test_l2_align_matches_oracle(dev, n, C, D, s, lr):
    """Writeback's L2 alternative: per-occurrence gradient 2 (M - e_i) at the pre-batch row, summed per row."""
    g = np.random.default_rng(n + D + 1)
    table = g.standard_normal((C, D)).astype(np.float32)
    rows = _zipf_rows(g, n, C, s)
    rows[g.random(n) < 0.01] = -1
    e = g.standard_normal((n, D)).astype(np.float32)
    t = torch.from_numpy(table).to(dev)
    hlr.writeback_rows(t, torch.from_numpy(rows).to(dev), torch.from_numpy(e).to(dev), mode=hlr.WB_L2_ALIGN, lr=lr)
    oracle.l2_align(table, rows, e, lr)
    assert bits_equal(to_np(t), table)


@pytest.mark.parametrize("n,C,D,masked,a,b", [(20_000, 3000, 128, True, 0.99, 0.01),
                                              (50_000, 1000, 128, False, 0.95, 0.05),
                                              (4097, 7, 4, False, 0.5, 0.5), (3000, 100, 512, True, 0.9, 0.1)])
def test_ema_matches_oracle(dev, n, C, D, masked, a, b):
    g = np.random.default_rng(n + C)
    table = g.standard_normal((C, D)).astype(np.float32)
    rows = _zipf_rows(g, n, C, 1.1)
    rows[g.random(n) < 0.01] = -1
    vals = g.standard_normal((n, D)).astype(np.float32)
    mask = (g.random(n) < 0.3).astype(np.uint8) if masked else None
    t = torch.from_numpy(table).to(dev)
    hlr.ema_update_rows(t, torch.from_numpy(rows).to(dev), torch.from_numpy(vals).to(dev),
                        None if mask is None else torch.from_numpy(mask).to(dev), a, b)
    oracle.ema(table, rows, vals, mask, a, b)
    assert bits_equal(to_np(t), table)


def score_close(got, ref, cond):
    """1e-6 relative, with an absolute floor of 1e-12 of the condition scale sum_d |x_d u_d|."""
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    return bool(np.all(err <= 1e-6 * np.abs(ref.astype(np.float64)) + 1e-12 * cond))


@pytest.mark.parametrize("R,K,D", [(3, 1000, 512), (4, 70, 256), (2, 33, 48), (2, 2500, 512), (3, 600, 256),
                                   (1, 512, 512)])
def test_dequant_score(dev, R, K, D):
    """Requests of 33 to 2,500 candidates (ragged last blocks of a request), dims with and without
    the register-resident user slice."""
    g = np.random.default_rng(R * K + D)
    C = 5000
    q = np.clip(np.rint(g.standard_normal((C, D)) * 42), -128, 127).astype(np.int8)
    scale = (g.random(C).astype(np.float32) * 0.004 + 0.001).astype(np.float32)
    bias = (g.standard_normal(C) * 0.005).astype(np.float32)
    rows = g.integers(-1, C, size=R * K).astype(np.int64)
    user = g.standard_normal((R, D)).astype(np.float32)
    out = hlr.gather_dequant_score(*(torch.from_numpy(x).to(dev) for x in (q, scale, bias, rows, user)), K)
    ref = oracle.dequant_score(q, scale, bias, rows, user, K)
    got = to_np(out)
    x = q.astype(np.float64) * scale[:, None] + bias[:, None]
    cond = np.einsum("rkd,rd->rk", np.abs(x[np.maximum(rows, 0)].reshape(R, K, D)), np.abs(user.astype(np.float64)))
    assert score_close(got, ref, cond)
    assert np.all(got[rows.reshape(R, K) < 0] == 0.0)


@pytest.mark.parametrize("D", [512, 256])
def test_dequant_score_repeated_rows(dev, D):
    """Candidates that repeat rows within a request: one request of a single row 1,500 times, one of a
    few rows with misses and out-of-range rows among them, one Zipf-skewed; scores equal the oracle's as
    in test_dequant_score, and every copy of a row in a request has the same score bit for bit (a
    candidate's score does not depend on the lane or block that computes it)."""
    g = np.random.default_rng(D + 11)
    C, R, K = 3000, 3, 1500
    q = np.clip(np.rint(g.standard_normal((C, D)) * 42), -128, 127).astype(np.int8)
    scale = (g.random(C).astype(np.float32) * 0.004 + 0.001).astype(np.float32)
    bias = (g.standard_normal(C) * 0.005).astype(np.float32)
    rows = np.empty((R, K), np.int64)
    rows[0] = 17
    rows[1] = g.choice(np.array([0, 5, C - 1, -1, C, -7]), K)
    rows[2] = np.minimum(g.zipf(1.3, K) - 1, C - 1)
    rows = rows.reshape(-1)
    user = g.standard_normal((R, D)).astype(np.float32)
    out = hlr.gather_dequant_score(*(torch.from_numpy(x).to(dev) for x in (q, scale, bias, rows, user)), K)
    valid = np.where((rows >= 0) & (rows < C), rows, -1)
    ref = oracle.dequant_score(q, scale, bias, valid, user, K)
    x = q.astype(np.float64) * scale[:, None] + bias[:, None]
    cond = np.einsum("rkd,rd->rk", np.abs(x[np.maximum(valid, 0)].reshape(R, K, D)), np.abs(user.astype(np.float64)))
    got = to_np(out)
    assert score_close(got, ref, cond)
    assert np.all(got.reshape(-1)[valid < 0] == 0.0)
    for r in range(R):
        rr, gg = rows.reshape(R, K)[r], got.reshape(R, K)[r]
        for v in np.unique(rr):
            assert np.unique(gg[rr == v].view(np.uint32)).size == 1


@pytest.mark.parametrize("P,D", [(8, 512), (8, 256), (4, 48), (8, 48), (16, 512)])
def test_mpzch_score_matches_lookup_then_score(dev, P, D):
    """mpzch_score (lookup-only MPZCH and the int8 dequant-score in one launch): rows and hit mask equal
    the oracle's lookup-only MPZCH (stored IDs, fresh IDs, invalid IDs), and the scores the oracle's
    dequant-score of those rows (1e-6 relative, absolute floor 1e-12 of sum |x u|); the identity tensor
    is not changed."""
    g = np.random.default_rng(P * 1000 + D)
    C = 4096
    ids_all = g.integers(0, 1 << 40, size=6000).astype(np.int64)
    identity = torch.full((C,), -1, dtype=torch.int64, device=dev)
    stamps = torch.full((C,), -1, dtype=torch.int64, device=dev)
    tab = oracle.MPZCHTable(C, P, 4, with_values=False)
    for k in range(3):
        b = ids_all[k * 2000:(k + 1) * 2000]
        hlr.mpzch_lookup_or_insert(identity, stamps, None, P, torch.from_numpy(b).to(dev), k + 1)
        tab.step(b, k + 1, zero_fill=False)
    R, K = (3, 700) if D != 512 else (2, 1300)
    cands = np.where(g.random(R * K) < 0.8, g.choice(ids_all, R * K), g.integers(1 << 41, 1 << 42, R * K))
    cands[::97] = -1  # invalid IDs
    cands[5::7] = ids_all[3]  # a stored ID named many times by every request
    cands[6::11] = 1 << 43  # a fresh ID named many times
    cands = cands.astype(np.int64)
    q = np.clip(np.rint(g.standard_normal((C, D)) * 42), -128, 127).astype(np.int8)
    scale = (g.random(C).astype(np.float32) * 0.004 + 0.001).astype(np.float32)
    bias = (g.standard_normal(C) * 0.005).astype(np.float32)
    user = g.standard_normal((R, D)).astype(np.float32)
    ident_before = to_np(identity).copy()
    rows_out = torch.empty(R * K, dtype=torch.int64, device=dev)
    hit_out = torch.empty(R * K, dtype=torch.int8, device=dev)
    out = hlr.mpzch_score(identity, P, torch.from_numpy(cands).to(dev),
                          *(torch.from_numpy(x).to(dev) for x in (q, scale, bias, user)), K,
                          out_rows=rows_out, out_hit=hit_out)
    orows, ohit, _, _ = tab.step(cands, 0, insert=False)
    assert np.array_equal(to_np(rows_out), orows) and np.array_equal(to_np(hit_out), ohit)
    assert 0 < ohit.mean() < 1
    assert np.array_equal(to_np(identity), ident_before)
    ref = oracle.dequant_score(q, scale, bias, orows, user, K)
    x = q.astype(np.float64) * scale[:, None] + bias[:, None]
    cond = np.einsum("rkd,rd->rk", np.abs(x[np.maximum(orows, 0)].reshape(R, K, D)), np.abs(user.astype(np.float64)))
    got = to_np(out)
    assert score_close(got, ref, cond)
    assert np.all(got[orows.reshape(R, K) < 0] == 0.0)


def test_dequant_score_edge_cases(dev):
    """An empty table scores every candidate 0; a ragged last block of candidates (K % 64 != 0)
    and rows at both ends of the table match the oracle."""
    R, K, D = 2, 5, 256
    user = torch.ones((R, D), dtype=torch.float32, device=dev)
    rows = torch.full((R * K,), -1, dtype=torch.int64, device=dev)
    empty_q = torch.empty((0, D), dtype=torch.int8, device=dev)
    empty_f = torch.empty(0, dtype=torch.float32, device=dev)
    out = hlr.gather_dequant_score(empty_q, empty_f, empty_f, rows, user, K)
    assert np.array_equal(to_np(out), np.zeros(R * K, np.float32).reshape(out.shape))
    g = np.random.default_rng(77)
    C, K = 130, 129
    q = g.integers(-128, 128, size=(C, D)).astype(np.int8)
    scale = (g.random(C) * 0.01 + 1e-4).astype(np.float32)
    bias = (g.standard_normal(C) * 0.1).astype(np.float32)
    rows = g.integers(0, C, size=R * K).astype(np.int64)
    rows[:4] = [0, C - 1, C, -5]
    user = g.standard_normal((R, D)).astype(np.float32)
    out = hlr.gather_dequant_score(*(torch.from_numpy(x).to(dev) for x in (q, scale, bias, rows, user)), K)
    ref = oracle.dequant_score(q, scale, bias, np.where((rows >= 0) & (rows < C), rows, -1), user, K)
    x = q.astype(np.float64) * scale[:, None] + bias[:, None]
    cond = np.einsum("rkd,rd->rk", np.abs(x[np.clip(rows, 0, C - 1)].reshape(R, K, D)),
                     np.abs(user.astype(np.float64)))
    got = to_np(out)
    assert score_close(got, ref, cond)
    assert got.reshape(-1)[2] == 0.0 and got.reshape(-1)[3] == 0.0


def test_hashed_rows(dev):
    ids = np.concatenate([np.arange(-50, 50), synth.dlrm_keys(synth.DLRM, 1, 1)[:5000]]).astype(np.int64)
    for nr in [1, 7, 4 * synth.MI, 24 * synth.MI]:
        out = hlr.hashed_rows(torch.from_numpy(ids).to(dev), nr)
        assert np.array_equal(to_np(out), oracle.hashed_rows(ids, nr))


def test_repeat_runs_are_bit_identical(dev):
    g = np.random.default_rng(0)
    n, C, D = 30_000, 2000, 128
    rows = torch.from_numpy(_zipf_rows(g, n, C, 1.2)).to(dev)
    vals = torch.from_numpy(g.standard_normal((n, D)).astype(np.float32)).to(dev)
    t0 = torch.from_numpy(g.standard_normal((C, D)).astype(np.float32)).to(dev)
    outs = []
    for _ in range(2):
        t = t0.clone()
        hlr.writeback_rows(t, rows, vals, mode=hlr.WB_SGD_SUM, lr=0.01)
        hlr.ema_update_rows(t, rows, vals, None, 0.95, 0.05)
        hlr.writeback_rows(t, rows, vals)
        outs.append(to_np(t))
    assert bits_equal(outs[0], outs[1])


@pytest.mark.parametrize("a,b", [(0.95, 0.05), (0.99, 0.01), (0.9, 0.1)])
def test_ema_long_row_many_chunks(dev, a, b):
    """One row with 36,000 occurrences and one with 4,000: many speculative chunks (warm-up
    ceil(28 / -ln a), chunks of twice that), bit-exact."""
    g = np.random.default_rng(40)
    n, D = 40_000, 128
    rows = np.zeros(n, np.int64)
    rows[g.random(n) < 0.1] = 1
    vals = g.standard_normal((n, D)).astype(np.float32)
    table = g.standard_normal((2, D)).astype(np.float32)
    t = torch.from_numpy(table).to(dev)
    hlr.ema_update_rows(t, torch.from_numpy(rows).to(dev), torch.from_numpy(vals).to(dev), None, a, b)
    oracle.ema(table, rows, vals, None, a, b)
    assert bits_equal(to_np(t), table)


@pytest.mark.parametrize("spike_at", [900, 1990, 3000])
def test_ema_speculation_fallback_is_exact(dev, spike_at):
    """Huge values just before a chunk's warm-up window make its speculative start wrong; the
    chunk must be recomputed from the exact state (a = 0.5: warm-up 41, chunks of 256)."""
    g = np.random.default_rng(spike_at)
    n, D = 4500, 8
    rows = np.zeros(n, np.int64)
    vals = g.standard_normal((n, D)).astype(np.float32)
    vals[spike_at:spike_at + 60] = 1e30
    table = np.zeros((1, D), np.float32)
    t = torch.from_numpy(table).to(dev)
    hlr.ema_update_rows(t, torch.from_numpy(rows).to(dev), torch.from_numpy(vals).to(dev), None, 0.5, 0.5)
    oracle.ema(table, rows, vals, None, 0.5, 0.5)
    assert bits_equal(to_np(t), table)


def test_sgd_sum_single_row_long_chain(dev):
    """One row with about 24,000 duplicate gradients: one running sum per element, in batch order."""
    g = np.random.default_rng(30)
    n, D = 30_000, 512
    rows = np.where(g.random(n) < 0.8, 7, g.integers(0, 10, size=n)).astype(np.int64)
    grads = (g.standard_normal((n, D)) * 1e-3).astype(np.float32)
    table = (g.standard_normal((10, D)) * 0.01).astype(np.float32)
    t = torch.from_numpy(table).to(dev)
    hlr.writeback_rows(t, torch.from_numpy(rows).to(dev), torch.from_numpy(grads).to(dev), mode=hlr.WB_SGD_SUM,
                       lr=0.01)
    oracle.sgd_sum(table, rows, grads, 0.01)
    assert bits_equal(to_np(t), table)


def test_sgd_sum_plan_applied_twice(dev):
    """One SGD_SUM plan applied twice (the heavy rows' work items are drawn from a counter in the plan,
    which the last heavy block returns to zero): the table equals two sequential oracle updates."""
    g = np.random.default_rng(31)
    n, D, C = 40_000, 64, 300
    rows = np.where(g.random(n) < 0.5, g.integers(0, 4, size=n), g.integers(0, C, size=n)).astype(np.int64)
    grads = (g.standard_normal((n, D)) * 1e-3).astype(np.float32)
    table = (g.standard_normal((C, D)) * 0.01).astype(np.float32)
    t = torch.from_numpy(table).to(dev)
    r, gr = torch.from_numpy(rows).to(dev), torch.from_numpy(grads).to(dev)
    ws = hlr.new_workspace(dev, hlr.writeback_workspace_size(C, D, n, hlr.WB_SGD_SUM))
    hlr.writeback_plan(C, r, ws, hlr.WB_SGD_SUM)
    hlr.writeback_apply(t, gr, ws, hlr.WB_SGD_SUM, 0.01)
    hlr.writeback_apply(t, gr, ws, hlr.WB_SGD_SUM, 0.01)
    oracle.sgd_sum(table, rows, grads, 0.01)
    oracle.sgd_sum(table, rows, grads, 0.01)
    assert bits_equal(to_np(t), table)


@pytest.mark.parametrize("k", [63, 64, 65, 511, 512, 513, 1000, 4097, 20_000])
@pytest.mark.parametrize("D", [4, 12, 512])
def test_sgd_sum_order_revealing_rows(dev, k, D):
    """Row 0's gradients in batch order are 1, then k - 1 copies of 2^-24 (negated in odd elements):
    summed left to right each tiny term rounds away (ties to even) and the row moves by exactly lr;
    any other order (tiny terms first, a split into partial sums, a permuted group of lanes) gives a
    different fp32 result.  Row 1 interleaves random gradients; rows of k - 1, k and k + 1
    occurrences cover the threshold between one wave per row and the per-element chains (512)."""
    g = np.random.default_rng(k * 7 + D)
    rows = np.concatenate([np.zeros(k, np.int64), np.ones(3 * k, np.int64), np.full(k - 1, 2), np.full(k + 1, 3)])
    perm = np.sort(g.permutation(rows.size)[:k])  # row 0 at increasing positions, spread over the batch
    rest = np.setdiff1d(np.arange(rows.size), perm)
    order = np.empty(rows.size, np.int64)
    order[perm] = 0
    order[rest] = rows[k:]
    rows = order
    grads = (g.standard_normal((rows.size, D)) * 1e-3).astype(np.float32)
    sign = np.where(np.arange(D) % 2 == 0, np.float32(1.0), np.float32(-1.0))
    p0 = np.nonzero(rows == 0)[0]
    grads[p0] = sign * np.float32(2.0 ** -24)
    grads[p0[0]] = sign
    table = np.zeros((4, D), np.float32)
    t = torch.from_numpy(table).to(dev)
    hlr.writeback_rows(t, torch.from_numpy(rows).to(dev), torch.from_numpy(grads).to(dev), mode=hlr.WB_SGD_SUM,
                       lr=1.0)
    oracle.sgd_sum(table, rows, grads, 1.0)
    assert np.array_equal(table[0], -sign)  # the oracle itself: left to right, the tiny terms vanish
    assert bits_equal(to_np(t), table)


def test_sgd_sum_gradients_over_2gib(dev):
    """Gradient array of 2 GiB (byte offsets past the 31-bit buffer range): 64-bit addressing path."""
    g = np.random.default_rng(31)
    n, D = 1 << 19, 1024
    rows = np.minimum(synth.zipf_ranks(g, 40, 1.3, n), 39).astype(np.int64)
    grads = np.empty((n, D), np.float32)
    grads[:] = (g.standard_normal((1, D)) * 1e-3).astype(np.float32)
    grads[:, ::7] = (g.standard_normal((n, 1)) * 1e-3).astype(np.float32)
    table = (g.standard_normal((40, D)) * 0.01).astype(np.float32)
    t = torch.from_numpy(table).to(dev)
    gd = torch.from_numpy(grads).to(dev)
    hlr.writeback_rows(t, torch.from_numpy(rows).to(dev), gd, mode=hlr.WB_SGD_SUM, lr=0.01)
    del gd
    oracle.sgd_sum(table, rows, grads, 0.01)
    assert bits_equal(to_np(t), table)
