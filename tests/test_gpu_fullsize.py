"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

  * Memory-Layer cache: 4,194,304 x 512 fp32, 8 probes, prefilled with a 20M-ID
    universe, then 65,536-ID steps (Zipf 1.05 + 0.5% fresh): rows, hit,
    evicted, stats every step; identity and stamps in full; every touched row
    bit for bit and the count of non-zero rows (no stray writes); the same in
    the benchmark's configuration (one call per half batch, two streams,
    lookahead, ring depth 3), every batch's gathered rows bit for bit.
  * Serving read path: that prefilled identity, an int8 4Mi x 512 table,
    256 requests x 1024 candidates: lookup-only rows/hit bit-exact, scores
    within 1e-6 of sum_d |x_d u_d|.
  * DLRMv4-like: 8 hashed tables (120 GiB), 131,072 keys per table, gather
    and duplicate-summed SGD (lr 0.01): hashed rows and every gathered row
    bit-exact; every touched row bit-exact; sampled untouched rows unchanged.
  * CS3 EMA: 1Mi/2Mi x 128 tables, 262,144 pairs, CTS on positives and CMS on
    all pairs, two steps: every row bit-exact.
The oracle works on compact copies of the touched rows where a table does not
fit in host memory (DLRM) — that is plumbing, not arithmetic.
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
    return a.shape == b.shape and np.ascontiguousarray(a).tobytes() == np.ascontiguousarray(b).tobytes()


def free(*ts):
    for t in ts:
        del t
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def prefilled(dev):
    """Memory-Layer table after the untimed coldest-first prefill, on both sides."""
    cfg = synth.MEMORY_LAYER
    C, P, D = cfg.capacity, cfg.probes, cfg.dim
    identity = torch.full((C,), -1, dtype=torch.int64, device=dev)
    stamps = torch.full((C,), -1, dtype=torch.int64, device=dev)
    tab = oracle.MPZCHTable(C, P, D, with_values=False)
    batches = synth.prefill_batches(cfg)
    for k, b in enumerate(batches, start=1):
        hlr.mpzch_lookup_or_insert(identity, stamps, None, P, torch.from_numpy(b).to(dev), k)
        tab.step(b, k, zero_fill=False)
    print(f"prefilled {len(batches)} batches", flush=True)
    assert np.array_equal(to_np(identity), tab.identity)
    assert np.array_equal(to_np(stamps), tab.stamps)
    return cfg, identity, stamps, tab, len(batches)


def test_memory_layer_full_size(dev, prefilled):
    cfg, identity0, stamps0, tab0, base = prefilled
    C, P, D, n = cfg.capacity, cfg.probes, cfg.dim, cfg.batch
    identity, stamps = identity0.clone(), stamps0.clone()
    values = torch.zeros((C, D), dtype=torch.float32, device=dev)
    tab = oracle.MPZCHTable(C, P, D, with_values=False)
    tab.identity, tab.stamps = tab0.identity.copy(), tab0.stamps.copy()
    tab.values = np.zeros((C, D), np.float32)
    stats = torch.zeros(6, dtype=torch.int64, device=dev)
    ev = torch.empty(n, dtype=torch.int64, device=dev)
    touched = set()
    fc = 0
    for t in range(1, 4):
        ids_np, fc = synth.mpzch_step_ids(cfg, t, fc)
        e = synth.normal_rows(n, D, cfg.e_std, cfg.config, t, device=dev)
        e_np = to_np(e)
        rows, hit, _, _ = hlr.mpzch_lookup_or_insert(identity, stamps, values, P, torch.from_numpy(ids_np).to(dev),
                                                     base + t, out_evicted=ev, out_stats=stats)
        out = hlr.gather_rows(values, rows)
        hlr.writeback_rows(values, rows, e)
        orows, ohit, oev, ost = tab.step(ids_np, base + t)
        oout = tab.gather(orows)
        tab.writeback(orows, e_np)
        assert np.array_equal(to_np(rows), orows), f"rows step {t}"
        assert np.array_equal(to_np(hit), ohit), f"hit step {t}"
        assert np.array_equal(to_np(ev), oev), f"evicted step {t}"
        s = to_np(stats)
        assert np.array_equal(s[:5], ost) and s[5] == 0, (s, ost)
        assert bits_equal(to_np(out), oout), f"gather step {t}"
        touched.update(np.unique(orows[orows >= 0]).tolist())
        print(f"step {t}: hits {ost[0]} inserts {ost[1]} evictions {ost[2]} overflows {ost[3]}", flush=True)
    assert np.array_equal(to_np(identity), tab.identity)
    assert np.array_equal(to_np(stamps), tab.stamps)
    idx = np.array(sorted(touched), dtype=np.int64)
    got = to_np(values[torch.from_numpy(idx).to(dev)])
    assert bits_equal(got, tab.values[idx])
    nonzero_gpu = int((values != 0).any(dim=1).sum().item())
    assert nonzero_gpu == int(np.count_nonzero(tab.values[idx].any(axis=1)))
    free(values, identity, stamps)


def test_memory_layer_full_size_one_call_lookahead(dev, prefilled):
    """The headline's launch configuration: memory_layer_step through MemoryLayerPipeline, two streams,
    ring depth 3, batch t+1's lookup enqueued before batch t's row traffic, no synchronisation between
    batches.  Every batch's gathered rows and stats, the ID table and every touched row bit-exact."""
    from hashed_lookup_row_amd.pipeline import MemoryLayerPipeline
    cfg, identity0, stamps0, tab0, base = prefilled
    C, P, D, n = cfg.capacity, cfg.probes, cfg.dim, cfg.batch
    identity, stamps = identity0.clone(), stamps0.clone()
    values = torch.zeros((C, D), dtype=torch.float32, device=dev)
    tab = oracle.MPZCHTable(C, P, D, with_values=False)
    tab.identity, tab.stamps = tab0.identity.copy(), tab0.stamps.copy()
    tab.values = np.zeros((C, D), np.float32)
    steps, fc = 4, 0
    ids_np = []
    for t in range(1, steps + 1):
        x, fc = synth.mpzch_step_ids(cfg, t, fc)
        ids_np.append(x)
    ids = [torch.from_numpy(x).to(dev) for x in ids_np]
    es = [synth.normal_rows(n, D, cfg.e_std, cfg.config, t + 1, device=dev) for t in range(steps)]
    outs = [torch.empty((n, D), dtype=torch.float32, device=dev) for _ in range(steps)]
    stats = [torch.zeros(6, dtype=torch.int64, device=dev) for _ in range(steps)]
    torch.cuda.synchronize()
    pipe = MemoryLayerPipeline(identity, stamps, values, P, n, depth=3)
    pipe.prefetch(ids[0], base + 1, stats=stats[0])
    for t in range(steps):
        if t + 1 < steps:
            pipe.prefetch(ids[t + 1], base + t + 2, stats=stats[t + 1])
        pipe.step(ids[t], base + t + 1, es[t], out=outs[t], stats=stats[t])
    touched = set()
    for t in range(steps):
        orows, ohit, oev, ost = tab.step(ids_np[t], base + t + 1)
        oout = tab.gather(orows)
        tab.writeback(orows, to_np(es[t]))
        assert bits_equal(to_np(outs[t]), oout), f"gather step {t}"
        s = to_np(stats[t])
        assert np.array_equal(s[:5], ost) and s[5] == 0, (t, s, ost)
        touched.update(np.unique(orows[orows >= 0]).tolist())
        print(f"step {t}: inserts {ost[1]}", flush=True)
    assert np.array_equal(to_np(identity), tab.identity)
    assert np.array_equal(to_np(stamps), tab.stamps)
    idx = np.array(sorted(touched), dtype=np.int64)
    assert bits_equal(to_np(values[torch.from_numpy(idx).to(dev)]), tab.values[idx])
    assert int((values != 0).any(dim=1).sum().item()) == int(np.count_nonzero(tab.values[idx].any(axis=1)))
    free(values, identity, stamps, *outs)


def test_serving_score_full_size(dev, prefilled):
    cfg, identity, _, tab, _ = prefilled
    sv = synth.SERVING
    C, D = sv.capacity, sv.dim
    keys = synth.universe_keys(cfg.universe, cfg.config)
    resident = np.isin(keys, tab.identity[tab.identity >= 0])
    cands = synth.serving_candidates(keys[resident], sv.requests, sv.cands, sv.zipf_s, sv.miss_frac)
    q, scale, bias = synth.int8_table(C, D, device=dev)
    user = synth.normal_rows(sv.requests, D, 1.0, 3, 0, device=dev)
    ids = torch.from_numpy(cands).to(dev)
    rows, hit, _, _ = hlr.mpzch_lookup_or_insert(identity, None, None, cfg.probes, ids, 0, insert=False)
    scores = hlr.gather_dequant_score(q, scale, bias, rows, user, sv.cands)
    orows, ohit, _, _ = tab.step(cands, 0, insert=False)
    assert np.array_equal(to_np(rows), orows) and np.array_equal(to_np(hit), ohit)
    q_np, s_np, b_np, u_np = to_np(q), to_np(scale), to_np(bias), to_np(user)
    ref = oracle.dequant_score(q_np, s_np, b_np, orows, u_np, sv.cands)
    got = to_np(scores)
    sel = orows.reshape(sv.requests, sv.cands)
    x = q_np[np.maximum(sel, 0)].astype(np.float64) * s_np[np.maximum(sel, 0)][..., None] + \
        b_np[np.maximum(sel, 0)][..., None]
    cond = np.einsum("rkd,rd->rk", np.abs(x), np.abs(u_np.astype(np.float64)))
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    assert np.all(err <= 1e-6 * cond), float((err / np.maximum(cond, 1e-300)).max())
    assert np.all(got[sel < 0] == 0.0)
    print(f"serving: hit rate {ohit.mean():.4f}, max err/cond {float((err / np.maximum(cond, 1e-300)).max()):.3e}")
    free(q, scale, bias, user, rows, scores)


def test_dlrm_hashed_tables_full_size(dev):
    cfg = synth.DLRM
    D, n = cfg.dim, cfg.per_table
    tables = []
    for t, nr in enumerate(cfg.table_rows):
        x = torch.empty((nr, D), dtype=torch.float32, device=dev)
        synth.dlrm_fill_table(t, nr, D, x)
        tables.append(x)
    torch.cuda.synchronize()
    print(f"allocated {sum(x.numel() for x in tables) * 4 / 2**30:.1f} GiB of tables", flush=True)
    rng = np.random.default_rng(44)
    for t, nr in enumerate(cfg.table_rows):
        keys = synth.dlrm_keys(cfg, t, 1)
        g = synth.normal_rows(n, D, cfg.g_std, 4, 100 + t, device=dev)
        rows = hlr.hashed_rows(torch.from_numpy(keys).to(dev), nr)
        out = hlr.gather_rows(tables[t], rows)
        hlr.writeback_rows(tables[t], rows, g, mode=hlr.WB_SGD_SUM, lr=cfg.lr)
        orows = oracle.hashed_rows(keys, nr)
        assert np.array_equal(to_np(rows), orows), f"table {t} rows"
        uniq, inv = np.unique(orows, return_inverse=True)
        sub = synth.dlrm_initial_rows(t, uniq, D).numpy()  # compact copy of the touched rows
        assert bits_equal(to_np(out), oracle.gather(sub, inv.reshape(-1))), f"table {t} gather"
        oracle.sgd_sum(sub, inv.reshape(-1), to_np(g), cfg.lr)
        got = to_np(tables[t][torch.from_numpy(uniq).to(dev)])
        assert bits_equal(got, sub), f"table {t} updated rows"
        untouched = np.setdiff1d(rng.integers(0, nr, size=4096), uniq)
        assert bits_equal(to_np(tables[t][torch.from_numpy(untouched).to(dev)]),
                          synth.dlrm_initial_rows(t, untouched, D).numpy())
        print(f"table {t}: {nr} rows, {uniq.size} distinct, top row x{np.bincount(inv.reshape(-1)).max()}",
              flush=True)
        free(g, rows, out)
    free(*tables)


def test_cs3_ema_full_size(dev):
    cfg = synth.CS3
    D = cfg.dim
    shapes = {"c_user": cfg.users, "s_user": cfg.users, "c_item": cfg.items, "s_item": cfg.items}
    gpu = {k: torch.zeros((m, D), dtype=torch.float32, device=dev) for k, m in shapes.items()}
    cpu = {k: np.zeros((m, D), np.float32) for k, m in shapes.items()}
    for step in range(1, 3):
        urows, irows, y = synth.cs3_step(cfg, step)
        v_item = synth.normal_rows(cfg.batch, D, 1.0, 5, step, stream=1, device=dev)
        v_user = synth.normal_rows(cfg.batch, D, 1.0, 5, step, stream=2, device=dev)
        h = synth.normal_rows(cfg.batch, D, 1.0, 5, step, stream=3, device=dev)
        ur, ir, yy = (torch.from_numpy(x).to(dev) for x in (urows, irows, y))
        hlr.ema_update_rows(gpu["c_user"], ur, v_item, yy, cfg.cts_a, cfg.cts_b)
        hlr.ema_update_rows(gpu["c_item"], ir, v_user, yy, cfg.cts_a, cfg.cts_b)
        hlr.ema_update_rows(gpu["s_user"], ur, h, None, cfg.cms_a, cfg.cms_b)
        hlr.ema_update_rows(gpu["s_item"], ir, h, None, cfg.cms_a, cfg.cms_b)
        vi, vu, hh = to_np(v_item), to_np(v_user), to_np(h)
        oracle.ema(cpu["c_user"], urows, vi, y, cfg.cts_a, cfg.cts_b)
        oracle.ema(cpu["c_item"], irows, vu, y, cfg.cts_a, cfg.cts_b)
        oracle.ema(cpu["s_user"], urows, hh, None, cfg.cms_a, cfg.cms_b)
        oracle.ema(cpu["s_item"], irows, hh, None, cfg.cms_a, cfg.cms_b)
        print(f"step {step}: positives {int(y.sum())}, top user x{np.bincount(urows).max()}", flush=True)
        free(v_item, v_user, h)
    for k in shapes:
        assert bits_equal(to_np(gpu[k]), cpu[k]), k
    free(*gpu.values())
