"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

  * Memory-Layer cache: 4,194,304 x 512 fp32, 8 probes, prefilled with a 20M-ID
    universe, then 65,536-ID steps (Zipf 1.05 + 0.5% fresh): rows, hit,
    evicted, stats every step; identity and stamps in full; every touched row
    bit for bit and the count of non-zero rows (no stray writes); then the
    benchmark's configuration (memory_layer_step, two streams, lookahead, ring
    depth 3, the 200 steps as one HIP graph): every step's rows, hit, evicted,
    stats and gathered rows, and the whole table at the end, bit for bit.
  * Serving read path: that prefilled identity, an int8 4Mi x 512 table,
    256 requests x 1024 candidates: lookup-only rows/hit bit-exact, scores
    within 1e-6 relative (absolute floor 1e-12 sum_d |x_d u_d|); the same
    over the table the 200 benched steps trained, row-quantised to int8.
  * DLRMv4-like: 8 hashed tables (120 GiB), 131,072 keys per table, gather
    and duplicate-summed SGD (lr 0.01) through the benched pipeline (groups of
    four tables, one batched apply each), three steps: every gathered row and
    every touched row bit-exact; sampled untouched rows unchanged.
  * CS3 EMA: 1Mi/2Mi x 128 tables, 262,144 pairs, CTS on positives and CMS on
    all pairs, ten steps through the benched pipeline: every row bit-exact.
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


@pytest.mark.timeout(600)
def test_res_publisher_full_size(dev, prefilled):
    """The RES bench's configuration at full size: MemoryLayerPipeline steps with a publisher (the one-call
    step's two halves, each batch's written rows marked from its row grouping), 20 batches, then one publish
    at the batch boundary (Memory Layer page, sec. 2, Raw Embedding Streaming; sec. 5, int8 rows): the packet
    lists exactly the rows the oracle wrote, each once, their int8 rows and scales equal the oracle's
    quantisation of its table, and the identity and stamps snapshot equals the oracle's after the last batch."""
    from hashed_lookup_row_amd.pipeline import MemoryLayerPipeline, RESPublisher
    cfg, identity0, stamps0, tab0, base = prefilled
    C, P, D, n = cfg.capacity, cfg.probes, cfg.dim, cfg.batch
    identity, stamps = identity0.clone(), stamps0.clone()
    values = torch.zeros((C, D), dtype=torch.float32, device=dev)
    tab = oracle.MPZCHTable(C, P, D, with_values=False)
    tab.identity, tab.stamps = tab0.identity.copy(), tab0.stamps.copy()
    tab.values = np.zeros((C, D), np.float32)
    steps, fc = 20, 0
    stream = []
    for t in range(1, steps + 1):
        ids_np, fc = synth.mpzch_step_ids(cfg, t, fc)
        stream.append(ids_np)
    e_pool = [synth.normal_rows(n, D, cfg.e_std, cfg.config, t + 1, device=dev) for t in range(4)]
    ids = [torch.from_numpy(x).to(dev) for x in stream]
    torch.cuda.synchronize()
    packets = []
    pipe = MemoryLayerPipeline(identity, stamps, values, P, n)
    pub = RESPublisher(pipe, 0, on_publish=packets.append, max_rows=1 << 20)
    for t in range(steps):
        pipe.step(ids[t], base + 1 + t, e_pool[t % 4], publisher=pub)
    pub.publish_now(pipe)
    pub.flush()
    torch.cuda.synchronize()
    written = set()
    for t in range(steps):
        orows, _, _, _ = tab.step(stream[t], base + 1 + t)
        tab.writeback(orows, to_np(e_pool[t % 4]))
        written |= set(np.unique(orows[orows >= 0]).tolist())
    assert len(packets) == 1
    p = packets[0]
    assert len(p["rows"]) == len(written) and set(p["rows"].tolist()) == written
    oq, osc, obi = oracle.quantize_rows(tab.values, p["rows"])
    assert np.array_equal(p["q"], oq) and bits_equal(p["scale"], osc) and bits_equal(p["bias"], obi)
    assert np.array_equal(p["identity"], tab.identity) and np.array_equal(p["stamps"], tab.stamps)
    print(f"published {len(written)} rows written by {steps} batches", flush=True)
    free(values, identity, stamps)


@pytest.mark.timeout(900)
def test_memory_layer_200_steps_benched_schedule_then_serving(dev, prefilled):
    """The headline's launch configuration over the workload's whole 200-step stream: memory_layer_step
    through MemoryLayerPipeline in the grouped two-stream schedule (the lookups of 4 batches back to back,
    two groups ahead of the row passes, ring depth 16), the 200 batches captured as one HIP graph and
    replayed, as bench.py times them.  Every step's rows,
    hit mask, evicted IDs, stats and gathered rows bit for bit, then the ID table and the whole 8 GiB
    table.  Then the serving table is that trained table row-quantised to int8 (quantize_rows_int8 over
    every row, bit for bit against the oracle's quantiser), and 256 x 1024 candidates are looked up
    (lookup-only) and scored against it: scores within 1e-6 relative (plus an absolute floor of 1e-12
    times the condition scale sum_d |x_d u_d|, for scores that nearly cancel)."""
    from hashed_lookup_row_amd.pipeline import MemoryLayerPipeline, StepGraph
    cfg, identity0, stamps0, tab0, base = prefilled
    C, P, D, n = cfg.capacity, cfg.probes, cfg.dim, cfg.batch
    steps = cfg.steps
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        identity, stamps = identity0.clone(), stamps0.clone()
        values = torch.zeros((C, D), dtype=torch.float32, device=dev)
        ids_np, fc = [], 0
        for t in range(1, steps + 1):
            x, fc = synth.mpzch_step_ids(cfg, t, fc)
            ids_np.append(x)
        ids = [torch.from_numpy(x).to(dev) for x in ids_np]
        npool = 16
        es = [synth.normal_rows(n, D, cfg.e_std, cfg.config, t + 1, device=dev) for t in range(npool)]
        outs = [torch.empty((n, D), dtype=torch.float32, device=dev) for _ in range(steps)]
        evs = [torch.empty(n, dtype=torch.int64, device=dev) for _ in range(steps)]
        sts = [torch.zeros(6, dtype=torch.int64, device=dev) for _ in range(steps)]
        rws = [torch.empty(n, dtype=torch.int64, device=dev) for _ in range(steps)]
        hts = [torch.empty(n, dtype=torch.int8, device=dev) for _ in range(steps)]
        # as bench.py: the grouped schedule captured, groups of 4 batches, lookups 2 groups ahead, ring of 16
        pipe = MemoryLayerPipeline(identity, stamps, values, P, n, depth=16)
        graph = StepGraph(pipe, [(ids[t], base + t + 1, es[t % npool], outs[t], evs[t], sts[t], rws[t], hts[t])
                                 for t in range(steps)], ahead=2, group=4)
        graph.replay()
        torch.cuda.synchronize()
    e_np = [to_np(x) for x in es]
    tab = oracle.MPZCHTable(C, P, D, with_values=False)
    tab.identity, tab.stamps = tab0.identity.copy(), tab0.stamps.copy()
    tab.values = np.zeros((C, D), np.float32)
    for t in range(steps):
        orows, ohit, oev, ost = tab.step(ids_np[t], base + t + 1)
        assert np.array_equal(to_np(rws[t]), orows), f"rows step {t}"
        assert np.array_equal(to_np(hts[t]), ohit), f"hit step {t}"
        assert np.array_equal(to_np(evs[t]), oev), f"evicted step {t}"
        s_ = to_np(sts[t])
        assert np.array_equal(s_[:5], ost) and s_[5] == 0, (t, s_, ost)
        assert bits_equal(to_np(outs[t]), tab.gather(orows)), f"gather step {t}"
        tab.writeback(orows, e_np[t % npool])
        if t % 50 == 0:
            print(f"step {t}: inserts {ost[1]}, hits {ost[0]}", flush=True)
    free(*outs)
    assert np.array_equal(to_np(identity), tab.identity)
    assert np.array_equal(to_np(stamps), tab.stamps)
    for r0 in range(0, C, 1 << 20):  # the whole table, in 2 GiB pieces
        assert bits_equal(to_np(values[r0:r0 + (1 << 20)]), tab.values[r0:r0 + (1 << 20)]), f"values from row {r0}"
    print("200 steps bit-exact", flush=True)

    # serving reads the trained table, row-quantised to int8
    sv = synth.SERVING
    allrows = torch.arange(C, dtype=torch.int64, device=dev)
    q, scale, bias = hlr.quantize_rows_int8(values, allrows)
    free(values)
    oq, osc, obi = oracle.quantize_rows(tab.values, np.arange(C, dtype=np.int64))
    q_np, s_np, b_np = to_np(q), to_np(scale), to_np(bias)
    assert bits_equal(q_np, oq) and bits_equal(s_np, osc) and bits_equal(b_np, obi), "int8 quantisation"
    del oq
    keys = synth.universe_keys(cfg.universe, cfg.config)
    resident = np.isin(keys, tab.identity[tab.identity >= 0])
    cands = synth.serving_candidates(keys[resident], sv.requests, sv.cands, sv.zipf_s, sv.miss_frac)
    user = synth.normal_rows(sv.requests, D, 1.0, 3, 0, device=dev)
    cid = torch.from_numpy(cands).to(dev)
    rows, hit, _, _ = hlr.mpzch_lookup_or_insert(identity, None, None, P, cid, 0, insert=False)
    scores = hlr.gather_dequant_score(q, scale, bias, rows, user, sv.cands)
    orows, ohit, _, _ = tab.step(cands, 0, insert=False)
    assert np.array_equal(to_np(rows), orows) and np.array_equal(to_np(hit), ohit)
    u_np = to_np(user)
    ref = oracle.dequant_score(q_np, s_np, b_np, orows, u_np, sv.cands).astype(np.float64)
    got = to_np(scores).astype(np.float64)
    sel = orows.reshape(sv.requests, sv.cands)
    x = q_np[np.maximum(sel, 0)].astype(np.float64) * s_np[np.maximum(sel, 0)][..., None] + \
        b_np[np.maximum(sel, 0)][..., None]
    cond = np.einsum("rkd,rd->rk", np.abs(x), np.abs(u_np.astype(np.float64)))
    err = np.abs(got - ref)
    assert np.all(err <= 1e-6 * np.abs(ref) + 1e-12 * cond), float((err / np.maximum(np.abs(ref), 1e-30)).max())
    assert np.all(got[sel < 0] == 0.0)
    print(f"serving from the trained table: hit rate {ohit.mean():.4f}, max rel err "
          f"{float((err / np.maximum(np.abs(ref), 1e-30)).max()):.3e}", flush=True)
    free(q, scale, bias, user, rows, scores, identity, stamps)


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
    # 1e-6 relative, plus an absolute floor of 1e-12 of the condition scale for scores that nearly cancel
    assert np.all(err <= 1e-6 * np.abs(ref.astype(np.float64)) + 1e-12 * cond), \
        float((err / np.maximum(np.abs(ref.astype(np.float64)), 1e-30)).max())
    assert np.all(got[sel < 0] == 0.0)
    print(f"serving: hit rate {ohit.mean():.4f}, max err/cond {float((err / np.maximum(cond, 1e-300)).max()):.3e}")
    # the same lookup and score in one launch (the serving bench's step): the same rows, hit mask and scores
    rows2 = torch.empty_like(rows)
    hit2 = torch.empty_like(hit)
    fused = hlr.mpzch_score(identity, cfg.probes, ids, q, scale, bias, user, sv.cands, out_rows=rows2, out_hit=hit2)
    assert np.array_equal(to_np(rows2), orows) and np.array_equal(to_np(hit2), ohit)
    assert bits_equal(to_np(fused), got)
    free(q, scale, bias, user, rows, scores, fused, rows2, hit2)


@pytest.mark.timeout(900)
def test_dlrm_hashed_tables_full_size(dev):
    """The bench's launch configuration: HashedTablesPipeline, tables in two groups of four, one batched
    SGD apply per group, three steps without synchronising in between (step t+1 gathers rows step t
    updated).  Every hashed row, every gathered row of every step and every touched row after the last
    step bit for bit; sampled untouched rows unchanged.  The oracle keeps a compact overlay of touched
    rows over the closed-form initial tables (120 GiB do not fit on the host)."""
    from hashed_lookup_row_amd.pipeline import HashedTablesPipeline
    cfg = synth.DLRM
    D, n = cfg.dim, cfg.per_table
    steps = 3
    tables = []
    for t, nr in enumerate(cfg.table_rows):
        x = torch.empty((nr, D), dtype=torch.float32, device=dev)
        synth.dlrm_fill_table(t, nr, D, x)
        tables.append(x)
    torch.cuda.synchronize()
    print(f"allocated {sum(x.numel() for x in tables) * 4 / 2**30:.1f} GiB of tables", flush=True)
    keys = [[synth.dlrm_keys(cfg, t, s + 1) for t in range(8)] for s in range(steps)]
    kd = [[torch.from_numpy(k).to(dev) for k in ks] for ks in keys]
    grads = [[synth.normal_rows(n, D, cfg.g_std, 4, 100 * s + t, device=dev) for t in range(8)] for s in range(steps)]
    outs = [[torch.empty((n, D), dtype=torch.float32, device=dev) for _ in range(8)] for _ in range(steps)]
    pipe = HashedTablesPipeline(tables, n, batch=True, group=4)
    for s in range(steps):
        pipe.step(kd[s], grads[s], cfg.lr, outs[s])
    torch.cuda.synchronize()
    rng = np.random.default_rng(44)
    for t, nr in enumerate(cfg.table_rows):
        state = {}  # row -> current fp32 vector (touched rows only)
        for s in range(steps):
            orows = oracle.hashed_rows(keys[s][t], nr)
            uniq, inv = np.unique(orows, return_inverse=True)
            inv = inv.reshape(-1)
            cur = synth.dlrm_initial_rows(t, uniq, D).numpy()
            have = np.array([r in state for r in uniq.tolist()])
            if have.any():
                cur[have] = np.stack([state[r] for r in uniq[have].tolist()])
            assert bits_equal(to_np(outs[s][t]), oracle.gather(cur, inv)), f"table {t} step {s} gather"
            oracle.sgd_sum(cur, inv, to_np(grads[s][t]), cfg.lr)
            for r, v in zip(uniq.tolist(), cur):
                state[r] = v
        touched = np.array(sorted(state), dtype=np.int64)
        got = to_np(tables[t][torch.from_numpy(touched).to(dev)])
        assert bits_equal(got, np.stack([state[r] for r in touched.tolist()])), f"table {t} touched rows"
        untouched = np.setdiff1d(rng.integers(0, nr, size=4096), touched)
        assert bits_equal(to_np(tables[t][torch.from_numpy(untouched).to(dev)]),
                          synth.dlrm_initial_rows(t, untouched, D).numpy())
        print(f"table {t}: {nr} rows, {touched.size} touched over {steps} steps", flush=True)
    free(*tables)


@pytest.mark.parametrize("pairs,derive", [(True, False), (False, True)])
def test_cs3_ema_full_size(dev, pairs, derive):
    """The bench's launch configuration: EMAPipeline with pair plans (each rule's user- and item-keyed
    updates planned by one sort, the CMS and the CTS pair on two lookup streams, all four applies as one
    launch), and the unpaired one (four plans, CTS cut out of CMS, on two lookup streams), in the grouped
    schedule (run(): plans of four steps back to back, a group ahead of the applies) for ten steps of
    262,144 pairs, after two step() calls, without synchronising in between; all four tables bit for bit
    against the sequential oracle over the twelve steps."""
    from hashed_lookup_row_amd.pipeline import EMAPipeline
    cfg = synth.CS3
    D, n = cfg.dim, cfg.batch
    steps = 12
    shapes = {"c_user": cfg.users, "s_user": cfg.users, "c_item": cfg.items, "s_item": cfg.items}
    gpu = {k: torch.zeros((m, D), dtype=torch.float32, device=dev) for k, m in shapes.items()}
    cpu = {k: np.zeros((m, D), np.float32) for k, m in shapes.items()}
    inp = []
    for step in range(1, steps + 1):
        urows, irows, y = synth.cs3_step(cfg, step)
        dvals = [synth.normal_rows(n, D, 1.0, 5, step, stream=k, device=dev) for k in (1, 2, 3)]  # v_item, v_user, h
        inp.append(((urows, irows, y), [torch.from_numpy(x).to(dev) for x in (urows, irows, y)], dvals))
    calls = [("c_user", 0, 0, True, cfg.cts_a, cfg.cts_b), ("c_item", 1, 1, True, cfg.cts_a, cfg.cts_b),
             ("s_user", 0, 2, False, cfg.cms_a, cfg.cms_b), ("s_item", 1, 2, False, cfg.cms_a, cfg.cms_b)]
    pipe = EMAPipeline([gpu[c[0]] for c in calls], n, depth=12, lookup_streams=2, batch=True, pairs=pairs,
                       derive=derive)
    args = [([x[c[1]] for c in calls], [x[2] if c[3] else None for c in calls], [v[c[2]] for c in calls],
             [(c[4], c[5]) for c in calls]) for _, x, v in inp]
    pipe.step(*args[0])
    pipe.step(*args[1])
    pipe.run(args[2:], group=4, ahead=1)
    torch.cuda.synchronize()
    for step, ((urows, irows, y), _, v) in enumerate(inp, start=1):
        vn = [to_np(x) for x in v]
        for name, ri, vi, masked, a, b in calls:
            oracle.ema(cpu[name], (urows, irows)[ri], vn[vi], y if masked else None, a, b)
        print(f"step {step}: positives {int(y.sum())}, top user x{np.bincount(urows).max()}", flush=True)
    for k in shapes:
        assert bits_equal(to_np(gpu[k]), cpu[k]), k
    free(*gpu.values())


def test_ema_values_over_2gib(dev):
    """EMA update with a values array of 2 GiB (n = 524,288 positions of 1024 floats): the heavy walk
    then addresses values with 64-bit offsets instead of 32-bit buffer offsets.  Few rows, so every
    row is long and cut into chunks; bit for bit against the oracle's batch-order loop (CS3 page, sec. 2)."""
    cfg = synth.CS3
    n, D, R = 524_288, 1024, 97
    g = np.random.default_rng(23)
    rows = np.minimum(synth.zipf_ranks(g, R, 1.1, n), R - 1).astype(np.int64)
    vals = g.standard_normal((n, D), dtype=np.float32)
    table = g.standard_normal((R, D), dtype=np.float32)
    assert vals.nbytes >= 1 << 31
    t = torch.from_numpy(table).to(dev)
    hlr.ema_update_rows(t, torch.from_numpy(rows).to(dev), torch.from_numpy(vals).to(dev), None, cfg.cms_a, cfg.cms_b)
    torch.cuda.synchronize()
    oracle.ema(table, rows, vals, None, cfg.cms_a, cfg.cms_b)
    assert bits_equal(to_np(t), table)
