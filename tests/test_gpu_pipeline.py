"""GPU parity of the split entry points (plan / apply, lookup without values + zero-fill) and of
the two-stream schedules in hashed_lookup_row_amd.pipeline, against the oracle.

The schedules are run for several batches without synchronising in between, so the lookup
stream really runs ahead of the compute stream; every output of every batch and the final
state must equal the oracle's sequential result bit for bit.
"""
import numpy as np
import pytest
import torch

import hashed_lookup_row_amd as hlr
import oracle
import synth
from hashed_lookup_row_amd import pipeline

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


def side_stream_plan(dev, plan):
    """Runs plan() on another stream and makes the current stream wait for it."""
    s = torch.cuda.Stream(dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        plan()
    torch.cuda.current_stream(dev).wait_stream(s)


@pytest.mark.parametrize("mode,lr", [(hlr.WB_LAST_WINS, 1.0), (hlr.WB_SGD_SUM, 0.01), (hlr.WB_L2_ALIGN, 0.1)])
@pytest.mark.parametrize("num_rows,n,D", [(50, 3000, 64), (5000, 20_000, 512), (7, 1, 4)])
def test_writeback_plan_apply(dev, mode, lr, num_rows, n, D):
    g = np.random.default_rng(num_rows + n + mode)
    rows = g.integers(-1, num_rows, size=n).astype(np.int64)
    rows[g.random(n) < 0.3] = 3 % num_rows  # a hot row
    src = g.standard_normal((n, D)).astype(np.float32)
    table = g.standard_normal((num_rows, D)).astype(np.float32)
    t = torch.from_numpy(table).to(dev)
    r = torch.from_numpy(rows).to(dev)
    ws = hlr.new_workspace(dev, hlr.writeback_workspace_size(num_rows, D, n, mode))
    side_stream_plan(dev, lambda: hlr.writeback_plan(num_rows, r, ws, mode))
    hlr.writeback_apply(t, torch.from_numpy(src).to(dev), ws, mode, lr)
    if mode == hlr.WB_LAST_WINS:
        oracle.writeback_last(table, rows, src)
    elif mode == hlr.WB_SGD_SUM:
        oracle.sgd_sum(table, rows, src, lr)
    else:
        oracle.l2_align(table, rows, src, lr)
    assert bits_equal(to_np(t), table)


@pytest.mark.parametrize("masked", [False, True])
def test_ema_plan_apply(dev, masked):
    g = np.random.default_rng(7 + masked)
    num_rows, n, D = 300, 30_000, 128
    rows = np.minimum(synth.zipf_ranks(g, num_rows, 1.1, n), num_rows - 1).astype(np.int64)
    vals = g.standard_normal((n, D)).astype(np.float32)
    mask = (g.random(n) < 0.5).astype(np.uint8) if masked else None
    table = g.standard_normal((num_rows, D)).astype(np.float32)
    t = torch.from_numpy(table).to(dev)
    r = torch.from_numpy(rows).to(dev)
    m = torch.from_numpy(mask).to(dev) if masked else None
    ws = hlr.new_workspace(dev, hlr.ema_workspace_size(num_rows, D, n))
    side_stream_plan(dev, lambda: hlr.ema_update_plan(num_rows, r, m, ws))
    hlr.ema_update_apply(t, torch.from_numpy(vals).to(dev), 0.95, 0.05, ws)
    oracle.ema(table, rows, vals, mask, 0.95, 0.05)
    assert bits_equal(to_np(t), table)


@pytest.mark.parametrize("src_masked", [False, True])
@pytest.mark.parametrize("num_rows,n,D,dense", [(300, 30_000, 128, 0.05), (5000, 20_000, 64, 0.7), (40, 777, 8, 0.3)])
def test_ema_plan_subset(dev, src_masked, num_rows, n, D, dense):
    """A plan cut out of another plan (positions with a second mask) applies like a plan made from the
    rows with both masks; the source plan is left intact and still applies to its own result."""
    g = np.random.default_rng(num_rows + n + src_masked)
    rows = np.minimum(synth.zipf_ranks(g, num_rows, 1.1, n), num_rows - 1).astype(np.int64)
    rows[g.random(n) < 0.02] = -1
    rows[g.random(n) < 0.01] = num_rows + 3  # out of range: takes no part
    vals = g.standard_normal((n, D)).astype(np.float32)
    m1 = (g.random(n) < 0.8).astype(np.uint8) if src_masked else None
    m2 = (g.random(n) < dense).astype(np.uint8)
    table = g.standard_normal((num_rows, D)).astype(np.float32)
    t_all, t_sub = (torch.from_numpy(table).to(dev) for _ in range(2))
    r, v = torch.from_numpy(rows).to(dev), torch.from_numpy(vals).to(dev)
    ws_src = hlr.new_workspace(dev, hlr.ema_workspace_size(num_rows, D, n))
    ws_sub = hlr.new_workspace(dev, hlr.ema_workspace_size(num_rows, D, n))
    hlr.ema_update_plan(num_rows, r, torch.from_numpy(m1).to(dev) if src_masked else None, ws_src)
    hlr.ema_update_plan_subset(num_rows, torch.from_numpy(m2).to(dev), ws_src, ws_sub)
    hlr.ema_update_apply(t_sub, v, 0.9, 0.1, ws_sub)
    hlr.ema_update_apply(t_all, v, 0.95, 0.05, ws_src)
    both = m2 if m1 is None else (m1 & m2)
    want_sub, want_all = table.copy(), table.copy()
    orows = np.where(rows < num_rows, rows, -1)  # the oracle takes -1 for "no row"
    oracle.ema(want_sub, orows, vals, both, 0.9, 0.1)
    oracle.ema(want_all, orows, vals, m1, 0.95, 0.05)
    assert bits_equal(to_np(t_sub), want_sub)
    assert bits_equal(to_np(t_all), want_all)


@pytest.mark.parametrize("src_masked", [False, True])
@pytest.mark.parametrize("U,I,n,D", [(4096, 8192, 30_000, 128), (300, 7, 20_000, 64), (1, 3000, 5000, 48),
                                     (2000, 2000, 777, 8)])
def test_ema_pair_plan(dev, src_masked, U, I, n, D):
    """A pair plan (the positions of a user-keyed and an item-keyed update grouped by one sort) applied with
    ema_update_apply_pairs equals the oracle's batch-order EMA on each table (CS3 page, sec. 2), with rows out
    of range in both halves, hot rows long enough to be cut into chunks, a table of a single row; a subset cut
    out of the pair plan applies like the two updates with both masks, and the source plan still applies."""
    g = np.random.default_rng(U + I + n + src_masked)
    r0 = np.minimum(synth.zipf_ranks(g, U, 1.1, n), U - 1).astype(np.int64)
    r1 = np.minimum(synth.zipf_ranks(g, I, 1.05, n), I - 1).astype(np.int64)
    r0[g.random(n) < 0.02] = -1
    r1[g.random(n) < 0.01] = I + 5
    v0 = g.standard_normal((n, D)).astype(np.float32)
    v1 = g.standard_normal((n, D)).astype(np.float32)
    m1 = (g.random(n) < 0.8).astype(np.uint8) if src_masked else None
    m2 = (g.random(n) < 0.3).astype(np.uint8)
    t0 = g.standard_normal((U, D)).astype(np.float32)
    t1 = g.standard_normal((I, D)).astype(np.float32)
    d = lambda x: torch.from_numpy(x).to(dev)
    a0, a1, s0, s1 = d(t0), d(t1), d(t0), d(t1)
    r0d, r1d, v0d, v1d = d(r0), d(r1), d(v0), d(v1)
    need = hlr.ema_pair_workspace_size(U, I, D, n)
    ws_src, ws_sub = hlr.new_workspace(dev, need), hlr.new_workspace(dev, need)
    hlr.ema_update_plan_pair(U, r0d, I, r1d, d(m1) if src_masked else None, ws_src)
    hlr.ema_update_plan_pair_subset(U, I, d(m2), ws_src, ws_sub)
    hlr.ema_update_apply_pairs([(s0, v0d, s1, v1d, 0.9, 0.1, ws_sub)])
    hlr.ema_update_apply_pairs([(a0, v0d, a1, v1d, 0.95, 0.05, ws_src)])
    both = m2 if m1 is None else (m1 & m2)
    o0 = np.where(r0 < U, r0, -1)
    o1 = np.where(r1 < I, r1, -1)  # the oracle takes -1 for "no row"
    w = {k: x.copy() for k, x in (("a0", t0), ("a1", t1), ("s0", t0), ("s1", t1))}
    oracle.ema(w["a0"], o0, v0, m1, 0.95, 0.05)
    oracle.ema(w["a1"], o1, v1, m1, 0.95, 0.05)
    oracle.ema(w["s0"], o0, v0, both, 0.9, 0.1)
    oracle.ema(w["s1"], o1, v1, both, 0.9, 0.1)
    for k, x in (("a0", a0), ("a1", a1), ("s0", s0), ("s1", s1)):
        assert bits_equal(to_np(x), w[k]), k


def test_ema_pair_argument_errors(dev):
    """Pair plans refuse sizes past the key range, shared tables and mismatched inputs (host-side errors)."""
    assert hlr.ema_pair_workspace_size(1 << 30, 1 << 30, 4, 10) == 0
    assert hlr.ema_pair_workspace_size(5, 5, 4, 10) > 0
    t = torch.zeros((64, 8), dtype=torch.float32, device=dev)
    v = torch.zeros((16, 8), dtype=torch.float32, device=dev)
    rows = torch.zeros(16, dtype=torch.int64, device=dev)
    ws = hlr.new_workspace(dev, hlr.ema_pair_workspace_size(64, 64, 8, 16))
    hlr.ema_update_plan_pair(64, rows, 64, rows, None, ws)
    with pytest.raises(hlr.HLRError):
        hlr.ema_update_apply_pairs([(t, v, t, v, 0.5, 0.5, ws)])  # one table twice
    with pytest.raises(hlr.HLRError):
        hlr.ema_update_plan_pair(64, rows, 64, rows[:8], None, ws)


def test_ema_apply_batch(dev):
    """Four updates of different tables in one launch (long and short chunks, masked and cut plans, a
    row count that differs per table) equal the oracle applied to each in turn."""
    g = np.random.default_rng(23)
    D, n = 64, 40_000
    specs = [(300, 1.1, 0.99, 0.01, 0.1), (5000, 1.05, 0.95, 0.05, None), (900, 1.2, 0.9, 0.1, 0.5),
             (300, 1.1, 0.97, 0.03, None)]
    ups, want = [], []
    for num_rows, z, a, b, dense in specs:
        rows = np.minimum(synth.zipf_ranks(g, num_rows, z, n), num_rows - 1).astype(np.int64)
        rows[g.random(n) < 0.01] = -1
        vals = g.standard_normal((n, D)).astype(np.float32)
        mask = (g.random(n) < dense).astype(np.uint8) if dense is not None else None
        table = g.standard_normal((num_rows, D)).astype(np.float32)
        t = torch.from_numpy(table).to(dev)
        ws = hlr.new_workspace(dev, hlr.ema_workspace_size(num_rows, D, n))
        hlr.ema_update_plan(num_rows, torch.from_numpy(rows).to(dev),
                            torch.from_numpy(mask).to(dev) if mask is not None else None, ws)
        ups.append((t, torch.from_numpy(vals).to(dev), a, b, ws))
        oracle.ema(table, rows, vals, mask, a, b)
        want.append(table)
    hlr.ema_update_apply_batch(ups)
    for (t, *_), w in zip(ups, want):
        assert bits_equal(to_np(t), w)


@pytest.mark.parametrize("mode,D", [("sgd", 64), ("l2", 64), ("sgd", 512), ("l2", 1024), ("sgd", 4)])
def test_wb_apply_batch(dev, mode, D):
    """Eight SGD_SUM (or L2_ALIGN) updates of different tables in one batch (multi-run rows, a tiny
    table, an empty update, different row counts and learning rates) equal the oracle applied to each
    in turn."""
    g = np.random.default_rng((29 if mode == "sgd" else 31) + D)
    m = hlr.WB_SGD_SUM if mode == "sgd" else hlr.WB_L2_ALIGN
    specs = [(300, 1.1, 30_000), (5000, 1.05, 20_000), (2, 1.0, 3000), (900, 1.2, 0), (60_000, 1.2, 50_000),
             (40, 1.1, 777), (300, 1.3, 9000), (10_000, 1.15, 4096)]
    ups, want = [], []
    for k, (num_rows, z, n) in enumerate(specs):
        rows = np.minimum(synth.zipf_ranks(g, num_rows, z, n), num_rows - 1).astype(np.int64)
        rows[g.random(n) < 0.01] = -1
        src = (g.standard_normal((n, D)) * (1e-3 if mode == "sgd" else 1.0)).astype(np.float32)
        table = (g.standard_normal((num_rows, D)) * 0.01).astype(np.float32)
        lr = 0.01 * (k + 1)
        t = torch.from_numpy(table).to(dev)
        ws = hlr.new_workspace(dev, hlr.writeback_workspace_size(num_rows, D, n, m))
        hlr.writeback_plan(num_rows, torch.from_numpy(rows).to(dev), ws, m)
        ups.append((t, torch.from_numpy(src).to(dev), lr, ws))
        (oracle.sgd_sum if mode == "sgd" else oracle.l2_align)(table, rows, src, np.float32(lr))
        want.append(table)
    hlr.writeback_apply_batch(ups, mode=m)
    for k, ((t, *_), w) in enumerate(zip(ups, want)):
        assert bits_equal(to_np(t), w), k


def prefilled_pair(dev, cfg):
    C, P, D = cfg.capacity, cfg.probes, cfg.dim
    identity = torch.full((C,), -1, dtype=torch.int64, device=dev)
    stamps = torch.full((C,), -1, dtype=torch.int64, device=dev)
    o = oracle.MPZCHTable(C, P, D, with_values=False)
    batches = synth.prefill_batches(cfg)
    for k, b in enumerate(batches, start=1):
        hlr.mpzch_lookup_or_insert(identity, stamps, None, P, torch.from_numpy(b).to(dev), k)
        o.step(b, k)
    o.values = np.zeros((C, D), np.float32)
    return identity, stamps, o, len(batches)


def test_lookup_without_values_then_zero_inserted(dev):
    cfg = synth.scaled_memory_layer(capacity=8_192, universe=60_000, batch=4_096, steps=4, dim=64)
    C, P, D = cfg.capacity, cfg.probes, cfg.dim
    identity, stamps, o, base = prefilled_pair(dev, cfg)
    g = np.random.default_rng(3)
    values_np = g.standard_normal((C, D)).astype(np.float32)  # stale rows that inserts must clear
    o.values = values_np.copy()
    values = torch.from_numpy(values_np).to(dev)
    for t, ids_np in enumerate(synth.mpzch_stream(cfg, cfg.steps), start=1):
        ids = torch.from_numpy(ids_np).to(dev)
        rows, hit, _, _ = hlr.mpzch_lookup_or_insert(identity, stamps, None, P, ids, base + t)
        hlr.mpzch_zero_inserted(values, rows, hit)
        orows, ohit, _, _ = o.step(ids_np, base + t)
        assert np.array_equal(to_np(rows), orows) and np.array_equal(to_np(hit), ohit)
        assert bits_equal(to_np(values), o.values), f"step {t}"


@pytest.mark.parametrize("depth,native,lookahead", [(2, True, False), (3, True, False), (2, False, False),
                                                    (2, True, True), (3, True, True)])
def test_memory_layer_pipeline(dev, depth, native, lookahead):
    """The batch as one library call (native) and as seven, and with the next batch looked up
    before the current batch's row traffic (lookahead), all against the oracle."""
    cfg = synth.scaled_memory_layer(capacity=16_384, universe=120_000, batch=8_192, steps=8)
    C, P, D, n = cfg.capacity, cfg.probes, cfg.dim, cfg.batch
    identity, stamps, o, base = prefilled_pair(dev, cfg)
    values = torch.zeros((C, D), dtype=torch.float32, device=dev)
    ids_np = synth.mpzch_stream(cfg, cfg.steps)
    e_np = [synth.normal_rows_np(n, D, cfg.e_std, 2, t) for t in range(1, cfg.steps + 1)]
    ids = [torch.from_numpy(x).to(dev) for x in ids_np]
    es = [torch.from_numpy(x).to(dev) for x in e_np]
    outs = [torch.empty((n, D), dtype=torch.float32, device=dev) for _ in ids]
    evs = [torch.empty(n, dtype=torch.int64, device=dev) for _ in ids]
    sts = [torch.zeros(6, dtype=torch.int64, device=dev) for _ in ids]
    torch.cuda.synchronize()
    pipe = pipeline.MemoryLayerPipeline(identity, stamps, values, P, n, depth=depth, native=native)
    if lookahead:
        pipe.prefetch(ids[0], base + 1, evicted=evs[0], stats=sts[0])
    for t in range(cfg.steps):  # no synchronisation between batches
        if lookahead and t + 1 < cfg.steps:
            pipe.prefetch(ids[t + 1], base + t + 2, evicted=evs[t + 1], stats=sts[t + 1])
        pipe.step(ids[t], base + t + 1, es[t], out=outs[t], evicted=evs[t], stats=sts[t])
    last_rows = [to_np(pipe.rows(k)).copy() for k in range(depth)]
    for t in range(cfg.steps):
        orows, ohit, oev, ost = o.step(ids_np[t], base + t + 1)
        assert bits_equal(to_np(outs[t]), o.gather(orows)), f"gather step {t}"
        o.writeback(orows, e_np[t])
        assert np.array_equal(to_np(evs[t]), oev), f"evicted step {t}"
        assert np.array_equal(to_np(sts[t])[:5], ost), f"stats step {t}"
        if t >= cfg.steps - depth:
            assert np.array_equal(last_rows[t % depth], orows)
    assert np.array_equal(to_np(identity), o.identity)
    assert np.array_equal(to_np(stamps), o.stamps)
    assert bits_equal(to_np(values), o.values)


@pytest.mark.parametrize("C,P,D,n,depth", [(64, 8, 4, 1, 2), (64, 8, 12, 1023, 2), (256, 4, 1024, 1025, 3),
                                            (2048, 8, 512, 3000, 3), (96, 32, 64, 5000, 2)])
def test_memory_layer_step_edge_cases(dev, C, P, D, n, depth):
    """The one-call step (one pass over the batch's rows) against the oracle on edge cases: stale
    rows (an insert must read as zero, not as the evicted ID's vector), invalid IDs (-1), buckets
    overflowing (every slot pinned: row -1, zero vector, no Writeback), hot IDs spread over many
    1024-position tiles, ragged batch sizes (1, 1023, 1025, ...) and dims of 1, 3 and 256 16-byte
    units, with lookahead and batches of different sizes."""
    g = np.random.default_rng(C + n + D)
    steps = 6
    values_np = g.standard_normal((C, D)).astype(np.float32)
    identity = torch.full((C,), -1, dtype=torch.int64, device=dev)
    stamps = torch.full((C,), -1, dtype=torch.int64, device=dev)
    values = torch.from_numpy(values_np.copy()).to(dev)
    o = oracle.MPZCHTable(C, P, D)
    o.values = values_np.copy()
    universe = g.choice(1 << 40, size=4 * C, replace=False).astype(np.int64)
    sizes = [n if t % 2 == 0 else max(1, n // 2 + 1) for t in range(steps)]
    ids_np = []
    for t in range(steps):
        r = np.minimum(synth.zipf_ranks(g, universe.size, 1.2, sizes[t]), universe.size - 1)
        x = universe[r]
        x[g.random(sizes[t]) < 0.02] = -1
        ids_np.append(x.astype(np.int64))
    ids = [torch.from_numpy(x).to(dev) for x in ids_np]
    es = [torch.from_numpy(g.standard_normal((sz, D)).astype(np.float32)).to(dev) for sz in sizes]
    outs = [torch.empty((sz, D), dtype=torch.float32, device=dev) for sz in sizes]
    evs = [torch.empty(sz, dtype=torch.int64, device=dev) for sz in sizes]
    sts = [torch.zeros(6, dtype=torch.int64, device=dev) for _ in sizes]
    pipe = pipeline.MemoryLayerPipeline(identity, stamps, values, P, n, depth=depth)
    pipe.prefetch(ids[0], 1, evicted=evs[0], stats=sts[0])
    for t in range(steps):
        if t + 1 < steps:
            pipe.prefetch(ids[t + 1], t + 2, evicted=evs[t + 1], stats=sts[t + 1])
        pipe.step(ids[t], t + 1, es[t], out=outs[t], evicted=evs[t], stats=sts[t])
    overflows = 0
    for t in range(steps):
        orows, ohit, oev, ost = o.step(ids_np[t], t + 1)
        assert bits_equal(to_np(outs[t]), o.gather(orows)), f"gather step {t}"
        o.writeback(orows, to_np(es[t]))
        assert np.array_equal(to_np(evs[t]), oev), f"evicted step {t}"
        assert np.array_equal(to_np(sts[t])[:5], ost), f"stats step {t}"
        overflows += int(ost[3])
    assert np.array_equal(to_np(identity), o.identity)
    assert np.array_equal(to_np(stamps), o.stamps)
    assert bits_equal(to_np(values), o.values)
    if C <= 256 and n > 100:
        assert overflows > 0  # the overflow path is exercised


@pytest.mark.parametrize("group,ahead,depth,steps", [(None, 1, 3, 6), (2, 1, 6, 6), (4, 2, 16, 6), (2, 2, 8, 9),
                                                     (4, 1, 12, 14)])
def test_step_graph_replays_match_oracle(dev, group, ahead, depth, steps):
    """A sequence of batches captured as one HIP graph (StepGraph: per-batch lookahead, or the grouped
    schedule, including ragged last groups whose slots were used before) and replayed three times, each
    time from the same restored state with eager work and synchronisation in between: every replay's
    gathered rows, evicted IDs, stats and final state equal the oracle's sequential result bit for bit.
    Eager batches then continue after the last replay."""
    cfg = synth.scaled_memory_layer(capacity=16_384, universe=120_000, batch=8_192, steps=steps)
    C, P, D, n = cfg.capacity, cfg.probes, cfg.dim, cfg.batch
    identity, stamps, o, base = prefilled_pair(dev, cfg)
    values = torch.zeros((C, D), dtype=torch.float32, device=dev)
    ids_np = synth.mpzch_stream(cfg, steps + 1)
    e_np = [synth.normal_rows_np(n, D, cfg.e_std, 2, t) for t in range(1, steps + 2)]
    ids = [torch.from_numpy(x).to(dev) for x in ids_np]
    es = [torch.from_numpy(x).to(dev) for x in e_np]
    expect = []
    for t in range(steps):
        orows, ohit, oev, ost = o.step(ids_np[t], base + t + 1)
        expect.append(o.gather(orows))
        o.writeback(orows, e_np[t])
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        snap = (identity.clone(), stamps.clone(), values.clone())
        outs = [torch.empty((n, D), dtype=torch.float32, device=dev) for _ in range(steps)]
        pipe = pipeline.MemoryLayerPipeline(identity, stamps, values, P, n, depth=depth)
        graph = pipeline.StepGraph(pipe, [(ids[t], base + t + 1, es[t], outs[t]) for t in range(steps)],
                                   ahead=ahead, group=group)
        for rep in range(3):
            identity.copy_(snap[0])
            stamps.copy_(snap[1])
            values.copy_(snap[2])
            for x in outs:
                x.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for t in range(steps):
                assert bits_equal(to_np(outs[t]), expect[t]), f"replay {rep} gather step {t}"
            assert np.array_equal(to_np(identity), o.identity), f"replay {rep} identity"
            assert np.array_equal(to_np(stamps), o.stamps), f"replay {rep} stamps"
            assert bits_equal(to_np(values), o.values), f"replay {rep} values"
        # an eager batch after the last replay
        out = pipe.step(ids[steps], base + steps + 1, es[steps])[0]
        torch.cuda.synchronize()
    orows, _, _, _ = o.step(ids_np[steps], base + steps + 1)
    assert bits_equal(to_np(out), o.gather(orows))
    o.writeback(orows, e_np[steps])
    assert bits_equal(to_np(values), o.values)


@pytest.mark.parametrize("group,ahead,steps", [(4, 1, 11), (2, 2, 9), (1, 1, 5), (3, 1, 3)])
def test_grouped_run_matches_oracle(dev, group, ahead, steps):
    """MemoryLayerPipeline.run: the lookup halves of a group of batches back to back, one cross-stream
    wait per stream per group, lookups `ahead` groups ahead, batches of varying size and a ragged last
    group.  Every batch's rows, hit mask, evicted IDs, stats and gathered rows, and the final state,
    equal the oracle's sequential result bit for bit; an eager batch then follows."""
    cfg = synth.scaled_memory_layer(capacity=16_384, universe=120_000, batch=8_192, steps=steps)
    C, P, D, n = cfg.capacity, cfg.probes, cfg.dim, cfg.batch
    identity, stamps, o, base = prefilled_pair(dev, cfg)
    values = torch.zeros((C, D), dtype=torch.float32, device=dev)
    ids_np = synth.mpzch_stream(cfg, steps + 1)
    ids_np = [x if t % 3 != 1 else x[: n - 777 * t] for t, x in enumerate(ids_np)]  # some smaller batches
    e_np = [synth.normal_rows_np(x.size, D, cfg.e_std, 2, t) for t, x in enumerate(ids_np, start=1)]
    ids = [torch.from_numpy(x).to(dev) for x in ids_np]
    es = [torch.from_numpy(x).to(dev) for x in e_np]
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        outs = [torch.full((x.size, D), float("nan"), dtype=torch.float32, device=dev) for x in ids_np[:steps]]
        evs = [torch.empty(x.size, dtype=torch.int64, device=dev) for x in ids_np[:steps]]
        sts = [torch.zeros(6, dtype=torch.int64, device=dev) for _ in range(steps)]
        rws = [torch.empty(x.size, dtype=torch.int64, device=dev) for x in ids_np[:steps]]
        hts = [torch.empty(x.size, dtype=torch.int8, device=dev) for x in ids_np[:steps]]
        pipe = pipeline.MemoryLayerPipeline(identity, stamps, values, P, n, depth=(ahead + 2) * group)
        pipe.run([(ids[t], base + t + 1, es[t], outs[t], evs[t], sts[t], rws[t], hts[t]) for t in range(steps)],
                 group=group, ahead=ahead)
        out = pipe.step(ids[steps], base + steps + 1, es[steps])[0]
        torch.cuda.synchronize()
    for t in range(steps):
        orows, ohit, oev, ost = o.step(ids_np[t], base + t + 1)
        assert np.array_equal(to_np(rws[t]), orows), f"rows batch {t}"
        assert np.array_equal(to_np(hts[t]), ohit), f"hit batch {t}"
        assert np.array_equal(to_np(evs[t]), oev), f"evicted batch {t}"
        s_ = to_np(sts[t])
        assert np.array_equal(s_[:5], ost) and s_[5] == 0, (t, s_, ost)
        assert bits_equal(to_np(outs[t]), o.gather(orows)), f"gather batch {t}"
        o.writeback(orows, e_np[t])
    orows, _, _, _ = o.step(ids_np[steps], base + steps + 1)  # the eager batch after run()
    assert bits_equal(to_np(out), o.gather(orows))
    o.writeback(orows, e_np[steps])
    assert np.array_equal(to_np(identity), o.identity)
    assert np.array_equal(to_np(stamps), o.stamps)
    assert bits_equal(to_np(values), o.values)


def test_grouped_run_argument_errors(dev):
    """run() refuses a ring depth that cannot hold (ahead + 2) groups, and lookahead left pending."""
    C, P, D, n = 1024, 8, 16, 64
    identity = torch.full((C,), -1, dtype=torch.int64, device=dev)
    stamps = torch.full((C,), -1, dtype=torch.int64, device=dev)
    values = torch.zeros((C, D), dtype=torch.float32, device=dev)
    pipe = pipeline.MemoryLayerPipeline(identity, stamps, values, P, n, depth=6)
    ids = torch.arange(n, dtype=torch.int64, device=dev)
    e = torch.zeros((n, D), dtype=torch.float32, device=dev)
    out = torch.empty((n, D), dtype=torch.float32, device=dev)
    with pytest.raises(hlr.HLRError):
        pipe.run([(ids, 1, e, out)], group=4)           # depth 6 < 3 groups of 4
    with pytest.raises(hlr.HLRError):
        pipe.run([(ids, 1, e, out)], group=2, ahead=2)  # depth 6 < 4 groups of 2
    pipe.prefetch(ids, 1)
    with pytest.raises(hlr.HLRError):
        pipe.run([(ids, 2, e, out)], group=2)
    pipe.step(ids, 1, e)
    pipe.run([(ids, 2, e, out)], group=2)
    torch.cuda.synchronize()
    assert int((identity >= 0).sum().item()) == n


def test_prefetch_limits(dev):
    """Lookahead is bounded by the ring depth and must be consumed in order (host-side errors)."""
    C, P, D, n = 1024, 8, 16, 64
    identity = torch.full((C,), -1, dtype=torch.int64, device=dev)
    stamps = torch.full((C,), -1, dtype=torch.int64, device=dev)
    values = torch.zeros((C, D), dtype=torch.float32, device=dev)
    pipe = pipeline.MemoryLayerPipeline(identity, stamps, values, P, n, depth=2)
    ids = [torch.arange(i * n, (i + 1) * n, dtype=torch.int64, device=dev) for i in range(4)]
    e = torch.zeros((n, D), dtype=torch.float32, device=dev)
    pipe.prefetch(ids[0], 1)
    pipe.prefetch(ids[1], 2)
    with pytest.raises(hlr.HLRError):
        pipe.prefetch(ids[2], 3)
    with pytest.raises(hlr.HLRError):
        pipe.step(ids[1], 2, e)
    pipe.step(ids[0], 1, e)
    pipe.step(ids[1], 2, e)
    torch.cuda.synchronize()
    assert int((identity >= 0).sum().item()) == 2 * n


@pytest.mark.parametrize("batch,group", [(True, 8), (True, 2), (False, 8)])
def test_hashed_tables_pipeline(dev, batch, group):
    g = np.random.default_rng(11)
    sizes, n, D, lr, steps = [5000, 700, 3000], 6000, 128, 0.01, 4
    tables_np = [(g.standard_normal((m, D)) * 0.01).astype(np.float32) for m in sizes]
    tables = [torch.from_numpy(x).to(dev) for x in tables_np]
    keys_np = [[(g.zipf(1.3, size=n) * 2654435761 % (1 << 40)).astype(np.int64) for _ in sizes]
               for _ in range(steps)]
    grads_np = [[(g.standard_normal((n, D)) * 1e-3).astype(np.float32) for _ in sizes] for _ in range(steps)]
    keys = [[torch.from_numpy(k).to(dev) for k in ks] for ks in keys_np]
    grads = [[torch.from_numpy(x).to(dev) for x in gs] for gs in grads_np]
    torch.cuda.synchronize()
    pipe = pipeline.HashedTablesPipeline(tables, n, batch=batch, group=group)
    assert pipe.batch == batch
    outs = [pipe.step(keys[s], grads[s], lr) for s in range(steps)]
    for s in range(steps):
        for i, m in enumerate(sizes):
            rows = oracle.hashed_rows(keys_np[s][i], m)
            assert bits_equal(to_np(outs[s][i]), oracle.gather(tables_np[i], rows)), (s, i)
            oracle.sgd_sum(tables_np[i], rows, grads_np[s][i], lr)
    for i in range(len(sizes)):
        assert bits_equal(to_np(tables[i]), tables_np[i]), i


@pytest.mark.parametrize("derive,lookup_streams,batch", [(True, 2, True), (True, 2, False), (True, 1, True),
                                                          (False, 2, True), (False, 1, False)])
def test_ema_pipeline(dev, derive, lookup_streams, batch):
    cfg = synth.CS3
    users, items, D, n = 4096, 8192, 128, 20_000
    g = np.random.default_rng(5)
    names = ["c_user", "c_item", "s_user", "s_item"]
    shapes = [users, items, users, items]
    cpu = [np.zeros((m, D), np.float32) for m in shapes]
    gpu = [torch.zeros((m, D), dtype=torch.float32, device=dev) for m in shapes]
    batches = []
    for step in range(3):
        u = np.minimum(synth.zipf_ranks(g, users, 1.1, n), users - 1).astype(np.int64)
        it = np.minimum(synth.zipf_ranks(g, items, 1.05, n), items - 1).astype(np.int64)
        y = (g.random(n) < 0.05).astype(np.uint8)
        v = [g.standard_normal((n, D)).astype(np.float32) for _ in range(3)]
        batches.append((u, it, y, v))
    dev_b = [tuple(torch.from_numpy(x).to(dev) for x in (u, it, y)) + ([torch.from_numpy(x).to(dev) for x in v],)
             for (u, it, y, v) in batches]
    torch.cuda.synchronize()
    pipe = pipeline.EMAPipeline(gpu, n, derive=derive, lookup_streams=lookup_streams, batch=batch)
    coeffs = [(cfg.cts_a, cfg.cts_b), (cfg.cts_a, cfg.cts_b), (cfg.cms_a, cfg.cms_b), (cfg.cms_a, cfg.cms_b)]
    for (ur, ir, yy, vv) in dev_b:
        pipe.step([ur, ir, ur, ir], [yy, yy, None, None], [vv[0], vv[1], vv[2], vv[2]], coeffs)
    for (u, it, y, v) in batches:
        oracle.ema(cpu[0], u, v[0], y, cfg.cts_a, cfg.cts_b)
        oracle.ema(cpu[1], it, v[1], y, cfg.cts_a, cfg.cts_b)
        oracle.ema(cpu[2], u, v[2], None, cfg.cms_a, cfg.cms_b)
        oracle.ema(cpu[3], it, v[2], None, cfg.cms_a, cfg.cms_b)
    for k, name in enumerate(names):
        assert bits_equal(to_np(gpu[k]), cpu[k]), name


@pytest.mark.parametrize("group,ahead,lookup_streams,derive", [(4, 1, 2, True), (2, 2, 2, True), (3, 1, 1, False),
                                                               (1, 1, 2, True)])
def test_ema_grouped_run_matches_oracle(dev, group, ahead, lookup_streams, derive):
    """EMAPipeline.run() (plans a group ahead, one wait per stream and group) between step() calls: every
    table bit-equal to the oracle's batch-order EMA after all batches (CS3 page, sec. 2), with a last
    group shorter than the others and batches of different sizes."""
    _ema_grouped(dev, group, ahead, lookup_streams, derive, graph=False)


@pytest.mark.parametrize("group,ahead,lookup_streams,derive", [(2, 2, 2, True), (4, 1, 2, False)])
def test_ema_run_graph_matches_oracle(dev, group, ahead, lookup_streams, derive):
    """The same grouped schedule captured as one HIP graph (RunGraph, every lookup stream joined back) and
    replayed once between step() calls: every table bit-equal to the oracle's batch-order EMA."""
    _ema_grouped(dev, group, ahead, lookup_streams, derive, graph=True)


def _ema_grouped(dev, group, ahead, lookup_streams, derive, graph):
    cfg = synth.CS3
    users, items, D, n = 4096, 8192, 128, 12_000
    g = np.random.default_rng(17 + group)
    shapes = [users, items, users, items]
    cpu = [np.zeros((m, D), np.float32) for m in shapes]
    gpu = [torch.zeros((m, D), dtype=torch.float32, device=dev) for m in shapes]
    batches = []
    for s in range(12):
        m = n - 1000 * (s % 3)
        u = np.minimum(synth.zipf_ranks(g, users, 1.1, m), users - 1).astype(np.int64)
        it = np.minimum(synth.zipf_ranks(g, items, 1.05, m), items - 1).astype(np.int64)
        y = (g.random(m) < 0.05).astype(np.uint8)
        v = [g.standard_normal((m, D)).astype(np.float32) for _ in range(3)]
        batches.append((u, it, y, v))
    dev_b = [tuple(torch.from_numpy(x).to(dev) for x in (u, it, y)) + ([torch.from_numpy(x).to(dev) for x in v],)
             for (u, it, y, v) in batches]
    torch.cuda.synchronize()
    depth = (ahead + 2) * group
    coeffs = [(cfg.cts_a, cfg.cts_b), (cfg.cts_a, cfg.cts_b), (cfg.cms_a, cfg.cms_b), (cfg.cms_a, cfg.cms_b)]

    def args(b):
        ur, ir, yy, vv = b
        return [ur, ir, ur, ir], [yy, yy, None, None], [vv[0], vv[1], vv[2], vv[2]], coeffs

    side = torch.cuda.Stream(dev)  # a graph cannot be captured on the legacy default stream
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        pipe = pipeline.EMAPipeline(gpu, n, depth=depth, derive=derive, lookup_streams=lookup_streams)
        pipe.step(*args(dev_b[0]))
        pipe.step(*args(dev_b[1]))
        if graph:
            g = pipeline.RunGraph(pipe, [args(b) for b in dev_b[2:11]], group=group, ahead=ahead)
            g.replay()
        else:
            pipe.run([args(b) for b in dev_b[2:11]], group=group, ahead=ahead)
        pipe.step(*args(dev_b[11]))
        torch.cuda.synchronize()
    for (u, it, y, v) in batches:
        oracle.ema(cpu[0], u, v[0], y, cfg.cts_a, cfg.cts_b)
        oracle.ema(cpu[1], it, v[1], y, cfg.cts_a, cfg.cts_b)
        oracle.ema(cpu[2], u, v[2], None, cfg.cms_a, cfg.cms_b)
        oracle.ema(cpu[3], it, v[2], None, cfg.cms_a, cfg.cms_b)
    for k in range(4):
        assert bits_equal(to_np(gpu[k]), cpu[k]), k


def test_ema_grouped_run_argument_errors(dev):
    """run() needs the batched apply and a ring that holds (ahead + 2) groups (host-side errors)."""
    D, n = 16, 64
    tabs = [torch.zeros((256, D), dtype=torch.float32, device=dev) for _ in range(2)]
    rows = torch.arange(n, dtype=torch.int64, device=dev)
    vals = torch.zeros((n, D), dtype=torch.float32, device=dev)
    b = ([rows, rows], [None, None], [vals, vals], [(0.5, 0.5), (0.5, 0.5)])
    with pytest.raises(hlr.HLRError):
        pipeline.EMAPipeline(tabs, n, depth=6).run([b], group=4)
    with pytest.raises(hlr.HLRError):
        pipeline.EMAPipeline(tabs, n, depth=12, batch=False).run([b], group=4)
    with pytest.raises(hlr.HLRError):
        pipeline.EMAPipeline(tabs, n, depth=12).run([([rows], [None], [vals], [(0.5, 0.5)])], group=4)
    pipe = pipeline.EMAPipeline(tabs, n, depth=12)
    pipe.run([b, b], group=4)
    torch.cuda.synchronize()
    assert bool((tabs[0][:n] == 0).all().item())


@pytest.mark.parametrize("derive,group", [(True, 4), (False, 2), (True, 1)])
def test_ema_pairs_pipeline_matches_oracle(dev, derive, group):
    """EMAPipeline(pairs=True): the user- and item-keyed updates of each rule planned by one sort (the CTS
    pair cut out of the CMS pair's plan when derive), all pairs applied by one launch, through step() and
    the grouped run(); every table bit-equal to the oracle's batch-order EMA (CS3 page, sec. 2)."""
    cfg = synth.CS3
    users, items, D, n = 4096, 8192, 128, 12_000
    g = np.random.default_rng(29 + group)
    shapes = [users, items, users, items]
    cpu = [np.zeros((m, D), np.float32) for m in shapes]
    gpu = [torch.zeros((m, D), dtype=torch.float32, device=dev) for m in shapes]
    batches = []
    for s in range(10):
        m = n - 700 * (s % 3)
        u = np.minimum(synth.zipf_ranks(g, users, 1.1, m), users - 1).astype(np.int64)
        it = np.minimum(synth.zipf_ranks(g, items, 1.05, m), items - 1).astype(np.int64)
        y = (g.random(m) < 0.05).astype(np.uint8)
        v = [g.standard_normal((m, D)).astype(np.float32) for _ in range(3)]
        batches.append((u, it, y, v))
    dev_b = [tuple(torch.from_numpy(x).to(dev) for x in (u, it, y)) + ([torch.from_numpy(x).to(dev) for x in v],)
             for (u, it, y, v) in batches]
    torch.cuda.synchronize()
    pipe = pipeline.EMAPipeline(gpu, n, depth=3 * group, derive=derive, pairs=True)
    coeffs = [(cfg.cts_a, cfg.cts_b), (cfg.cts_a, cfg.cts_b), (cfg.cms_a, cfg.cms_b), (cfg.cms_a, cfg.cms_b)]

    def args(b):
        ur, ir, yy, vv = b
        return [ur, ir, ur, ir], [yy, yy, None, None], [vv[0], vv[1], vv[2], vv[2]], coeffs

    pipe.step(*args(dev_b[0]))
    pipe.run([args(b) for b in dev_b[1:9]], group=group, ahead=1)
    pipe.step(*args(dev_b[9]))
    for (u, it, y, v) in batches:
        oracle.ema(cpu[0], u, v[0], y, cfg.cts_a, cfg.cts_b)
        oracle.ema(cpu[1], it, v[1], y, cfg.cts_a, cfg.cts_b)
        oracle.ema(cpu[2], u, v[2], None, cfg.cms_a, cfg.cms_b)
        oracle.ema(cpu[3], it, v[2], None, cfg.cms_a, cfg.cms_b)
    for k in range(4):
        assert bits_equal(to_np(gpu[k]), cpu[k]), k
    with pytest.raises(hlr.HLRError):  # the two updates of a pair share their mask
        ur, ir, yy, vv = dev_b[0]
        pipe.step([ur, ir, ur, ir], [yy, None, None, None], [vv[0], vv[1], vv[2], vv[2]], coeffs)
