"""GPU parity of the publishing side (Raw Embedding Streaming): int8 row quantisation, the
written-row set, the distinct rows of a Writeback plan, and the RESPublisher schedule, against
the oracle (quantisation) and numpy set operations (row sets, whose order is unspecified)."""
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


@pytest.mark.parametrize("C,D,n", [(5000, 512, 3000), (300, 128, 1000), (64, 1024, 64), (40, 8, 77)])
def test_quantize_compact_matches_oracle(dev, C, D, n):
    g = np.random.default_rng(C + D)
    table = (g.standard_normal((C, D)) * g.uniform(1e-3, 50, size=(C, 1))).astype(np.float32)
    table[1] = 2.5  # a constant row
    rows = g.integers(-1, C, size=n).astype(np.int64)
    rows[:3] = [1, -1, 1]
    q, sc, bi = hlr.quantize_rows_int8(torch.from_numpy(table).to(dev), torch.from_numpy(rows).to(dev))
    oq, osc, obi = oracle.quantize_rows(table, rows)
    assert np.array_equal(to_np(q), oq)
    assert bits_equal(to_np(sc), osc) and bits_equal(to_np(bi), obi)


def test_quantize_scatter_and_count(dev):
    g = np.random.default_rng(5)
    C, D, n = 2000, 256, 900
    table = g.standard_normal((C, D)).astype(np.float32)
    rows = g.permutation(C)[:n].astype(np.int64)
    rows[10] = -1
    t, r = torch.from_numpy(table).to(dev), torch.from_numpy(rows).to(dev)
    q, sc, bi = hlr.quantize_rows_int8(t, r, scatter=True)
    oq, osc, obi = oracle.quantize_rows(table, rows, scatter=True)
    assert np.array_equal(to_np(q), oq) and bits_equal(to_np(sc), osc) and bits_equal(to_np(bi), obi)
    cnt = torch.tensor([123], dtype=torch.int64, device=dev)
    q, sc, bi = hlr.quantize_rows_int8(t, r, count=cnt)
    oq, osc, obi = oracle.quantize_rows(table, rows, count=123)
    assert np.array_equal(to_np(q), oq) and bits_equal(to_np(sc), osc) and bits_equal(to_np(bi), obi)


def test_mark_rows_and_clear(dev):
    g = np.random.default_rng(6)
    C = 10_000
    flags = torch.zeros(C, dtype=torch.int32, device=dev)
    lst = torch.empty(C, dtype=torch.int64, device=dev)
    cnt = torch.zeros(1, dtype=torch.int64, device=dev)
    seen = set()
    for step in range(5):
        rows = g.integers(-1, C, size=4000).astype(np.int64)
        rows[:100] = 7  # repeats within and across calls
        hlr.mark_rows(torch.from_numpy(rows).to(dev), C, flags, lst, cnt)
        seen |= set(rows[rows >= 0].tolist())
        c = int(to_np(cnt)[0])
        got = to_np(lst)[:c]
        assert c == len(seen) and len(set(got.tolist())) == c and set(got.tolist()) == seen
    hlr.clear_marks(lst, cnt, C, flags)
    assert int(to_np(cnt)[0]) == 0 and not to_np(flags).any()
    limit = torch.tensor([10], dtype=torch.int64, device=dev)
    hlr.mark_rows(torch.arange(50, dtype=torch.int64, device=dev), C, flags, lst, cnt, count=limit)
    assert sorted(to_np(lst)[:int(to_np(cnt)[0])].tolist()) == list(range(10))


def test_writeback_plan_rows(dev):
    g = np.random.default_rng(7)
    C, n = 3000, 20_000
    rows = g.integers(-1, C, size=n).astype(np.int64)
    rows[g.random(n) < 0.3] = 17
    r = torch.from_numpy(rows).to(dev)
    ws = hlr.new_workspace(dev, hlr.writeback_workspace_size(C, 64, n, hlr.WB_LAST_WINS))
    hlr.writeback_plan(C, r, ws, hlr.WB_LAST_WINS)
    out, cnt = hlr.writeback_plan_rows(C, n, ws)
    c = int(to_np(cnt)[0])
    got = to_np(out)[:c]
    want = np.unique(rows[rows >= 0])
    assert c == want.size and np.array_equal(np.sort(got), want)


@pytest.mark.parametrize("native", [True, False])
def test_res_publisher_schedule(dev, native):
    """Memory-Layer batches through the two-stream pipeline with a publish every 3 batches: each
    publish carries exactly the rows written since the previous one, quantised from the table as it
    is after that batch, and identity/stamps as they are after that batch's lookup.  native: the batch
    runs as the one-call step's two halves and its written rows come from the step's row grouping
    (memory_layer_step_mark_written); else call by call, the rows from the Writeback plan."""
    cfg = synth.scaled_memory_layer(capacity=8_192, universe=60_000, batch=4_096, steps=10, dim=64)
    C, P, D, n = cfg.capacity, cfg.probes, cfg.dim, cfg.batch
    identity = torch.full((C,), -1, dtype=torch.int64, device=dev)
    stamps = torch.full((C,), -1, dtype=torch.int64, device=dev)
    o = oracle.MPZCHTable(C, P, D, with_values=False)
    for k, b in enumerate(synth.prefill_batches(cfg), start=1):
        hlr.mpzch_lookup_or_insert(identity, stamps, None, P, torch.from_numpy(b).to(dev), k)
        o.step(b, k)
    base = len(synth.prefill_batches(cfg))
    o.values = np.zeros((C, D), np.float32)
    values = torch.zeros((C, D), dtype=torch.float32, device=dev)
    ids_np = synth.mpzch_stream(cfg, cfg.steps)
    e_np = [synth.normal_rows_np(n, D, cfg.e_std, 2, t) for t in range(1, cfg.steps + 1)]
    ids = [torch.from_numpy(x).to(dev) for x in ids_np]
    es = [torch.from_numpy(x).to(dev) for x in e_np]
    torch.cuda.synchronize()
    packets = []
    pipe = pipeline.MemoryLayerPipeline(identity, stamps, values, P, n, native=native)
    pub = pipeline.RESPublisher(pipe, every=3, on_publish=packets.append)
    for t in range(cfg.steps):
        pipe.step(ids[t], base + t + 1, es[t], publisher=pub)
    pub.publish_now(pipe)  # the rows of batch 9, written after the last periodic publish
    pub.flush()
    torch.cuda.synchronize()
    assert [p["step"] for p in packets] == [2, 5, 8, 9]
    written, states = set(), {}
    for t in range(cfg.steps):
        orows, _, _, _ = o.step(ids_np[t], base + t + 1)
        o.writeback(orows, e_np[t])
        written |= set(orows[orows >= 0].tolist())
        if (t + 1) % 3 == 0 or t == cfg.steps - 1:
            states[t] = (written, o.values.copy(), o.identity.copy(), o.stamps.copy())
            written = set()
    for p in packets:
        want_rows, vals, ident, stmp = states[p["step"]]
        assert len(p["rows"]) == len(want_rows) and set(p["rows"].tolist()) == want_rows
        oq, osc, obi = oracle.quantize_rows(vals, p["rows"])
        assert np.array_equal(p["q"], oq) and bits_equal(p["scale"], osc) and bits_equal(p["bias"], obi)
        assert np.array_equal(p["identity"], ident) and np.array_equal(p["stamps"], stmp)
