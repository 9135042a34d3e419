"""The allocation-free MPZCH entry point (mpzch_lookup_or_insert_static, scratch in a device array
inside the library) against the workspace entry point, through the C ABI: two calls in a row, the
second with a smaller batch, every output and the table state bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import hashed_lookup_row_amd as hlr
import synth

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hlr.load_library()
    return torch.device("cuda:0")


class Table:
    def __init__(self, dev, C, D, seed):
        g = np.random.default_rng(seed)
        self.identity = torch.full((C,), -1, dtype=torch.int64, device=dev)
        self.stamps = torch.full((C,), -1, dtype=torch.int64, device=dev)
        self.values = torch.from_numpy(g.standard_normal((C, D)).astype(np.float32)).to(dev)


def test_static_entry_point_matches_workspace_entry_point(dev):
    lib = hlr.load_library()
    C, P, D = 1 << 16, 8, 64
    assert lib.mpzch_lookup_or_insert_static_max_n() == 262144
    a, b = Table(dev, C, D, 5), Table(dev, C, D, 5)
    s = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    g = np.random.default_rng(11)
    universe = g.choice(1 << 50, size=300_000, replace=False).astype(np.int64)
    for call, n in enumerate([200_000, 5_000]):  # the second call smaller than the first
        ids_np = universe[np.minimum(synth.zipf_ranks(g, universe.size, 1.05, n), universe.size - 1)]
        ids_np[g.random(n) < 0.01] = -1
        ids = torch.from_numpy(ids_np).to(dev)
        out = {}
        for name, t in (("static", a), ("ws", b)):
            rows = torch.empty(n, dtype=torch.int64, device=dev)
            hit = torch.empty(n, dtype=torch.int8, device=dev)
            ev = torch.empty(n, dtype=torch.int64, device=dev)
            st = torch.zeros(6, dtype=torch.int64, device=dev)
            args = (_p(t.identity), _p(t.stamps), _p(t.values), C, P, D, _p(ids), n, call + 1, 1, _p(rows), _p(hit),
                    _p(ev), _p(st))
            if name == "static":
                rc = lib.mpzch_lookup_or_insert_static(*args, s)
            else:
                need = lib.mpzch_lookup_or_insert_workspace_size(n, 1)
                ws = torch.empty(need + 256, dtype=torch.uint8, device=dev)
                base = (ws.data_ptr() + 255) // 256 * 256
                rc = lib.mpzch_lookup_or_insert(*args, ctypes.c_void_p(base), need, s)
            assert rc == 0, (name, rc)
            torch.cuda.synchronize()
            out[name] = [x.cpu().numpy() for x in (rows, hit, ev, st)]
        for x, y, what in zip(out["static"], out["ws"], ("rows", "hit", "evicted", "stats")):
            assert np.array_equal(x, y), f"call {call}: {what}"
        assert out["static"][3][1] > 0  # inserts happen
        for x, y, what in ((a.identity, b.identity, "identity"), (a.stamps, b.stamps, "stamps"),
                           (a.values, b.values, "values")):
            assert torch.equal(x, y), f"call {call}: {what}"
