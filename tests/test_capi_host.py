"""Host-side checks of the C ABI (CPU only: no kernel is launched).

The library must load, export every entry point include/hlr.h declares, and
reject host-checkable faults with the documented status before enqueueing
anything.
"""
import ctypes
import os
import re

import pytest

import hashed_lookup_row_amd as hlr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hlr.h")

OK, INVALID, DIM, MISALIGNED, WS_SMALL = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hlr.LIB_PATH):
        pytest.fail("libhlr.so is not built (run __graft_entry__.build())")
    return hlr.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w[\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)) - {"defined"})


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 13, names
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(hlr.exported_symbols())


def test_status_strings_and_version(lib):
    for code, s in hlr.STATUS.items():
        assert lib.hlr_status_string(code).decode() == s
    assert lib.hlr_status_string(99).decode() == "unknown status"
    assert lib.hlr_version() >= 100


def test_workspace_sizes_are_host_only_and_monotone(lib):
    assert lib.mpzch_lookup_or_insert_workspace_size(1000, 0) == 0
    a = lib.mpzch_lookup_or_insert_workspace_size(1000, 1)
    b = lib.mpzch_lookup_or_insert_workspace_size(65536, 1)
    assert 0 < a < b and b % 256 == 0
    assert lib.dedup_ids_workspace_size(65536) > lib.dedup_ids_workspace_size(100) > 0
    assert lib.writeback_rows_workspace_size(1 << 22, 512, 65536, 0) > 0
    assert lib.writeback_rows_workspace_size(1 << 22, 512, 65536, 1) > 0
    assert lib.ema_update_rows_workspace_size(1 << 20, 128, 262144) > 0


P16 = ctypes.c_void_p(1 << 20)       # 16-byte aligned stand-in address (never dereferenced)
P_ODD = ctypes.c_void_p((1 << 20) + 4)


def test_gather_argument_errors(lib):
    s = None
    assert lib.gather_rows(P16, 10, 3, P16, 5, P16, s) == DIM
    assert lib.gather_rows(P16, 10, 0, P16, 5, P16, s) == DIM
    assert lib.gather_rows(P16, 10, 8, P16, -1, P16, s) == INVALID
    assert lib.gather_rows(P16, 10, 8, None, 5, P16, s) == INVALID
    assert lib.gather_rows(P_ODD, 10, 8, P16, 5, P16, s) == MISALIGNED
    assert lib.gather_rows(P16, 10, 8, P16, 0, P16, s) == OK  # n == 0: nothing to do


def test_mpzch_argument_errors(lib):
    s = None
    args = lambda cap, probes, n, ins, ws, wsb: lib.mpzch_lookup_or_insert(
        P16, P16, None, cap, probes, 0, P16, n, 5, ins, P16, P16, None, None, ws, wsb, s)
    assert args(100, 8, 10, 1, None, 0) == INVALID  # capacity % probes != 0
    assert args(64, 0, 10, 1, None, 0) == INVALID
    assert args(64, 33, 10, 1, None, 0) == INVALID
    assert args(64, 8, -3, 1, None, 0) == INVALID
    assert args(64, 8, 10, 2, None, 0) == INVALID
    assert args(64, 8, 10, 1, None, 0) == WS_SMALL
    need = lib.mpzch_lookup_or_insert_workspace_size(10, 1)
    assert args(64, 8, 10, 1, P16, need - 1) == WS_SMALL
    assert args(64, 8, 10, 1, ctypes.c_void_p((1 << 20) + 16), need) == MISALIGNED
    # values given with a dim that is not a multiple of 4
    assert lib.mpzch_lookup_or_insert(P16, P16, P16, 64, 8, 6, P16, 10, 5, 1, P16, P16, None, None, P16, need,
                                      s) == DIM


def test_writeback_and_ema_argument_errors(lib):
    s = None
    need = lib.writeback_rows_workspace_size(100, 8, 10, 0)
    assert lib.writeback_rows(P16, 100, 8, P16, P16, 10, 0, 0.5, P16, need, s) == INVALID  # last-wins needs lr=1
    assert lib.writeback_rows(P16, 100, 8, P16, P16, 10, 7, 1.0, P16, need, s) == INVALID  # unknown mode
    assert lib.writeback_rows(P16, 100, 6, P16, P16, 10, 0, 1.0, P16, need, s) == DIM
    assert lib.writeback_rows(P16, 100, 8, P16, P16, 10, 0, 1.0, None, 0, s) == WS_SMALL
    assert lib.writeback_rows(P16, 100, 8, P16, P_ODD, 10, 1, 0.1, P16, 1 << 30, s) == MISALIGNED
    assert lib.ema_update_rows(P16, 100, 2048, P16, P16, None, 10, 0.9, 0.1, P16, 1 << 30, s) == DIM
    assert lib.ema_update_rows(P16, 100, 8, P16, P16, None, 10, 0.9, 0.1, None, 0, s) == WS_SMALL


def test_split_entry_point_argument_errors(lib):
    s = None
    need = lib.writeback_rows_workspace_size(100, 8, 10, 1)
    assert lib.writeback_plan(100, P16, 10, 7, P16, need, s) == INVALID  # unknown mode
    assert lib.writeback_plan(100, P16, -1, 0, P16, need, s) == INVALID
    assert lib.writeback_plan(100, None, 10, 1, P16, need, s) == INVALID
    assert lib.writeback_plan(100, P16, 10, 1, None, 0, s) == WS_SMALL
    assert lib.writeback_plan(100, P16, 0, 1, None, 0, s) == OK  # nothing to plan
    assert lib.writeback_apply(P16, 100, 8, P16, 10, 0, 0.5, P16, need, s) == INVALID  # last-wins needs lr=1
    assert lib.writeback_apply(P16, 100, 6, P16, 10, 1, 0.1, P16, need, s) == DIM
    assert lib.writeback_apply(P16, 100, 8, P_ODD, 10, 1, 0.1, P16, need, s) == MISALIGNED
    assert lib.writeback_apply(P16, 100, 8, P16, 10, 1, 0.1, P16, need - 1, s) == WS_SMALL
    eneed = lib.ema_update_rows_workspace_size(100, 8, 10)
    assert lib.ema_update_plan(100, P16, None, -5, P16, eneed, s) == INVALID
    assert lib.ema_update_plan(100, P_ODD, None, 10, P16, eneed, s) == MISALIGNED
    assert lib.ema_update_plan(100, P16, None, 10, ctypes.c_void_p((1 << 20) + 16), eneed, s) == MISALIGNED
    assert lib.ema_update_apply(P16, 100, 2048, P16, 10, 0.9, 0.1, P16, eneed, s) == DIM
    assert lib.ema_update_apply(P16, 100, 8, P16, 10, 0.9, 0.1, None, 0, s) == WS_SMALL
    assert lib.mpzch_zero_inserted(P16, 64, 6, P16, P16, 10, s) == DIM
    assert lib.mpzch_zero_inserted(P16, 0, 8, P16, P16, 10, s) == INVALID
    assert lib.mpzch_zero_inserted(P16, 64, 8, None, P16, 10, s) == INVALID
    assert lib.mpzch_zero_inserted(P_ODD, 64, 8, P16, P16, 10, s) == MISALIGNED


def test_ema_apply_batch_argument_errors(lib):
    """Every host-checkable fault of the batched apply returns before anything is enqueued."""
    class Up(ctypes.Structure):
        _fields_ = [("table", ctypes.c_void_p), ("num_rows", ctypes.c_int64), ("dim", ctypes.c_int64),
                    ("vals", ctypes.c_void_p), ("n", ctypes.c_int64), ("a", ctypes.c_float), ("b", ctypes.c_float),
                    ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t)]
    s = None
    need = lib.ema_update_rows_workspace_size(100, 8, 10)
    base = 1 << 30  # stand-in addresses, far apart (never dereferenced)

    def up(k, dim=8, table=None, ws=None, wsb=need, n=10, num_rows=100):
        return Up(table if table is not None else base + k * (1 << 24), num_rows, dim, base + (1 << 28) + k * (1 << 24),
                  n, 0.9, 0.1, ws if ws is not None else base + (1 << 29) + k * (1 << 24), wsb)

    def call(*ups, count=None):
        arr = (Up * max(1, len(ups)))(*ups)
        return lib.ema_update_apply_batch(len(ups) if count is None else count, ctypes.cast(arr, ctypes.c_void_p), s)
    assert call(up(0), up(1), up(2), up(3), up(4)) == INVALID             # at most four
    assert call(up(0), count=-1) == INVALID
    assert lib.ema_update_apply_batch(2, None, s) == INVALID
    assert call(up(0), up(1, dim=16, wsb=lib.ema_update_rows_workspace_size(100, 16, 10))) == INVALID  # one dim
    assert call(up(0), up(1, table=base)) == INVALID                      # same table
    assert call(up(0), up(1, ws=base + (1 << 29))) == INVALID             # same workspace
    assert call(up(0), up(1, dim=6)) == DIM
    assert call(up(0), up(1, wsb=need - 1)) == WS_SMALL
    assert call(up(0, n=-1)) == INVALID
    assert call(up(0, table=base + 4)) == MISALIGNED
    assert call(up(0, n=0), up(1, num_rows=0)) == OK                      # nothing to do
    assert lib.ema_update_apply_batch(0, None, s) == OK


def test_mark_written_argument_errors(lib):
    """memory_layer_step_mark_written checks its sizes and pointers before enqueueing anything."""
    s = None
    need = lib.memory_layer_step_workspace_size(1000, 4096)
    ws, f, l, c = (ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 24), ctypes.c_void_p(1 << 25),
                   ctypes.c_void_p(1 << 26))
    call = lambda n=100, n_max=1000, ws=ws, wsb=need, cap=4096, f=f, l=l, c=c: \
        lib.memory_layer_step_mark_written(ws, wsb, n, n_max, cap, f, l, c, s)
    assert call(n=1001) == INVALID
    assert call(n=-1) == INVALID
    assert call(cap=0) == INVALID
    assert call(f=None) == INVALID
    assert call(ws=ctypes.c_void_p((1 << 20) + 64)) == MISALIGNED
    assert call(c=ctypes.c_void_p((1 << 26) + 4)) == MISALIGNED
    assert call(wsb=need - 1) == WS_SMALL
    assert call(n=0) == OK


def test_ema_pair_argument_errors(lib):
    """Every host-checkable fault of the EMA pair plans returns before anything is enqueued."""
    class Pair(ctypes.Structure):
        _fields_ = [("table0", ctypes.c_void_p), ("num_rows0", ctypes.c_int64), ("vals0", ctypes.c_void_p),
                    ("table1", ctypes.c_void_p), ("num_rows1", ctypes.c_int64), ("vals1", ctypes.c_void_p),
                    ("dim", ctypes.c_int64), ("n", ctypes.c_int64), ("a", ctypes.c_float), ("b", ctypes.c_float),
                    ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t)]
    s = None
    P16 = ctypes.c_void_p(1 << 20)
    P_ODD = ctypes.c_void_p((1 << 20) + 4)
    # sizes: the joint key range must leave room for the sentinel, 2n must fit the batch limit
    assert lib.ema_update_pair_workspace_size(100, 50, 8, 10) == lib.ema_update_rows_workspace_size(150, 8, 20)
    assert lib.ema_update_pair_workspace_size(1 << 30, 1 << 30, 8, 10) == 0
    assert lib.ema_update_pair_workspace_size(-1, 5, 8, 10) == 0
    need = lib.ema_update_pair_workspace_size(100, 50, 4, 10)
    plan = lambda r0=P16, r1=P16, n=10, ws=P16, wsb=need, nr0=100, nr1=50: lib.ema_update_plan_pair(
        nr0, r0, nr1, r1, None, n, ws, wsb, s)
    assert plan(r1=None) == INVALID
    assert plan(r0=P_ODD) == MISALIGNED
    assert plan(ws=ctypes.c_void_p((1 << 20) + 16)) == MISALIGNED
    assert plan(wsb=need - 1) == WS_SMALL
    assert plan(n=-1) == INVALID
    assert plan(nr0=1 << 30, nr1=1 << 30) == INVALID
    assert plan(n=0) == OK                                               # nothing to do
    base = 1 << 30
    wneed = lib.ema_update_pair_workspace_size(100, 50, 8, 10)

    def pr(k, dim=8, t0=None, t1=None, ws=None, wsb=wneed):
        return Pair(t0 if t0 is not None else base + k * (1 << 24), 100, base + (1 << 27) + k * (1 << 24),
                    t1 if t1 is not None else base + (1 << 26) + k * (1 << 24), 50,
                    base + (1 << 27) + (1 << 26) + k * (1 << 24), dim, 10, 0.9, 0.1,
                    ws if ws is not None else base + (1 << 29) + k * (1 << 24), wsb)

    def call(*ps, count=None):
        arr = (Pair * max(1, len(ps)))(*ps)
        return lib.ema_update_apply_pairs(len(ps) if count is None else count, ctypes.cast(arr, ctypes.c_void_p), s)
    assert call(*(pr(k) for k in range(5))) == INVALID                  # at most four
    assert lib.ema_update_apply_pairs(1, None, s) == INVALID
    assert call(pr(0, t1=base)) == INVALID                               # one table twice in a pair
    assert call(pr(0), pr(1, t0=base + (1 << 26))) == INVALID            # a table shared between pairs
    assert call(pr(0), pr(1, ws=base + (1 << 29))) == INVALID            # a workspace shared between pairs
    assert call(pr(0, dim=6)) == DIM
    assert call(pr(0), pr(1, dim=16, wsb=lib.ema_update_pair_workspace_size(100, 50, 16, 10))) == INVALID
    assert call(pr(0, wsb=wneed - 1)) == WS_SMALL
    assert call(pr(0, t1=base + (1 << 26) + 8)) == MISALIGNED
    assert lib.ema_update_apply_pairs(0, None, s) == OK


def test_wb_apply_batch_argument_errors(lib):
    """Every host-checkable fault of the batched SGD apply returns before anything is enqueued."""
    class Up(ctypes.Structure):
        _fields_ = [("table", ctypes.c_void_p), ("num_rows", ctypes.c_int64), ("dim", ctypes.c_int64),
                    ("src", ctypes.c_void_p), ("n", ctypes.c_int64), ("lr", ctypes.c_float),
                    ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t)]
    s, SGD, L2 = None, 1, 2
    need = lib.writeback_rows_workspace_size(100, 8, 10, SGD)
    base = 1 << 30  # stand-in addresses, far apart (never dereferenced)

    def up(k, dim=8, table=None, ws=None, wsb=need, n=10, num_rows=100):
        return Up(table if table is not None else base + k * (1 << 24), num_rows, dim, base + (1 << 28) + k * (1 << 24),
                  n, 0.5, ws if ws is not None else base + (1 << 29) + k * (1 << 24), wsb)

    def call(*ups, count=None, mode=SGD):
        arr = (Up * max(1, len(ups)))(*ups)
        return lib.writeback_apply_batch(len(ups) if count is None else count, ctypes.cast(arr, ctypes.c_void_p),
                                         mode, s)
    assert call(*[up(k) for k in range(9)]) == INVALID                   # at most eight
    assert call(up(0), count=-1) == INVALID
    assert lib.writeback_apply_batch(2, None, SGD, s) == INVALID
    assert call(up(0), mode=0) == INVALID                                 # LAST_WINS has no batch
    assert call(up(0), up(1, dim=16, wsb=lib.writeback_rows_workspace_size(100, 16, 10, SGD))) == INVALID
    assert call(up(0), up(1, table=base)) == INVALID                      # same table
    assert call(up(0), up(1, ws=base + (1 << 29))) == INVALID             # same workspace
    assert call(up(0), up(1, dim=6)) == DIM
    assert call(up(0), up(1, wsb=need - 1)) == WS_SMALL
    assert call(up(0, n=-1)) == INVALID
    assert call(up(0, table=base + 4)) == MISALIGNED
    assert call(up(0, n=0), up(1, num_rows=0), mode=L2) == OK             # nothing to do
    assert lib.writeback_apply_batch(0, None, SGD, s) == OK


def test_ema_plan_subset_argument_errors(lib):
    s = None
    need = lib.ema_update_rows_workspace_size(100, 4, 10)
    other = ctypes.c_void_p(1 << 40)  # a second stand-in workspace, far from P16 (never dereferenced)
    call = lambda mask=P16, n=10, src=P16, srcb=need, ws=other, wsb=need: lib.ema_update_plan_subset(
        100, mask, n, src, srcb, ws, wsb, s)
    assert call(mask=None) == INVALID
    assert call(ws=P16) == INVALID                                   # the two plans overlap
    assert call(ws=ctypes.c_void_p((1 << 20) + need - 256)) == INVALID
    assert call(srcb=need - 1) == WS_SMALL
    assert call(wsb=need - 1) == WS_SMALL
    assert call(src=None, srcb=0) == WS_SMALL
    assert call(src=ctypes.c_void_p((1 << 20) + 16)) == MISALIGNED
    assert call(n=-1) == INVALID
    assert call(n=0, src=None, srcb=0, ws=None, wsb=0) == OK        # nothing to plan


def test_publishing_entry_point_argument_errors(lib):
    s = None
    assert lib.quantize_rows_int8(P16, 10, 6, P16, 5, None, 0, P16, P16, P16, s) == DIM
    assert lib.quantize_rows_int8(P16, 10, 2048, P16, 5, None, 0, P16, P16, P16, s) == DIM
    assert lib.quantize_rows_int8(P16, 10, 8, P16, 5, None, 2, P16, P16, P16, s) == INVALID  # scatter flag
    assert lib.quantize_rows_int8(P16, 10, 8, P16, -5, None, 0, P16, P16, P16, s) == INVALID
    assert lib.quantize_rows_int8(P16, 10, 8, None, 5, None, 0, P16, P16, P16, s) == INVALID
    assert lib.quantize_rows_int8(P_ODD, 10, 8, P16, 5, None, 0, P16, P16, P16, s) == MISALIGNED
    assert lib.quantize_rows_int8(P16, 10, 8, P16, 0, None, 0, P16, P16, P16, s) == OK
    assert lib.mark_rows(P16, -1, None, 10, P16, P16, P16, s) == INVALID
    assert lib.mark_rows(P16, 5, None, 10, None, P16, P16, s) == INVALID
    assert lib.mark_rows(P_ODD, 5, None, 10, P16, P16, P16, s) == MISALIGNED
    assert lib.clear_marks(P16, None, 10, P16, s) == INVALID
    assert lib.clear_marks(P16, P16, -1, P16, s) == INVALID
    need = lib.writeback_rows_workspace_size(100, 4, 10, 0)
    assert lib.writeback_plan_rows(100, 10, P16, need, P16, None, s) == INVALID
    assert lib.writeback_plan_rows(100, 10, P16, need - 1, P16, P16, s) == WS_SMALL
    assert lib.writeback_plan_rows(100, -2, P16, need, P16, P16, s) == INVALID


def test_key_store_argument_errors(lib):
    s = None
    need = lib.dks_workspace_size(10)
    call = lambda cap, ins, ws, wsb, dim=8, shift=6, nch=2, chunks=P16, nxt=P16, n=10: lib.dks_lookup_or_insert(
        P16, P16, cap, chunks, shift, nch, dim, nxt, P16, n, 3, ins, P16, P16, None, ws, wsb, s)
    assert call(1000, 1, P16, need) == INVALID      # key capacity not a power of two
    assert call(1024, 2, P16, need) == INVALID      # insert flag
    assert call(1024, 1, None, 0) == WS_SMALL
    assert call(1024, 1, P16, need - 1) == WS_SMALL
    assert call(1024, 1, ctypes.c_void_p((1 << 20) + 16), need) == MISALIGNED
    assert call(1024, 1, P16, need, dim=6) == DIM
    assert call(1024, 1, P16, need, n=-1) == INVALID
    assert call(1024, 1, P16, need, shift=3) == INVALID and call(1024, 1, P16, need, shift=25) == INVALID
    assert call(1024, 1, P16, need, chunks=None) == INVALID   # chunks in use but no chunk table
    assert call(1024, 1, P16, need, chunks=P_ODD) == MISALIGNED
    assert call(1024, 1, P16, need, nxt=None) == INVALID      # insert needs next_row
    assert lib.dks_chunk_bytes(6, 8) == (4 * 8 + 8 + 4) * 64
    assert lib.dks_chunk_bytes(3, 8) == 0 and lib.dks_chunk_bytes(6, 6) == 0
    assert lib.dks_chunk_init(None, 6, 8, s) == INVALID
    assert lib.dks_chunk_init(P_ODD, 6, 8, s) == MISALIGNED
    assert lib.dks_gather_rows(P16, 6, 2, 8, P16, -1, P16, s) == INVALID
    assert lib.dks_gather_rows(P16, 6, 2, 6, P16, 10, P16, s) == DIM
    assert lib.dks_gather_rows(P16, 6, 2, 8, P16, 10, P_ODD, s) == MISALIGNED
    assert lib.dks_rehash(P16, P16, 1024, P16, P16, 512, s) == INVALID  # smaller table
    assert lib.dks_rehash(P16, P16, 1024, P16, P16, 3000, s) == INVALID
    assert lib.dks_rehash(P_ODD, P16, 1024, P16, P16, 2048, s) == MISALIGNED


def test_memory_layer_step_argument_errors(lib):
    """Every host-checkable fault returns before anything is enqueued (no stream or event is touched)."""
    s = None
    n, C, D, P = 1000, 4096, 64, 8
    mzb = lib.mpzch_lookup_or_insert_workspace_size(n, 1)
    wbb = lib.memory_layer_step_workspace_size(n, C)

    def call(cap=C, probes=P, dim=D, n=n, n_max=n, values=P16, ids=P16, mzb=mzb, wbb=wbb, looked=P16, planned=P16,
             gb=None, ge=None, halves=3):
        return lib.memory_layer_step(P16, P16, values, cap, probes, dim, ids, n, n_max, 5, P16, P16, P16, None,
                                     None, P16, P16, mzb, P16, wbb, s, s, None, looked, planned, gb, ge, None, halves)
    assert call(cap=4095) == INVALID                 # capacity % probes
    assert call(probes=0) == INVALID
    assert call(n=-1) == INVALID
    assert call(n=n + 1) == INVALID                  # a batch larger than the workspaces serve (n_max)
    assert call(dim=6) == DIM
    assert call(values=None) == INVALID
    assert call(ids=None) == INVALID
    assert call(values=P_ODD) == MISALIGNED
    assert call(mzb=mzb - 1) == WS_SMALL
    assert call(wbb=wbb - 1) == WS_SMALL
    assert call(halves=0) == INVALID and call(halves=4) == INVALID


def test_static_mpzch_rejects_batches_beyond_its_array(lib):
    """The allocation-free MPZCH call refuses a batch larger than its device array serves, before
    anything is enqueued (no device is touched here)."""
    m = lib.mpzch_lookup_or_insert_static_max_n()
    assert m == 262144
    args = (P16, P16, None, 4096, 8, 64, P16)
    tail = (7, 1, P16, P16, None, None, None)
    assert lib.mpzch_lookup_or_insert_static(*args, m + 1, *tail) == INVALID
    assert lib.mpzch_lookup_or_insert_static(*args, -1, *tail) == INVALID


def test_score_dedup_hashed_argument_errors(lib):
    s = None
    assert lib.gather_dequant_score(P16, P16, P16, 10, 520, P16, 2, 3, P16, P16, s) == DIM
    assert lib.gather_dequant_score(P_ODD, P16, P16, 10, 512, P16, 2, 3, P16, P16, s) == MISALIGNED
    assert lib.gather_dequant_score(P16, P16, P16, 10, 512, P16, -1, 3, P16, P16, s) == INVALID
    assert lib.dedup_ids(P16, 10, P16, P16, None, None, P16, 1 << 30, s) == INVALID  # count pointer required
    assert lib.dedup_ids(P16, 10, P16, P16, None, P16, None, 0, s) == WS_SMALL
    assert lib.hashed_rows(P16, 10, 0, P16, s) == INVALID
    assert lib.hashed_rows(P_ODD, 10, 5, P16, s) == MISALIGNED


def test_binding_refuses_cpu_tensors():
    import torch
    t = torch.zeros((4, 4))
    with pytest.raises(hlr.HLRError):
        hlr.gather_rows(t, torch.zeros(2, dtype=torch.int64))
