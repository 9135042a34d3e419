"""CPU oracle for the in-model embedding cache — TEST INFRASTRUCTURE ONLY.

A plain, single-threaded C implementation (oracle.c) of what the cache computes,
loaded through ctypes.  Only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does, and the
two share no code.

Every function restates the operation from the pages (see oracle.c's header
for the citations and for the readings taken where the pages are silent).  The
oracle is pinned in tests/test_oracle_*.py to things other than itself:
published SplitMix64 outputs, textbook set-associative LRU behaviour, library
routines (numpy unique/take/matmul), exact rational arithmetic and closed forms.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

OK, EINVAL, ENOMEM, ESTAMP = 0, 1, 2, 3


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # HLR_ORACLE_LIBRARY names another build of oracle.c to load instead (the mutation tests run the
            # pins against copies of the oracle with a planted mistake)
            alt = os.environ.get("HLR_ORACLE_LIBRARY")
            if not alt:
                build(force=False)
            lib = ctypes.CDLL(alt or _LIB)
            i64, i32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
            lib.orc_mix64.restype = ctypes.c_uint64
            lib.orc_mix64.argtypes = [ctypes.c_uint64]
            lib.orc_bucket.restype = i64
            lib.orc_bucket.argtypes = [i64, i64]
            lib.orc_mpzch_step.restype = ctypes.c_int
            lib.orc_mpzch_step.argtypes = [p, p, p, i64, i32, i64, p, i64, i64, i32, p, p, p, p]
            lib.orc_gather.restype = ctypes.c_int
            lib.orc_gather.argtypes = [p, i64, i64, p, i64, p]
            lib.orc_dedup.restype = i64
            lib.orc_dedup.argtypes = [p, i64, p, p, p]
            lib.orc_writeback_last.restype = ctypes.c_int
            lib.orc_writeback_last.argtypes = [p, i64, i64, p, p, i64]
            lib.orc_sgd_sum.restype = ctypes.c_int
            lib.orc_sgd_sum.argtypes = [p, i64, i64, p, p, i64, ctypes.c_float]
            lib.orc_dks_step.restype = ctypes.c_int
            lib.orc_dks_step.argtypes = [p, p, i64, p, p, p, i64, i64, p, p, i64, i64, i32, p, p, p]
            lib.orc_l2_align.restype = ctypes.c_int
            lib.orc_l2_align.argtypes = [p, i64, i64, p, p, i64, ctypes.c_float]
            lib.orc_quantize_rows.restype = ctypes.c_int
            lib.orc_quantize_rows.argtypes = [p, i64, i64, p, i64, i64, i32, p, p, p]
            lib.orc_ema.restype = ctypes.c_int
            lib.orc_ema.argtypes = [p, i64, i64, p, p, p, i64, ctypes.c_float, ctypes.c_float]
            lib.orc_dequant_score.restype = ctypes.c_int
            lib.orc_dequant_score.argtypes = [p, p, p, i64, i64, p, i64, i64, p, p]
            lib.orc_hashed_rows.restype = ctypes.c_int
            lib.orc_hashed_rows.argtypes = [p, i64, i64, p]
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _check(rc, what):
    if rc != OK:
        raise ValueError(f"oracle {what} failed with code {rc}")


# ---------------------------------------------------------------- primitives
def mix64(x: int) -> int:
    """SplitMix64 finaliser of the 64-bit pattern of x."""
    return int(_load().orc_mix64(ctypes.c_uint64(x & 0xFFFFFFFFFFFFFFFF)))


def bucket(id_: int, num_buckets: int) -> int:
    return int(_load().orc_bucket(int(id_), int(num_buckets)))


class MPZCHTable:
    """Oracle state of one MPZCH table: identity, LRU stamps and (optional) fp32 values."""

    def __init__(self, capacity: int, probes: int, dim: int, with_values: bool = True):
        self.capacity, self.probes, self.dim = int(capacity), int(probes), int(dim)
        self.identity = np.full(self.capacity, -1, dtype=np.int64)
        self.stamps = np.full(self.capacity, -1, dtype=np.int64)
        self.values = np.zeros((self.capacity, self.dim), dtype=np.float32) if with_values else None

    def step(self, ids, now: int, insert: bool = True, zero_fill: bool = True):
        """One lookup_or_insert batch; returns (rows, hit, evicted, stats)."""
        ids = _c(ids, np.int64)
        n = ids.size
        rows = np.empty(n, np.int64)
        hit = np.empty(n, np.int8)
        ev = np.empty(n, np.int64)
        st = np.zeros(5, np.int64)
        vals = self.values if (zero_fill and self.values is not None) else None
        rc = _load().orc_mpzch_step(_ptr(self.identity), _ptr(self.stamps), _ptr(vals), self.capacity,
                                    self.probes, self.dim, _ptr(ids), n, int(now), 1 if insert else 0,
                                    _ptr(rows), _ptr(hit), _ptr(ev), _ptr(st))
        _check(rc, "mpzch_step")
        return rows, hit, ev, st

    def gather(self, rows):
        return gather(self.values, rows)

    def writeback(self, rows, e):
        writeback_last(self.values, rows, e)


def mpzch_step(identity, stamps, values, capacity, probes, dim, ids, now, insert=True):
    """Functional form operating on caller-owned numpy state (modified in place)."""
    ids = _c(ids, np.int64)
    n = ids.size
    rows = np.empty(n, np.int64)
    hit = np.empty(n, np.int8)
    ev = np.empty(n, np.int64)
    st = np.zeros(5, np.int64)
    rc = _load().orc_mpzch_step(_ptr(identity), _ptr(stamps), _ptr(values), int(capacity), int(probes), int(dim),
                                _ptr(ids), n, int(now), 1 if insert else 0, _ptr(rows), _ptr(hit), _ptr(ev),
                                _ptr(st))
    _check(rc, "mpzch_step")
    return rows, hit, ev, st


def gather(table, rows):
    table = np.ascontiguousarray(table, dtype=np.float32)
    rows = _c(rows, np.int64)
    out = np.empty((rows.size, table.shape[1]), np.float32)
    _check(_load().orc_gather(_ptr(table), table.shape[0], table.shape[1], _ptr(rows), rows.size, _ptr(out)), "gather")
    return out


def dedup(keys):
    """(unique ascending, last position of each, inverse index per position)."""
    keys = _c(keys, np.int64)
    n = keys.size
    uq = np.empty(n, np.int64)
    lp = np.empty(n, np.int64)
    inv = np.empty(n, np.int64)
    u = _load().orc_dedup(_ptr(keys), n, _ptr(uq), _ptr(lp), _ptr(inv))
    if u < 0:
        raise MemoryError("oracle dedup")
    return uq[:u].copy(), lp[:u].copy(), inv


def writeback_last(table, rows, e):
    """In place on `table` (float32 C-contiguous numpy array)."""
    assert table.dtype == np.float32 and table.flags.c_contiguous
    rows = _c(rows, np.int64)
    e = _c(e, np.float32)
    _check(_load().orc_writeback_last(_ptr(table), table.shape[0], table.shape[1], _ptr(rows), _ptr(e), rows.size),
           "writeback_last")


def sgd_sum(table, rows, g, lr):
    """Per row: s = one fp32 running sum of its gradients in batch order; M <- fl(M - fl(lr*s))."""
    assert table.dtype == np.float32 and table.flags.c_contiguous
    rows = _c(rows, np.int64)
    g = _c(g, np.float32)
    _check(_load().orc_sgd_sum(_ptr(table), table.shape[0], table.shape[1], _ptr(rows), _ptr(g), rows.size,
                               ctypes.c_float(lr)), "sgd_sum")


class KeyStore:
    """Decoupled key store (open addressing, linear probing) + value store (rows handed out in order, each
    with its last-touch stamp and lookup count).  max_rows: the arrays' size; step(capacity=...) gives the
    rows the store holds during that batch (the caller's growth)."""

    def __init__(self, key_cap: int, max_rows: int, dim: int, with_values: bool = True):
        self.key_cap, self.max_rows, self.dim = int(key_cap), int(max_rows), int(dim)
        self.keys = np.full(self.key_cap, -1, np.int64)
        self.krows = np.full(self.key_cap, -1, np.int64)
        self.stamps = np.full(self.max_rows, -1, np.int64)
        self.counts = np.zeros(self.max_rows, np.uint32)
        self.values = np.zeros((self.max_rows, self.dim), np.float32) if with_values else None
        self.next_row = np.zeros(1, np.int64)

    def step(self, ids, now: int, insert: bool = True, capacity=None):
        ids = _c(ids, np.int64)
        n = ids.size
        cap = self.max_rows if capacity is None else int(capacity)
        if not 0 <= cap <= self.max_rows:
            raise ValueError("capacity beyond the oracle's arrays")
        rows = np.empty(n, np.int64)
        hit = np.empty(n, np.int8)
        stats = np.zeros(4, np.int64)
        _check(_load().orc_dks_step(_ptr(self.keys), _ptr(self.krows), self.key_cap, _ptr(self.stamps),
                                    _ptr(self.counts), _ptr(self.values), self.dim, cap, _ptr(self.next_row),
                                    _ptr(ids), n, int(now), 1 if insert else 0, _ptr(rows), _ptr(hit), _ptr(stats)),
               "dks_step")
        return rows, hit, stats

    def mapping(self):
        """{key: row} of the stored keys (every key but -1, the empty marker, is a valid key)."""
        m = self.keys != -1
        return dict(zip(self.keys[m].tolist(), self.krows[m].tolist()))


def l2_align(table, rows, e, lr):
    """SGD on ||M[r] - e_i||^2: per occurrence g = 2 (M - e_i), summed per row as in sgd_sum."""
    assert table.dtype == np.float32 and table.flags.c_contiguous
    rows = _c(rows, np.int64)
    e = _c(e, np.float32)
    _check(_load().orc_l2_align(_ptr(table), table.shape[0], table.shape[1], _ptr(rows), _ptr(e), rows.size,
                                ctypes.c_float(lr)), "l2_align")


def quantize_rows(table, rows, count=-1, scatter=False, out=None):
    """int8 per-row min-max quantisation of table[rows[i]].  Returns (q, scale, bias):
    compact (index i) or, with scatter=True, written at index rows[i] of `out` = (q, scale, bias)."""
    assert table.dtype == np.float32 and table.flags.c_contiguous
    rows = _c(rows, np.int64)
    dim = table.shape[1]
    if out is None:
        m = table.shape[0] if scatter else rows.size
        out = (np.zeros((m, dim), np.int8), np.zeros(m, np.float32), np.zeros(m, np.float32))
    q, sc, bi = out
    _check(_load().orc_quantize_rows(_ptr(table), table.shape[0], dim, _ptr(rows), rows.size, int(count),
                                     1 if scatter else 0, _ptr(q), _ptr(sc), _ptr(bi)), "quantize_rows")
    return q, sc, bi


def ema(table, rows, vals, mask, a, b):
    assert table.dtype == np.float32 and table.flags.c_contiguous
    rows = _c(rows, np.int64)
    vals = _c(vals, np.float32)
    m = None if mask is None else _c(mask, np.uint8)
    _check(_load().orc_ema(_ptr(table), table.shape[0], table.shape[1], _ptr(rows), _ptr(vals), _ptr(m), rows.size,
                           ctypes.c_float(a), ctypes.c_float(b)), "ema")


def dequant_score(qtable, scale, bias, rows, user, cands):
    qtable = _c(qtable, np.int8)
    scale = _c(scale, np.float32)
    bias = _c(bias, np.float32)
    rows = _c(rows, np.int64)
    user = _c(user, np.float32)
    nreq = user.shape[0]
    out = np.empty((nreq, cands), np.float32)
    _check(_load().orc_dequant_score(_ptr(qtable), _ptr(scale), _ptr(bias), qtable.shape[0], qtable.shape[1],
                                     _ptr(rows), nreq, int(cands), _ptr(user), _ptr(out)), "dequant_score")
    return out


def hashed_rows(ids, num_rows):
    ids = _c(ids, np.int64)
    out = np.empty(ids.size, np.int64)
    _check(_load().orc_hashed_rows(_ptr(ids), ids.size, int(num_rows), _ptr(out)), "hashed_rows")
    return out
