"""MI355X-native hot path of an in-model embedding cache (MPZCH + Writeback).

Thin ctypes binding over libhlr.so (include/hlr.h).  Every step runs in the
library's HIP kernels; this module only marshals torch tensors (device memory
and the current HIP stream) into the C ABI and turns status codes into
exceptions.  There is no CPU fallback: if the library is missing, or a tensor
is not on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhlr.so")

HLR_OK = 0
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported dim", 3: "misaligned pointer", 4: "workspace too small",
          5: "HIP launch error"}
WB_LAST_WINS = 0
WB_SGD_SUM = 1
WB_L2_ALIGN = 2
EMPTY_ID = -1

_lib = None
_lock = threading.Lock()
_ws = {}


class HLRError(RuntimeError):
    pass


def load_library():
    """Loads libhlr.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise HLRError(f"{LIB_PATH} is missing: build it with `python -m hashed_lookup_row_amd.build` "
                           "(or __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        i64, i32, p, sz, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
        sig = {
            "hlr_status_string": (ctypes.c_char_p, [i32]),
            "hlr_version": (i32, []),
            "mpzch_lookup_or_insert_workspace_size": (sz, [i64, i32]),
            "mpzch_lookup_or_insert": (i32, [p, p, p, i64, i32, i64, p, i64, i64, i32, p, p, p, p, p, sz, p]),
            "gather_rows": (i32, [p, i64, i64, p, i64, p, p]),
            "dedup_ids_workspace_size": (sz, [i64]),
            "dedup_ids": (i32, [p, i64, p, p, p, p, p, sz, p]),
            "writeback_rows_workspace_size": (sz, [i64, i64, i64, i32]),
            "writeback_rows": (i32, [p, i64, i64, p, p, i64, i32, f32, p, sz, p]),
            "ema_update_rows_workspace_size": (sz, [i64, i64, i64]),
            "ema_update_rows": (i32, [p, i64, i64, p, p, p, i64, f32, f32, p, sz, p]),
            "gather_dequant_score": (i32, [p, p, p, i64, i64, p, i64, i64, p, p, p]),
            "mpzch_score": (i32, [p, i64, i32, p, p, p, p, i64, i64, i64, p, p, p, p, p]),
            "hashed_rows": (i32, [p, i64, i64, p, p]),
            "mpzch_zero_inserted": (i32, [p, i64, i64, p, p, i64, p]),
            "writeback_plan": (i32, [i64, p, i64, i32, p, sz, p]),
            "writeback_apply": (i32, [p, i64, i64, p, i64, i32, f32, p, sz, p]),
            "ema_update_plan": (i32, [i64, p, p, i64, p, sz, p]),
            "ema_update_apply": (i32, [p, i64, i64, p, i64, f32, f32, p, sz, p]),
            "ema_update_plan_subset": (i32, [i64, p, i64, p, sz, p, sz, p]),
            "ema_update_apply_batch": (i32, [i32, p, p]),
            "ema_update_pair_workspace_size": (sz, [i64, i64, i64, i64]),
            "ema_update_plan_pair": (i32, [i64, p, i64, p, p, i64, p, sz, p]),
            "ema_update_apply_pairs": (i32, [i32, p, p]),
            "writeback_apply_batch": (i32, [i32, p, i32, p]),
            "writeback_plan_rows": (i32, [i64, i64, p, sz, p, p, p]),
            "quantize_rows_int8": (i32, [p, i64, i64, p, i64, p, i32, p, p, p, p]),
            "mark_rows": (i32, [p, i64, p, i64, p, p, p, p]),
            "clear_marks": (i32, [p, p, i64, p, p]),
            "dks_workspace_size": (sz, [i64]),
            "dks_lookup_or_insert": (i32, [p, p, i64, p, i32, i64, i64, p, p, i64, i64, i32, p, p, p, p, sz, p]),
            "dks_chunk_bytes": (i64, [i32, i64]),
            "dks_chunk_init": (i32, [p, i32, i64, p]),
            "dks_gather_rows": (i32, [p, i32, i64, i64, p, i64, p, p]),
            "dks_rehash": (i32, [p, p, i64, p, p, i64, p]),
            "memory_layer_step": (i32, [p, p, p, i64, i32, i64, p, i64, i64, i64, p, p, p, p, p, p, p, sz, p, sz,
                                        p, p, p, p, p, p, p, p, i32]),
            "memory_layer_step_workspace_size": (sz, [i64, i64]),
            "mpzch_lookup_or_insert_static_max_n": (i64, []),
            "mpzch_lookup_or_insert_static": (i32, [p, p, p, i64, i32, i64, p, i64, i64, i32, p, p, p, p, p]),
            "memory_layer_step_workspace_init": (i32, [p, sz, p, sz, i64, i64, p]),
            "memory_layer_step_mark_written": (i32, [p, sz, i64, i64, i64, p, p, p, p]),
        }
        for name, (res, args) in sig.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
        return lib


def exported_symbols():
    return ["hlr_status_string", "hlr_version", "mpzch_lookup_or_insert_workspace_size", "mpzch_lookup_or_insert",
            "gather_rows", "dedup_ids_workspace_size", "dedup_ids", "writeback_rows_workspace_size",
            "writeback_rows", "ema_update_rows_workspace_size", "ema_update_rows", "gather_dequant_score", "mpzch_score",
            "hashed_rows", "mpzch_zero_inserted", "writeback_plan", "writeback_apply", "ema_update_plan",
            "ema_update_apply", "writeback_plan_rows", "quantize_rows_int8", "mark_rows", "clear_marks",
            "dks_workspace_size", "dks_lookup_or_insert", "dks_rehash", "dks_chunk_bytes", "dks_chunk_init",
            "dks_gather_rows", "memory_layer_step",
            "memory_layer_step_workspace_size", "memory_layer_step_workspace_init", "memory_layer_step_mark_written",
            "mpzch_lookup_or_insert_static_max_n", "mpzch_lookup_or_insert_static", "ema_update_plan_subset", "ema_update_apply_batch",
            "writeback_apply_batch", "ema_update_pair_workspace_size", "ema_update_plan_pair", "ema_update_apply_pairs"]


def _check(rc: int, what: str):
    if rc != HLR_OK:
        raise HLRError(f"{what}: {STATUS.get(rc, rc)} (status {rc})")


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise HLRError(f"{name} must be a GPU tensor (got {t.device}); there is no CPU path")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise HLRError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device, stream=None):
    """HIP stream handle: `stream` (a torch stream or a raw handle) or the device's current stream."""
    if stream is not None:
        return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    if _raw_stream is not None:
        return ctypes.c_void_p(_raw_stream(device.index if device.index is not None else torch.cuda.current_device()))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace(device, nbytes: int) -> torch.Tensor:
    """Grow-only scratch buffer per device (calls on one stream may share it)."""
    if nbytes <= 0:
        return None
    key = torch.device(device).index
    buf = _ws.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(int(nbytes * 1.25) + 4096, dtype=torch.uint8, device=device)
        _ws[key] = buf
    return buf


def _ws_args(device, nbytes):
    buf = workspace(device, nbytes)
    if buf is None:
        return None, 0
    base = buf.data_ptr()
    aligned = (base + 255) // 256 * 256
    return ctypes.c_void_p(aligned), buf.numel() - (aligned - base)


# ----------------------------------------------------------------- entry points
def mpzch_workspace_size(n, insert=True) -> int:
    return int(load_library().mpzch_lookup_or_insert_workspace_size(int(n), 1 if insert else 0))


def mpzch_lookup_or_insert(identity, stamps, values, probes, ids, now, insert=True, out_rows=None, out_hit=None,
                           out_evicted=None, out_stats=None, ws=None, stream=None):
    """MPZCH lookup (insert=False) or lookup-or-insert with LRU eviction.

    ws: optional caller workspace (uint8 GPU tensor, new_workspace()); default: the
    per-device shared buffer (calls that share it must be ordered on one stream).
    Returns (rows int64[n], hit int8[n], evicted int64[n] or None, stats int64[6] or None)."""
    lib = load_library()
    _dev(identity, "identity", torch.int64)
    if stamps is not None:
        _dev(stamps, "stamps", torch.int64)
    if values is not None:
        _dev(values, "values", torch.float32)
    _dev(ids, "ids", torch.int64)
    dev = identity.device
    n = ids.numel()
    dim = values.shape[1] if values is not None else 0
    rows = out_rows if out_rows is not None else torch.empty(n, dtype=torch.int64, device=dev)
    hit = out_hit if out_hit is not None else torch.empty(n, dtype=torch.int8, device=dev)
    need = lib.mpzch_lookup_or_insert_workspace_size(n, 1 if insert else 0)
    if ws is not None and need > 0:
        ws, wsb = _own_ws(ws, need)
    else:
        ws, wsb = _ws_args(dev, need)
    rc = lib.mpzch_lookup_or_insert(_ptr(identity), _ptr(stamps), _ptr(values), identity.numel(), int(probes), dim,
                                    _ptr(ids), n, int(now), 1 if insert else 0, _ptr(rows), _ptr(hit),
                                    _ptr(out_evicted), _ptr(out_stats), ws, wsb, _stream(dev, stream))
    _check(rc, "mpzch_lookup_or_insert")
    return rows, hit, out_evicted, out_stats


def gather_rows(table, rows, out=None, stream=None):
    lib = load_library()
    _dev(table, "table", torch.float32)
    _dev(rows, "rows", torch.int64)
    n, dim = rows.numel(), table.shape[1]
    out = out if out is not None else torch.empty((n, dim), dtype=torch.float32, device=table.device)
    _check(lib.gather_rows(_ptr(table), table.shape[0], dim, _ptr(rows), n, _ptr(out), _stream(table.device, stream)),
           "gather_rows")
    return out


def dedup_ids(keys, out_unique=None, out_last_pos=None, out_inverse=None, out_num_unique=None, inverse=True, stream=None):
    """Returns (unique[n], last_pos[n], inverse[n] or None, num_unique int64[1]); first u entries valid."""
    lib = load_library()
    _dev(keys, "keys", torch.int64)
    dev, n = keys.device, keys.numel()
    uq = out_unique if out_unique is not None else torch.empty(n, dtype=torch.int64, device=dev)
    lp = out_last_pos if out_last_pos is not None else torch.empty(n, dtype=torch.int64, device=dev)
    inv = out_inverse if out_inverse is not None else (torch.empty(n, dtype=torch.int64, device=dev)
                                                       if inverse else None)
    nu = out_num_unique if out_num_unique is not None else torch.empty(1, dtype=torch.int64, device=dev)
    ws, wsb = _ws_args(dev, lib.dedup_ids_workspace_size(n))
    _check(lib.dedup_ids(_ptr(keys), n, _ptr(uq), _ptr(lp), _ptr(inv), _ptr(nu), ws, wsb, _stream(dev, stream)),
           "dedup_ids")
    return uq, lp, inv, nu


def writeback_rows(table, rows, src, mode=WB_LAST_WINS, lr=1.0, stream=None):
    lib = load_library()
    _dev(table, "table", torch.float32)
    _dev(rows, "rows", torch.int64)
    _dev(src, "src", torch.float32)
    n, dim = rows.numel(), table.shape[1]
    if src.numel() != n * dim:
        raise HLRError("src must be [n, dim]")
    ws, wsb = _ws_args(table.device, lib.writeback_rows_workspace_size(table.shape[0], dim, n, int(mode)))
    _check(lib.writeback_rows(_ptr(table), table.shape[0], dim, _ptr(rows), _ptr(src), n, int(mode), float(lr), ws,
                              wsb, _stream(table.device, stream)), "writeback_rows")
    return table


def ema_update_rows(table, rows, vals, mask, a, b, stream=None):
    lib = load_library()
    _dev(table, "table", torch.float32)
    _dev(rows, "rows", torch.int64)
    _dev(vals, "vals", torch.float32)
    if mask is not None:
        _dev(mask, "mask", torch.uint8)
    n, dim = rows.numel(), table.shape[1]
    if vals.numel() != n * dim:
        raise HLRError("vals must be [n, dim]")
    ws, wsb = _ws_args(table.device, lib.ema_update_rows_workspace_size(table.shape[0], dim, n))
    _check(lib.ema_update_rows(_ptr(table), table.shape[0], dim, _ptr(rows), _ptr(vals), _ptr(mask), n, float(a),
                               float(b), ws, wsb, _stream(table.device, stream)), "ema_update_rows")
    return table


def gather_dequant_score(qtable, scale, bias, rows, user, cands, out=None, stream=None):
    lib = load_library()
    _dev(qtable, "qtable", torch.int8)
    _dev(scale, "scale", torch.float32)
    _dev(bias, "bias", torch.float32)
    _dev(rows, "rows", torch.int64)
    _dev(user, "user", torch.float32)
    nreq, dim = user.shape[0], qtable.shape[1]
    out = out if out is not None else torch.empty((nreq, cands), dtype=torch.float32, device=qtable.device)
    _check(lib.gather_dequant_score(_ptr(qtable), _ptr(scale), _ptr(bias), qtable.shape[0], dim, _ptr(rows), nreq,
                                    int(cands), _ptr(user), _ptr(out), _stream(qtable.device, stream)),
           "gather_dequant_score")
    return out


def mpzch_score(identity, probes, ids, qtable, scale, bias, user, cands, out=None, out_rows=None, out_hit=None,
                stream=None):
    """Lookup-only MPZCH of ids and the int8 dequant-score of the rows found, in one launch (qtable holds
    one row per identity slot).  Returns the scores [requests, cands]."""
    lib = load_library()
    _dev(identity, "identity", torch.int64)
    _dev(ids, "ids", torch.int64)
    _dev(qtable, "qtable", torch.int8)
    _dev(scale, "scale", torch.float32)
    _dev(bias, "bias", torch.float32)
    _dev(user, "user", torch.float32)
    if qtable.shape[0] != identity.numel():
        raise HLRError("qtable must hold one row per identity slot")
    nreq, dim = user.shape[0], qtable.shape[1]
    if ids.numel() != nreq * int(cands):
        raise HLRError("ids must hold requests x cands IDs")
    for t, name, dt in ((out_rows, "out_rows", torch.int64), (out_hit, "out_hit", torch.int8)):
        if t is not None:
            _dev(t, name, dt)
            if t.numel() < ids.numel():
                raise HLRError(f"{name} must hold one entry per ID")
    out = out if out is not None else torch.empty((nreq, cands), dtype=torch.float32, device=qtable.device)
    _check(lib.mpzch_score(_ptr(identity), identity.numel(), int(probes), _ptr(ids), _ptr(qtable), _ptr(scale),
                           _ptr(bias), dim, nreq, int(cands), _ptr(user), _ptr(out), _ptr(out_rows), _ptr(out_hit),
                           _stream(qtable.device, stream)), "mpzch_score")
    return out


def hashed_rows(ids, num_rows, out=None, stream=None):
    lib = load_library()
    _dev(ids, "ids", torch.int64)
    out = out if out is not None else torch.empty(ids.numel(), dtype=torch.int64, device=ids.device)
    _check(lib.hashed_rows(_ptr(ids), ids.numel(), int(num_rows), _ptr(out), _stream(ids.device, stream)), "hashed_rows")
    return out


# ------------------------------------------------- split (plan / apply) forms
def new_workspace(device, nbytes: int) -> torch.Tensor:
    """A caller-owned scratch buffer for the plan/apply entry points (one per plan in flight)."""
    return torch.empty(max(int(nbytes), 1) + 256, dtype=torch.uint8, device=device)


def _own_ws(ws: torch.Tensor, need: int):
    _dev(ws, "ws", torch.uint8)
    base = ws.data_ptr()
    aligned = (base + 255) // 256 * 256
    avail = ws.numel() - (aligned - base)
    if avail < need:
        raise HLRError(f"workspace too small: {avail} bytes, need {need}")
    return ctypes.c_void_p(aligned), avail


def writeback_workspace_size(num_rows, dim, n, mode=WB_LAST_WINS) -> int:
    return int(load_library().writeback_rows_workspace_size(int(num_rows), int(dim), int(n), int(mode)))


def memory_layer_step_workspace_size(n, capacity) -> int:
    return int(load_library().memory_layer_step_workspace_size(int(n), int(capacity)))


def ema_workspace_size(num_rows, dim, n) -> int:
    return int(load_library().ema_update_rows_workspace_size(int(num_rows), int(dim), int(n)))


def mpzch_zero_inserted(values, rows, hit, stream=None):
    """Zero the rows a lookup (run with values=None) inserted: rows[i] for hit[i] == 0."""
    lib = load_library()
    _dev(values, "values", torch.float32)
    _dev(rows, "rows", torch.int64)
    _dev(hit, "hit", torch.int8)
    _check(lib.mpzch_zero_inserted(_ptr(values), values.shape[0], values.shape[1], _ptr(rows), _ptr(hit),
                                   rows.numel(), _stream(values.device, stream)), "mpzch_zero_inserted")


def writeback_plan(num_rows, rows, ws, mode=WB_LAST_WINS, stream=None):
    lib = load_library()
    _dev(rows, "rows", torch.int64)
    n = rows.numel()
    w, wb = _own_ws(ws, lib.writeback_rows_workspace_size(int(num_rows), 4, n, int(mode)))
    _check(lib.writeback_plan(int(num_rows), _ptr(rows), n, int(mode), w, wb, _stream(rows.device, stream)),
           "writeback_plan")


def writeback_apply(table, src, ws, mode=WB_LAST_WINS, lr=1.0, stream=None):
    lib = load_library()
    _dev(table, "table", torch.float32)
    _dev(src, "src", torch.float32)
    dim = table.shape[1]
    n = src.numel() // dim
    w, wb = _own_ws(ws, lib.writeback_rows_workspace_size(table.shape[0], dim, n, int(mode)))
    _check(lib.writeback_apply(_ptr(table), table.shape[0], dim, _ptr(src), n, int(mode), float(lr), w, wb,
                               _stream(table.device, stream)), "writeback_apply")
    return table


class _WbApply(ctypes.Structure):
    """hlr_wb_apply (include/hlr.h)."""
    _fields_ = [("table", ctypes.c_void_p), ("num_rows", ctypes.c_int64), ("dim", ctypes.c_int64),
                ("src", ctypes.c_void_p), ("n", ctypes.c_int64), ("lr", ctypes.c_float),
                ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t)]


def writeback_apply_batch(updates, mode=WB_SGD_SUM, stream=None):
    """Applies up to eight independent SGD_SUM / L2_ALIGN updates, each (table, src, lr, ws) with its
    plan in ws, in two launches; the results equal writeback_apply for each in turn."""
    lib = load_library()
    arr = (_WbApply * max(1, len(updates)))()
    dev = None
    for i, (table, src, lr, ws) in enumerate(updates):
        _dev(table, "table", torch.float32)
        _dev(src, "src", torch.float32)
        dim = table.shape[1]
        n = src.numel() // dim
        w, wb = _own_ws(ws, lib.writeback_rows_workspace_size(table.shape[0], dim, n, int(mode)))
        arr[i] = _WbApply(table.data_ptr(), table.shape[0], dim, src.data_ptr(), n, float(lr), w.value, wb)
        dev = table.device
    if not updates:
        return
    _check(lib.writeback_apply_batch(len(updates), ctypes.cast(arr, ctypes.c_void_p), int(mode),
                                     _stream(dev, stream)), "writeback_apply_batch")


def ema_update_plan(num_rows, rows, mask, ws, stream=None):
    lib = load_library()
    _dev(rows, "rows", torch.int64)
    if mask is not None:
        _dev(mask, "mask", torch.uint8)
    n = rows.numel()
    w, wb = _own_ws(ws, lib.ema_update_rows_workspace_size(int(num_rows), 4, n))
    _check(lib.ema_update_plan(int(num_rows), _ptr(rows), _ptr(mask), n, w, wb, _stream(rows.device, stream)),
           "ema_update_plan")


def ema_update_plan_subset(num_rows, mask, src_ws, ws, stream=None):
    """The plan of the positions of the plan in src_ws whose mask is set (no sort)."""
    lib = load_library()
    _dev(mask, "mask", torch.uint8)
    n = mask.numel()
    need = lib.ema_update_rows_workspace_size(int(num_rows), 4, n)
    sw, swb = _own_ws(src_ws, need)
    w, wb = _own_ws(ws, need)
    _check(lib.ema_update_plan_subset(int(num_rows), _ptr(mask), n, sw, swb, w, wb, _stream(mask.device, stream)),
           "ema_update_plan_subset")


class _EmaApply(ctypes.Structure):
    """hlr_ema_apply (include/hlr.h)."""
    _fields_ = [("table", ctypes.c_void_p), ("num_rows", ctypes.c_int64), ("dim", ctypes.c_int64),
                ("vals", ctypes.c_void_p), ("n", ctypes.c_int64), ("a", ctypes.c_float), ("b", ctypes.c_float),
                ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t)]


def ema_update_apply_batch(updates, stream=None):
    """Applies up to four independent EMA updates, each (table, vals, a, b, ws) with its plan in ws,
    in one launch; the results equal ema_update_apply for each in turn."""
    lib = load_library()
    arr = (_EmaApply * max(1, len(updates)))()
    dev = None
    for i, (table, vals, a, b, ws) in enumerate(updates):
        _dev(table, "table", torch.float32)
        _dev(vals, "vals", torch.float32)
        dim = table.shape[1]
        n = vals.numel() // dim
        w, wb = _own_ws(ws, lib.ema_update_rows_workspace_size(table.shape[0], dim, n))
        arr[i] = _EmaApply(table.data_ptr(), table.shape[0], dim, vals.data_ptr(), n, float(a), float(b), w.value, wb)
        dev = table.device
    if not updates:
        return
    _check(lib.ema_update_apply_batch(len(updates), ctypes.cast(arr, ctypes.c_void_p), _stream(dev, stream)),
           "ema_update_apply_batch")


def ema_pair_workspace_size(num_rows0, num_rows1, dim, n) -> int:
    """Bytes of a pair plan's workspace (0 for sizes out of range)."""
    return int(load_library().ema_update_pair_workspace_size(int(num_rows0), int(num_rows1), int(dim), int(n)))


def ema_update_plan_pair(num_rows0, rows0, num_rows1, rows1, mask, ws, stream=None):
    """One plan for two updates keyed by rows0 (a table of num_rows0 rows) and rows1 (num_rows1 rows), with the
    same mask (or None); its subsets come from ema_update_plan_subset(num_rows0 + num_rows1, mask2, ...)
    with a mask of n elements and a workspace of ema_pair_workspace_size."""
    lib = load_library()
    _dev(rows0, "rows0", torch.int64)
    _dev(rows1, "rows1", torch.int64)
    n = rows0.numel()
    if rows1.numel() != n:
        raise HLRError("rows0 and rows1 must have the same number of positions")
    if mask is not None:
        _dev(mask, "mask", torch.uint8)
        if mask.numel() != n:
            raise HLRError("mask must have one entry per position")
    w, wb = _own_ws(ws, lib.ema_update_pair_workspace_size(int(num_rows0), int(num_rows1), 4, n))
    _check(lib.ema_update_plan_pair(int(num_rows0), _ptr(rows0), int(num_rows1), _ptr(rows1), _ptr(mask), n, w, wb,
                                    _stream(rows0.device, stream)), "ema_update_plan_pair")


def ema_update_plan_pair_subset(num_rows0, num_rows1, mask, src_ws, ws, stream=None):
    """The pair plan of the positions of the pair plan in src_ws whose mask (n elements) is set."""
    lib = load_library()
    _dev(mask, "mask", torch.uint8)
    n = mask.numel()
    need = lib.ema_update_pair_workspace_size(int(num_rows0), int(num_rows1), 4, n)
    sw, swb = _own_ws(src_ws, need)
    w, wb = _own_ws(ws, need)
    _check(lib.ema_update_plan_subset(int(num_rows0) + int(num_rows1), _ptr(mask), 2 * n, sw, swb, w, wb,
                                      _stream(mask.device, stream)), "ema_update_plan_subset")


class _EmaApplyPair(ctypes.Structure):
    """hlr_ema_apply_pair (include/hlr.h)."""
    _fields_ = [("table0", ctypes.c_void_p), ("num_rows0", ctypes.c_int64), ("vals0", ctypes.c_void_p),
                ("table1", ctypes.c_void_p), ("num_rows1", ctypes.c_int64), ("vals1", ctypes.c_void_p),
                ("dim", ctypes.c_int64), ("n", ctypes.c_int64), ("a", ctypes.c_float), ("b", ctypes.c_float),
                ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t)]


def ema_update_apply_pairs(pairs, stream=None):
    """Applies up to four pair plans in one launch; each pair is (table0, vals0, table1, vals1, a, b, ws) with its
    plan in ws.  The results equal ema_update_apply on each table in turn."""
    lib = load_library()
    arr = (_EmaApplyPair * max(1, len(pairs)))()
    dev = None
    for i, (t0, v0, t1, v1, a, b, ws) in enumerate(pairs):
        for t, name in ((t0, "table0"), (v0, "vals0"), (t1, "table1"), (v1, "vals1")):
            _dev(t, name, torch.float32)
        dim = t0.shape[1]
        if t1.shape[1] != dim:
            raise HLRError("both tables of a pair must have the same dim")
        n = v0.numel() // dim
        if v1.numel() != n * dim:
            raise HLRError("vals0 and vals1 must both hold n x dim values")
        w, wb = _own_ws(ws, lib.ema_update_pair_workspace_size(t0.shape[0], t1.shape[0], dim, n))
        arr[i] = _EmaApplyPair(t0.data_ptr(), t0.shape[0], v0.data_ptr(), t1.data_ptr(), t1.shape[0], v1.data_ptr(),
                               dim, n, float(a), float(b), w.value, wb)
        dev = t0.device
    if not pairs:
        return
    _check(lib.ema_update_apply_pairs(len(pairs), ctypes.cast(arr, ctypes.c_void_p), _stream(dev, stream)),
           "ema_update_apply_pairs")


def ema_update_apply(table, vals, a, b, ws, stream=None):
    lib = load_library()
    _dev(table, "table", torch.float32)
    _dev(vals, "vals", torch.float32)
    dim = table.shape[1]
    n = vals.numel() // dim
    w, wb = _own_ws(ws, lib.ema_update_rows_workspace_size(table.shape[0], dim, n))
    _check(lib.ema_update_apply(_ptr(table), table.shape[0], dim, _ptr(vals), n, float(a), float(b), w, wb,
                                _stream(table.device, stream)), "ema_update_apply")
    return table


def writeback_plan_rows(num_rows, n, ws, out_rows=None, out_count=None, stream=None):
    """Distinct rows of a LAST_WINS plan in `ws` (unspecified order): (rows int64[n], count int64[1])."""
    lib = load_library()
    dev = ws.device
    rows = out_rows if out_rows is not None else torch.empty(max(int(n), 1), dtype=torch.int64, device=dev)
    cnt = out_count if out_count is not None else torch.empty(1, dtype=torch.int64, device=dev)
    w, wb = _own_ws(ws, lib.writeback_rows_workspace_size(int(num_rows), 4, int(n), WB_LAST_WINS))
    _check(lib.writeback_plan_rows(int(num_rows), int(n), w, wb, _ptr(rows), _ptr(cnt), _stream(dev, stream)),
           "writeback_plan_rows")
    return rows, cnt


def quantize_rows_int8(table, rows, count=None, scatter=False, out=None, stream=None):
    """int8 per-row min-max quantisation of table[rows[i]] (first min(n, *count) entries).
    Returns (q int8, scale fp32, bias fp32): compact [n] rows, or with scatter=True written at index
    rows[i] of `out` (arrays of table.shape[0] rows; allocated zeroed if not given)."""
    lib = load_library()
    _dev(table, "table", torch.float32)
    _dev(rows, "rows", torch.int64)
    if count is not None:
        _dev(count, "count", torch.int64)
    dev, n, dim = table.device, rows.numel(), table.shape[1]
    if out is None:
        m = table.shape[0] if scatter else n
        out = (torch.zeros((m, dim), dtype=torch.int8, device=dev), torch.zeros(m, dtype=torch.float32, device=dev),
               torch.zeros(m, dtype=torch.float32, device=dev))
    q, sc, bi = out
    _check(lib.quantize_rows_int8(_ptr(table), table.shape[0], dim, _ptr(rows), n, _ptr(count), 1 if scatter else 0,
                                  _ptr(q), _ptr(sc), _ptr(bi), _stream(dev, stream)), "quantize_rows_int8")
    return q, sc, bi


def mark_rows(rows, num_rows, flags, lst, list_count, count=None, stream=None):
    """Appends the rows not yet flagged to `lst` (flags uint32[num_rows], lst int64[num_rows], list_count int64[1])."""
    lib = load_library()
    _dev(rows, "rows", torch.int64)
    _dev(flags, "flags", torch.int32)
    _dev(lst, "list", torch.int64)
    _dev(list_count, "list_count", torch.int64)
    if count is not None:
        _dev(count, "count", torch.int64)
    _check(lib.mark_rows(_ptr(rows), rows.numel(), _ptr(count), int(num_rows), _ptr(flags), _ptr(lst),
                         _ptr(list_count), _stream(rows.device, stream)), "mark_rows")


def clear_marks(lst, list_count, num_rows, flags, stream=None):
    lib = load_library()
    _dev(lst, "list", torch.int64)
    _dev(list_count, "list_count", torch.int64)
    _dev(flags, "flags", torch.int32)
    _check(lib.clear_marks(_ptr(lst), _ptr(list_count), int(num_rows), _ptr(flags), _stream(lst.device, stream)),
           "clear_marks")


def dks_workspace_size(n) -> int:
    return int(load_library().dks_workspace_size(int(n)))


def dks_chunk_bytes(chunk_shift, dim) -> int:
    """Bytes of one value-store chunk of 2^chunk_shift rows (0 for an invalid shift or dim)."""
    return int(load_library().dks_chunk_bytes(int(chunk_shift), int(dim)))


def dks_chunk_init(chunk, chunk_shift, dim, stream=None):
    """Clears a value-store chunk (a uint8 GPU tensor of dks_chunk_bytes bytes) before it joins the store."""
    lib = load_library()
    _dev(chunk, "chunk", torch.uint8)
    if chunk.numel() < lib.dks_chunk_bytes(int(chunk_shift), int(dim)):
        raise HLRError("chunk smaller than dks_chunk_bytes(chunk_shift, dim)")
    _check(lib.dks_chunk_init(_ptr(chunk), int(chunk_shift), int(dim), _stream(chunk.device, stream)),
           "dks_chunk_init")


def dks_lookup_or_insert(keys, krows, chunks, chunk_shift, num_chunks, dim, next_row, ids, now, insert=True,
                         out_rows=None, out_hit=None, out_stats=None, ws=None, stream=None):
    """Decoupled key store lookup (insert=False) or lookup-or-insert.  chunks: int64 GPU tensor of the value
    store's chunk addresses (its first num_chunks entries are used).  Returns (rows, hit, stats or None)."""
    lib = load_library()
    _dev(keys, "keys", torch.int64)
    _dev(krows, "krows", torch.int64)
    _dev(ids, "ids", torch.int64)
    _dev(chunks, "chunks", torch.int64)
    if chunks.numel() < int(num_chunks):
        raise HLRError("chunks holds fewer addresses than num_chunks")
    if next_row is not None:
        _dev(next_row, "next_row", torch.int64)
    dev, n = keys.device, ids.numel()
    rows = out_rows if out_rows is not None else torch.empty(n, dtype=torch.int64, device=dev)
    hit = out_hit if out_hit is not None else torch.empty(n, dtype=torch.int8, device=dev)
    need = lib.dks_workspace_size(n) if insert else 0
    if ws is not None and need > 0:
        w, wb = _own_ws(ws, need)
    else:
        w, wb = _ws_args(dev, need)
    _check(lib.dks_lookup_or_insert(_ptr(keys), _ptr(krows), keys.numel(), _ptr(chunks), int(chunk_shift),
                                    int(num_chunks), int(dim), _ptr(next_row), _ptr(ids), n, int(now),
                                    1 if insert else 0, _ptr(rows), _ptr(hit), _ptr(out_stats), w, wb,
                                    _stream(dev, stream)), "dks_lookup_or_insert")
    return rows, hit, out_stats


def dks_gather_rows(chunks, chunk_shift, num_chunks, dim, rows, out=None, stream=None):
    """out[n][dim] = the value-store vectors of rows (zeros for rows < 0 or beyond the rows held)."""
    lib = load_library()
    _dev(chunks, "chunks", torch.int64)
    _dev(rows, "rows", torch.int64)
    if chunks.numel() < int(num_chunks):
        raise HLRError("chunks holds fewer addresses than num_chunks")
    n = rows.numel()
    if out is None:
        out = torch.empty((n, int(dim)), dtype=torch.float32, device=rows.device)
    _dev(out, "out", torch.float32)
    if out.numel() != n * int(dim):
        raise HLRError("out must hold n x dim values")
    _check(lib.dks_gather_rows(_ptr(chunks), int(chunk_shift), int(num_chunks), int(dim), _ptr(rows), n, _ptr(out),
                               _stream(rows.device, stream)), "dks_gather_rows")
    return out


def dks_rehash(keys, krows, new_cap, stream=None):
    """New (keys, krows) of new_cap slots holding the same key -> row map."""
    lib = load_library()
    _dev(keys, "keys", torch.int64)
    _dev(krows, "krows", torch.int64)
    nk = torch.empty(int(new_cap), dtype=torch.int64, device=keys.device)
    nr = torch.empty(int(new_cap), dtype=torch.int64, device=keys.device)
    _check(lib.dks_rehash(_ptr(keys), _ptr(krows), keys.numel(), _ptr(nk), _ptr(nr), int(new_cap),
                          _stream(keys.device, stream)), "dks_rehash")
    return nk, nr
