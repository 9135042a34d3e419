"""A growable key store with a growable value store ("MTGR: Industrial-Scale Generative Recommendation
Framework in Meituan", sec. 3.2): dks_lookup_or_insert maps keys to rows; when the key store could pass
half full during the next batch it is rehashed into one twice as large (keys and row indices only), and
when the value store could run out of rows it gains chunks of rows (no row ever moves).  Each row holds
its vector, the last batch that touched it and the number of lookups that reached it.

After every batch the number of rows in use is copied to pinned memory behind an event, and both
growth checks use the newest copy whose event has completed plus an upper bound for what the batches
enqueued since can have added (a batch inserts at most n keys).  The host runs ahead of the GPU, so
that bound can be loose by many batches: the key store is grown on it as it stands (keys are cheap),
but before the value store gains a chunk the host waits for the oldest pending copies until the bound
fits the rows held or no copy is pending; those copies belong to batches the GPU has already reached
or is about to, so the batches queued after them keep it busy."""
from __future__ import annotations

from collections import deque

import torch

from . import (HLRError, dks_chunk_bytes, dks_chunk_init, dks_gather_rows, dks_lookup_or_insert, dks_rehash,
               dks_workspace_size, new_workspace)


class ChunkedValues:
    """The value store: chunks of 2^chunk_shift rows, each one allocation holding the rows' vectors (fp32,
    dim each), then their stamps (int64, -1 = never touched), then their lookup counts (uint32); `table`
    holds the chunks' device addresses, so row r is row r mod 2^chunk_shift of chunk r >> chunk_shift.
    The store holds at most max_rows rows, rounded up to whole chunks."""

    def __init__(self, dim, max_rows, device, chunk_shift=16, stream=None):
        self.dim, self.shift, self.device = int(dim), int(chunk_shift), torch.device(device)
        self.rows_per_chunk = 1 << self.shift
        self.bytes = dks_chunk_bytes(self.shift, self.dim)
        if self.bytes <= 0:
            raise HLRError(f"no value-store chunk for chunk_shift {chunk_shift} and dim {dim}")
        self.max_chunks = max(1, -(-int(max_rows) // self.rows_per_chunk))
        self.table = torch.zeros(self.max_chunks, dtype=torch.int64, device=self.device)
        self.chunks = []
        self.stream = stream

    @property
    def capacity(self) -> int:
        """Rows the store holds now."""
        return len(self.chunks) << self.shift

    @property
    def max_rows(self) -> int:
        return self.max_chunks << self.shift

    def grow_to(self, rows):
        """Adds cleared chunks until the store holds at least `rows` rows (at most max_rows)."""
        want = min(-(-int(rows) // self.rows_per_chunk), self.max_chunks)
        s = self.stream if self.stream is not None else torch.cuda.current_stream(self.device)
        while len(self.chunks) < want:
            with torch.cuda.stream(s):  # allocated, cleared and listed on the store's stream
                c = torch.empty(self.bytes, dtype=torch.uint8, device=self.device)
                dks_chunk_init(c, self.shift, self.dim, stream=s)
                self.table[len(self.chunks)].fill_(c.data_ptr())
            self.chunks.append(c)

    def _part(self, k, what):
        c, R, D = self.chunks[k], self.rows_per_chunk, self.dim
        if what == "vectors":
            return c[:4 * D * R].view(torch.float32).view(R, D)
        if what == "stamps":
            return c[4 * D * R:(4 * D + 8) * R].view(torch.int64)
        return c[(4 * D + 8) * R:(4 * D + 12) * R].view(torch.int32)  # uint32 counts, read as int32 bits

    def dump(self):
        """(vectors [capacity, dim], stamps [capacity], counts [capacity] as int64) copies of the whole store."""
        if not self.chunks:
            z = torch.empty(0, dtype=torch.int64, device=self.device)
            return torch.empty((0, self.dim), dtype=torch.float32, device=self.device), z, z
        vec = torch.cat([self._part(k, "vectors") for k in range(len(self.chunks))])
        st = torch.cat([self._part(k, "stamps") for k in range(len(self.chunks))])
        ct = torch.cat([self._part(k, "counts") for k in range(len(self.chunks))]).to(torch.int64) & 0xFFFFFFFF
        return vec, st, ct

    def gather(self, rows, out=None):
        return dks_gather_rows(self.table, self.shift, len(self.chunks), self.dim, rows, out=out, stream=self.stream)


class DynamicKeyStore:
    """stream: the torch stream the store's kernels run on (None: the current stream at each call).  The
    tables are filled on the current stream at construction; a given stream is ordered after that fill, and
    the tables a rehash replaces are kept alive for the allocator until the stream is done with them.
    capacity_history: the rows the value store held during each batch."""

    def __init__(self, dim, max_rows, device, key_cap=1 << 16, chunk_shift=16, stream=None, max_load=0.5,
                 initial_rows=0):
        dev = torch.device(device)
        if stream is not None and not isinstance(stream, torch.cuda.Stream):
            raise TypeError("stream must be a torch.cuda.Stream (or None for the current stream)")
        self.max_load = float(max_load)
        self.values = ChunkedValues(dim, max_rows, dev, chunk_shift, stream)
        self.max_rows = self.values.max_rows
        self.keys = torch.full((key_cap,), -1, dtype=torch.int64, device=dev)
        self.krows = torch.full((key_cap,), -1, dtype=torch.int64, device=dev)
        self.next_row = torch.zeros(1, dtype=torch.int64, device=dev)
        self.stream = stream
        if stream is not None:  # the fills above ran on the current stream
            stream.wait_stream(torch.cuda.current_stream(dev))
            for t in (self.keys, self.krows, self.next_row, self.values.table):
                t.record_stream(stream)
        # pinned copies of next_row, each with its event (created here: creating events per batch can
        # stall the GPU now and then while the runtime grows its signal pool)
        self._pinned = deque((torch.zeros(1, dtype=torch.int64, pin_memory=True), torch.cuda.Event())
                             for _ in range(8))
        for _, ev in self._pinned:  # torch creates an event's HIP event at its first record
            ev.record(torch.cuda.current_stream(dev))
        self._pending = deque()  # (event, pinned copy of next_row, keys offered up to that batch)
        self._offered = 0        # keys offered to the store so far (an upper bound for rows in use)
        self._known_used = 0
        self._known_offered = 0
        self._ws = None
        self.rehashes = 0
        self.capacity_history = []
        if initial_rows:
            self.values.grow_to(min(int(initial_rows), self.max_rows))

    def _refresh(self):
        while self._pending and self._pending[0][0].query():
            ev, pin, offered = self._pending.popleft()
            self._known_used, self._known_offered = int(pin[0]), offered
            self._pinned.append((pin, ev))

    def bound(self, n):
        """Upper bound for the rows in use after a batch of n more keys."""
        self._refresh()
        return self._known_used + (self._offered - self._known_offered) + n

    def grow_for(self, n):
        need = min(self.bound(n), self.max_rows)
        cap = self.keys.numel()
        while need > self.max_load * cap:
            cap *= 2
        if cap != self.keys.numel():
            old = (self.keys, self.krows)
            if self.stream is not None:
                # the new tables are allocated on the store's stream, which the rehash fills them on; the old
                # ones are kept from reuse until that stream is done reading them
                with torch.cuda.stream(self.stream):
                    self.keys, self.krows = dks_rehash(self.keys, self.krows, cap, stream=self.stream)
                for t in old:
                    t.record_stream(self.stream)
            else:
                self.keys, self.krows = dks_rehash(self.keys, self.krows, cap)
            self.rehashes += 1
        if need > self.values.capacity:
            while self._pending and need > self.values.capacity:  # tighten the bound first
                self._pending[0][0].synchronize()
                self._refresh()
                need = min(self.bound(n), self.max_rows)
            self.values.grow_to(need)

    def step(self, ids, now, out_rows=None, out_hit=None, out_stats=None):
        n = ids.numel()
        self.grow_for(n)
        need = dks_workspace_size(n)
        if self._ws is None or self._ws.numel() < need + 256:
            self._ws = new_workspace(ids.device, need)
        v = self.values
        rows, hit, _ = dks_lookup_or_insert(self.keys, self.krows, v.table, v.shift, len(v.chunks), v.dim,
                                            self.next_row, ids, now, True, out_rows=out_rows, out_hit=out_hit,
                                            out_stats=out_stats, ws=self._ws, stream=self.stream)
        self.capacity_history.append(v.capacity)
        self._offered += n
        if self._pinned:
            s = self.stream if self.stream is not None else torch.cuda.current_stream(ids.device)
            pin, ev = self._pinned.popleft()
            with torch.cuda.stream(s):
                pin.copy_(self.next_row, non_blocking=True)
                ev.record(s)
            self._pending.append((ev, pin, self._offered))
        return rows, hit

    def lookup(self, ids, out_rows=None, out_hit=None):
        """Lookup only (serving): rows and hit mask; nothing changes."""
        v = self.values
        rows, hit, _ = dks_lookup_or_insert(self.keys, self.krows, v.table, v.shift, len(v.chunks), v.dim,
                                            None, ids, 0, False, out_rows=out_rows, out_hit=out_hit,
                                            stream=self.stream)
        return rows, hit

    def gather(self, rows, out=None):
        """The value-store vectors of rows (zeros for rows < 0)."""
        return self.values.gather(rows, out=out)
