"""A growable key store with a fixed value store ("MTGR: Industrial-Scale Generative Recommendation
Framework in Meituan", sec. 3.2): dks_lookup_or_insert maps keys to rows; when the key store could
pass half full during the next batch it is rehashed into one twice as large (keys and row indices
only; the value rows never move).

The host never waits for the GPU: after every batch the number of rows in use is copied to pinned
memory behind an event, and the growth check uses the newest copy whose event has completed plus
an upper bound for what the batches enqueued since can have added (a batch inserts at most n keys)."""
from __future__ import annotations

from collections import deque

import torch

from . import dks_lookup_or_insert, dks_rehash, dks_workspace_size, new_workspace


class DynamicKeyStore:
    """stream: the torch stream the store's kernels run on (None: the current stream at each call).  The
    tables are filled on the current stream at construction; a given stream is ordered after that fill, and
    the tables a rehash replaces are kept alive for the allocator until the stream is done with them."""

    def __init__(self, values, max_rows, key_cap=1 << 16, stream=None, max_load=0.5):
        dev = values.device
        if stream is not None and not isinstance(stream, torch.cuda.Stream):
            raise TypeError("stream must be a torch.cuda.Stream (or None for the current stream)")
        self.values, self.max_rows, self.max_load = values, int(max_rows), float(max_load)
        self.keys = torch.full((key_cap,), -1, dtype=torch.int64, device=dev)
        self.krows = torch.full((key_cap,), -1, dtype=torch.int64, device=dev)
        self.stamps = torch.full((self.max_rows,), -1, dtype=torch.int64, device=dev)
        self.next_row = torch.zeros(1, dtype=torch.int64, device=dev)
        self.stream = stream
        if stream is not None:  # the fills above ran on the current stream
            stream.wait_stream(torch.cuda.current_stream(dev))
            for t in (self.keys, self.krows, self.stamps, self.next_row, values):
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
            self.keys, self.krows = dks_rehash(self.keys, self.krows, cap, stream=self.stream)
            if self.stream is not None:
                # the rehash reads the old tables and fills the new ones on self.stream: tell the caching
                # allocator, so it neither reuses the old blocks nor hands out the new ones elsewhere early
                for t in old + (self.keys, self.krows):
                    t.record_stream(self.stream)
            self.rehashes += 1

    def step(self, ids, now, out_rows=None, out_hit=None, out_stats=None):
        n = ids.numel()
        self.grow_for(n)
        need = dks_workspace_size(n)
        if self._ws is None or self._ws.numel() < need + 256:
            self._ws = new_workspace(ids.device, need)
        rows, hit, _ = dks_lookup_or_insert(self.keys, self.krows, self.stamps, self.values, self.max_rows,
                                            self.next_row, ids, now, True, out_rows=out_rows, out_hit=out_hit,
                                            out_stats=out_stats, ws=self._ws, stream=self.stream)
        self._offered += n
        if self._pinned:
            s = self.stream if self.stream is not None else torch.cuda.current_stream(ids.device)
            pin, ev = self._pinned.popleft()
            with torch.cuda.stream(s):
                pin.copy_(self.next_row, non_blocking=True)
                ev.record(s)
            self._pending.append((ev, pin, self._offered))
        return rows, hit
