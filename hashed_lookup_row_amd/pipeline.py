"""Two-stream schedules of the cache's per-batch work.

The work of a batch splits into a part that needs only IDs and rows (MPZCH
lookup/insert, hashed-row mapping, the grouping half of Writeback / SGD-sum /
EMA) and a part that moves row data (zero-filling new rows, gather, applying
updates).  The first part is latency-bound and light on HBM, the second is
HBM-bound, so they overlap well: the ID-side work of batch t runs on a lookup
stream while the row traffic of batch t-1 runs on the compute stream, the
overlap of the dispatch (embedding lookup) and compute streams in "MTGR:
Industrial-Scale Generative Recommendation Framework in Meituan", sec. 3.5.

Only kernels of libhlr.so run; this module enqueues them on two torch streams
and orders them with events.  Every schedule gives the same results as the
same calls made one after another on one stream (the tests check this against
the oracle).

Ordering, per batch t (ring of `depth` buffer sets, k = t mod depth):
  lookup stream:  wait compute(t - depth) done  ->  ID-side calls of t into set k, an event after each
  compute stream: wait for the event each row-side call needs  ->  row-side calls of t  ->  record done(t)
A lookup without `values` leaves the rows it inserts untouched; the compute
stream zero-fills them (mpzch_zero_inserted) after batch t-1's Writeback has
written them and before batch t gathers them, which is the order a single
stream would give.

The compute stream is the caller's current stream when the pipeline is built.
Inputs handed to step() (IDs, keys, rows, masks) must already be written when
step() is called (for example uploaded and synchronised ahead of time): the
lookup stream does not wait for the compute stream.
"""
from __future__ import annotations

import ctypes
from collections import deque

import torch

from ._hip import hip
from . import (WB_LAST_WINS, WB_SGD_SUM, HLRError, _check, _dev, _own_ws, clear_marks, ema_update_apply,
               ema_workspace_size, gather_rows, hashed_rows, load_library, mark_rows,
               mpzch_lookup_or_insert, mpzch_workspace_size, mpzch_zero_inserted, new_workspace, quantize_rows_int8,
               writeback_apply, writeback_plan, writeback_plan_rows, writeback_workspace_size,
               memory_layer_step_workspace_size)


class _Ring:
    """Ring of `depth` buffer sets shared by a lookup stream and the compute stream.

    Events marks[k][j] are recorded on the lookup stream at the j-th point the compute
    stream has to wait for; done[k] is recorded on the compute stream when set k is free.
    Raw HIP events and stream handles keep the host cost of a step low."""

    def __init__(self, device, depth, points=1, lookup=None):
        self.device = torch.device(device)
        self.depth = depth
        self.lookup = lookup if lookup is not None else torch.cuda.Stream(self.device)  # default priority
        self.compute = torch.cuda.current_stream(self.device)
        self.ls, self.cs = self.lookup.cuda_stream, self.compute.cuda_stream
        self.hip = hip()
        self.marks = [[self.hip.event() for _ in range(points)] for _ in range(depth)]
        self.done = [self.hip.event() for _ in range(depth)]
        self.fork = self.hip.event()
        self.t = 0

    def restart(self):
        """Orders the lookup stream after everything enqueued on the compute stream so far and
        starts a fresh ring (no waits on earlier ring events).  Needed to begin a graph capture
        on the compute stream: the lookup stream then joins the capture from this point."""
        self.hip.record(self.fork, self.cs)
        self.hip.wait(self.ls, self.fork)
        self.t = 0

    def begin_lookup(self):
        k = self.t % self.depth
        if self.t >= self.depth:
            self.hip.wait(self.ls, self.done[k])
        return k

    def mark(self, k, j):
        self.hip.record(self.marks[k][j], self.ls)

    def wait(self, k, j):
        self.hip.wait(self.cs, self.marks[k][j])

    def end_compute(self, k):
        self.hip.record(self.done[k], self.cs)
        self.t += 1


def _on(stream, *tensors):
    """Tells torch's allocator that `stream` uses these caller tensors."""
    for x in tensors:
        if x is not None:
            x.record_stream(stream)


class MemoryLayerPipeline:
    """MPZCH lookup/insert + gather + Writeback (last occurrence wins, lr = 1) per batch.

    lookup stream:  mpzch_lookup_or_insert(values=None) -> writeback_plan(LAST_WINS)
    compute stream: mpzch_zero_inserted -> gather_rows -> writeback_apply(LAST_WINS)
                    (native: no zero-fill; the gather and the apply read the rows the lookup
                    inserted as zero through its hit mask, with the same results)
    step() returns the gathered rows (on the compute stream) and leaves rows/hit of
    the batch in ring slot k (`rows(k)`, `hit(k)`).

    With native=True (the default) a batch is enqueued by one library call
    (memory_layer_step) whenever no per-call hook (mark, publisher) is given; the
    schedule and the results are the same as the call-by-call path.

    Lookahead (native only): prefetch(ids, now) enqueues the ID-side half of a later
    batch right away; the step() of that batch (same ids tensor, same now) then
    enqueues only its row traffic.  Calling prefetch(batch t+1) before step(batch t)
    lets the lookup kernels of t+1 run beside the row traffic of t instead of after
    it (the data loader usually has the next batch's IDs early).  At most `depth`
    batches may be looked up and not yet stepped."""

    def __init__(self, identity, stamps, values, probes, n, depth=2, native=True):
        self.identity, self.stamps, self.values, self.probes, self.n = identity, stamps, values, probes, n
        dev = values.device
        self.ring = _Ring(dev, depth, points=2)
        C, D = values.shape
        wsb = writeback_workspace_size(C, D, n, WB_LAST_WINS)
        self._rows = [torch.empty(n, dtype=torch.int64, device=dev) for _ in range(depth)]
        self._hit = [torch.empty(n, dtype=torch.int8, device=dev) for _ in range(depth)]
        self._ws = [new_workspace(dev, wsb) for _ in range(depth)]  # the call-by-call Writeback plans
        self._mz_ws = new_workspace(dev, mpzch_workspace_size(n))
        self.native = native
        if native:
            for t, name, dt in ((identity, "identity", torch.int64), (stamps, "stamps", torch.int64),
                                (values, "values", torch.float32)):
                _dev(t, name, dt)
            self._fn = load_library().memory_layer_step
            # the one-call step's row groupings, apart from the call-by-call plans: the step keeps its
            # tables clear from batch to batch, which a call-by-call plan written there would break
            ssb = memory_layer_step_workspace_size(n, C)
            self._sws = [new_workspace(dev, ssb) for _ in range(depth)]
            self._smz_ws = new_workspace(dev, mpzch_workspace_size(n))  # the step's own, laid out for n
            self._mz = _own_ws(self._smz_ws, mpzch_workspace_size(n))
            self._wb = [_own_ws(w, ssb) for w in self._sws]
            self._prepare()
            self._const = (identity.data_ptr(), stamps.data_ptr(), values.data_ptr(), C, int(probes), D)
        self._tl = 0              # lookup halves enqueued (the ring's t counts row halves)
        self._ahead = deque()     # (ids, now, slot, evicted, stats) looked up ahead of their step()

    def _prepare(self):
        """Clears the one-call step's workspaces (its tables stay clear from batch to batch after that);
        on the compute stream, which the lookup stream waits for at its first batch (restart)."""
        init = load_library().memory_layer_step_workspace_init
        C = self.values.shape[0]
        mz, mzb = self._mz
        for wb, wbb in self._wb:
            _check(init(mz, mzb, wb, wbb, self.n, C, self.ring.cs), "memory_layer_step_workspace_init")
        self.ring.restart()

    def restart(self):
        if self._ahead:
            raise HLRError("restart() with batches looked up ahead of step()")
        self.ring.restart()
        self._tl = 0

    def rows(self, k):
        return self._rows[k]

    def hit(self, k):
        return self._hit[k]

    def prefetch(self, ids, now, evicted=None, stats=None):
        """Enqueues the ID-side half (lookup/insert, grouping by row) of a later batch now; returns its ring
        slot (rows(k), hit(k) hold the batch's rows and hit mask until its row half is done)."""
        if not self.native:
            raise HLRError("prefetch() needs native=True")
        r = self.ring
        if self._tl - r.t >= r.depth:  # lookup j reuses the slot of row half j - depth, which must be enqueued
            raise HLRError(f"at most {r.depth} batches may be looked up and not yet stepped")
        self._check_ids(ids, evicted, stats)
        k = self._tl % r.depth
        self._call(ids, now, None, None, evicted, stats, None, k, 1)
        self._ahead.append((ids, int(now), k, evicted, stats))
        return k

    def step(self, ids, now, e, out=None, evicted=None, stats=None, mark=None, publisher=None, gather_events=None):
        """mark: optional callable, called with 0 just before and 1 just after the gather is
        enqueued on the compute stream (e.g. to record timing events there).
        gather_events: optional pair of HIP events recorded on the compute stream around the gather.
        publisher: optional RESPublisher; it collects the rows this batch wrote and publishes
        them at its own cadence."""
        if self.native and mark is None and publisher is None:
            return self._native_step(ids, now, e, out, evicted, stats, gather_events)
        if self._ahead:
            raise HLRError("a step with mark or publisher cannot follow prefetch()")
        if self.native and mark is None:
            return self._native_published_step(ids, now, e, out, evicted, stats, gather_events, publisher)
        if gather_events is not None:
            if mark is not None:
                raise ValueError("give mark or gather_events, not both")
            h, cs = self.ring.hip, self.ring.cs
            mark = lambda j: h.record(gather_events[j], cs)  # noqa: E731
        r = self.ring
        k = r.begin_lookup()
        _on(r.lookup, ids, evicted, stats)
        mpzch_lookup_or_insert(self.identity, self.stamps, None, self.probes, ids, now, True,
                               out_rows=self._rows[k], out_hit=self._hit[k], out_evicted=evicted, out_stats=stats,
                               ws=self._mz_ws, stream=r.ls)
        r.mark(k, 0)
        writeback_plan(self.values.shape[0], self._rows[k], self._ws[k], WB_LAST_WINS, stream=r.ls)
        r.mark(k, 1)
        if publisher is not None:
            publisher.after_lookup(self)
        r.wait(k, 0)
        mpzch_zero_inserted(self.values, self._rows[k], self._hit[k], stream=r.cs)
        if mark is not None:
            mark(0)
        out = gather_rows(self.values, self._rows[k], out, stream=r.cs)
        if mark is not None:
            mark(1)
        r.wait(k, 1)
        writeback_apply(self.values, e, self._ws[k], WB_LAST_WINS, 1.0, stream=r.cs)
        if publisher is not None:
            publisher.after_apply(self, self._ws[k])
        r.end_compute(k)
        return out, k

    def _check_ids(self, ids, evicted, stats):
        n = ids.numel()
        if not (ids.is_cuda and ids.dtype == torch.int64 and ids.is_contiguous() and n <= self.n):
            raise HLRError(f"ids must be a contiguous GPU int64 tensor of at most {self.n} elements")
        for t, name, m in ((evicted, "evicted", n), (stats, "stats", 6)):
            if t is not None and not (t.is_cuda and t.dtype == torch.int64 and t.is_contiguous() and t.numel() >= m):
                raise HLRError(f"{name} must be a contiguous GPU int64 tensor of at least {m} elements")

    def _native_published_step(self, ids, now, e, out, evicted, stats, gather_events, publisher):
        """The one-call step in two halves around the publisher: the lookup half, the publisher's snapshot on
        the lookup stream at this batch boundary, the compute half, then the rows it wrote added to the
        publisher's set (memory_layer_step_mark_written, from this slot's grouping) before the slot is
        released."""
        r = self.ring
        D = self._const[5]
        n = ids.numel()
        if not (e.is_cuda and e.dtype == torch.float32 and e.is_contiguous() and e.numel() == n * D):
            raise HLRError(f"e must be a contiguous GPU float32 tensor of {n} x {D} elements")
        if out is None:
            out = torch.empty((n, D), dtype=torch.float32, device=self.values.device)
        elif not (out.is_cuda and out.dtype == torch.float32 and out.is_contiguous() and out.numel() == n * D):
            raise HLRError(f"out must be a contiguous GPU float32 tensor of {n} x {D} elements")
        self._check_ids(ids, evicted, stats)
        k = self._tl % r.depth
        self._call(ids, now, e, out, evicted, stats, gather_events, k, 1)
        publisher.after_lookup(self)
        self._call(ids, now, e, out, evicted, stats, gather_events, k, 2, done=False)
        publisher.after_native_apply(self, k, n)
        r.end_compute(k)
        return out, k

    def _call(self, ids, now, e, out, evicted, stats, gather_events, k, halves, done=True):
        r = self.ring
        if halves & 1:
            _on(r.lookup, ids, evicted, stats)
            slot_free = r.done[k] if self._tl >= r.depth else None
        else:
            slot_free = None
        gb, ge = gather_events if gather_events is not None else (None, None)
        mz, mzb = self._mz
        wb, wbb = self._wb[k]
        rc = self._fn(*self._const, ids.data_ptr(), ids.numel(), self.n, int(now), None if e is None else e.data_ptr(),
                      self._rows[k].data_ptr(), self._hit[k].data_ptr(),
                      None if evicted is None else evicted.data_ptr(), None if stats is None else stats.data_ptr(),
                      None if out is None else out.data_ptr(), mz, mzb, wb, wbb, r.ls, r.cs, slot_free,
                      r.marks[k][0], r.marks[k][1], gb, ge, r.done[k] if done else None, halves)
        _check(rc, "memory_layer_step")
        if halves & 1:
            self._tl += 1

    def _native_step(self, ids, now, e, out, evicted, stats, gather_events):
        r = self.ring
        D = self._const[5]
        n = ids.numel()
        if not (e.is_cuda and e.dtype == torch.float32 and e.is_contiguous() and e.numel() == n * D):
            raise HLRError(f"e must be a contiguous GPU float32 tensor of {n} x {D} elements")
        if out is None:
            out = torch.empty((n, D), dtype=torch.float32, device=self.values.device)
        elif not (out.is_cuda and out.dtype == torch.float32 and out.is_contiguous() and out.numel() == n * D):
            raise HLRError(f"out must be a contiguous GPU float32 tensor of {n} x {D} elements")
        if self._ahead:
            pids, pnow, k, pev, pst = self._ahead[0]
            if pids is not ids or pnow != int(now) or pev is not evicted or pst is not stats:
                raise HLRError("step() must take the batches in the order prefetch() looked them up")
            self._ahead.popleft()
            self._call(ids, now, e, out, evicted, stats, gather_events, k, 2)
        else:
            self._check_ids(ids, evicted, stats)
            k = self._tl % r.depth
            self._call(ids, now, e, out, evicted, stats, gather_events, k, 3)
        r.t += 1
        return out, k


    def run(self, batches, group=4, ahead=1, gather_events=None):
        """Enqueues a known sequence of batches (eager, no graph) with one cross-stream wait per stream per
        group of `group` batches: the lookup stream enqueues the lookup halves of a group back to back and
        records one event after the last; the compute stream waits once for that event, then runs the
        group's row halves back to back and records one event after the last.  The lookup halves run
        `ahead` groups ahead of the row halves.

        A queue that reaches a wait for another stream's event before the event completes resumes about
        10 us after it completes; a wait whose event has completed costs nothing.  With the lookups a
        group ahead, each stream's waits have normally completed when reached, and the host enqueues two
        waits per group instead of two per batch.  Ring slots: batch b uses slot b mod depth, so a
        group's lookups reuse the slots of the group depth / group groups back, and wait for that
        group's row halves: depth must be a multiple of `group`, at least (ahead + 2) * group.

        batches: as StepGraph's, (ids, now, e, out) per batch, optionally followed by (evicted, stats,
        rows, hit).  gather_events: optional list of (begin, end) HIP event pairs, one per batch (or
        None), recorded on the compute stream around each batch's row pass.  Returns after enqueueing;
        the lookup stream is then ordered after everything enqueued so far (restart())."""
        if not self.native:
            raise HLRError("run() needs native=True")
        if self._ahead:
            raise HLRError("run(): finish the batches looked up ahead first")
        r = self.ring
        G, A, D = int(group), int(ahead), r.depth
        if G < 1 or A < 1 or D % G != 0 or D < (A + 2) * G:
            raise HLRError(f"run(): need group >= 1, ahead >= 1 and depth a multiple of group, at least "
                           f"(ahead + 2) * group (depth {D}, group {G}, ahead {A})")
        bs = [tuple(b) + (None,) * (8 - len(b)) for b in batches]
        nD = self._const[5]
        for b in bs:
            ids, _, e, out, ev, st, ro, ho = b
            self._check_ids(ids, ev, st)
            n = ids.numel()
            for t, name in ((e, "e"), (out, "out")):
                if not (t is not None and t.is_cuda and t.dtype == torch.float32 and t.is_contiguous() and
                        t.numel() == n * nD):
                    raise HLRError(f"{name} must be a contiguous GPU float32 tensor of {n} x {nD} elements")
            if ro is not None and not (ro.is_cuda and ro.dtype == torch.int64 and ro.numel() >= n):
                raise HLRError("rows copy must be a GPU int64 tensor of at least n elements")
            if ho is not None and not (ho.is_cuda and ho.dtype == torch.int8 and ho.numel() >= n):
                raise HLRError("hit copy must be a GPU int8 tensor of at least n elements")
        self.restart()
        h, fn, mz = r.hip, self._fn, self._mz
        ngroups = (len(bs) + G - 1) // G

        def last(gi):  # slot of the group's last batch: its events are the group's
            return (min(len(bs), gi * G + G) - 1) % D

        def lookup_group(gi):
            b0, b1 = gi * G, min(len(bs), gi * G + G)
            kl = last(gi)
            # the group's slots were last used by the full group depth / group groups back, which released
            # them all with the done event of its last slot (not this group's last slot when it is ragged)
            kfree = (b0 + G - 1) % D
            for b in range(b0, b1):
                ids, now, _, _, ev, st, ro, ho = bs[b]
                k = b % D
                wb, wbb = self._wb[k]
                _on(r.lookup, ids, ev, st)
                rc = fn(*self._const, ids.data_ptr(), ids.numel(), self.n, int(now), None,
                        self._rows[k].data_ptr(), self._hit[k].data_ptr(), None if ev is None else ev.data_ptr(),
                        None if st is None else st.data_ptr(), None, mz[0], mz[1], wb, wbb, r.ls, r.cs,
                        r.done[kfree] if (b == b0 and b >= D) else None, None, r.marks[kl][1] if b == b1 - 1 else None,
                        None, None, None, 1)
                _check(rc, "memory_layer_step")
                n = ids.numel()
                if ro is not None:
                    h.copy_d2d(ro.data_ptr(), self._rows[k].data_ptr(), 8 * n, r.ls)
                if ho is not None:
                    h.copy_d2d(ho.data_ptr(), self._hit[k].data_ptr(), n, r.ls)

        def compute_group(gi):
            b0, b1 = gi * G, min(len(bs), gi * G + G)
            kl = last(gi)
            for b in range(b0, b1):
                ids, now, e, out, ev, st, _, _ = bs[b]
                k = b % D
                wb, wbb = self._wb[k]
                _on(r.compute, e, out)
                gb, ge = gather_events[b] if gather_events is not None and gather_events[b] is not None \
                    else (None, None)
                rc = fn(*self._const, None, ids.numel(), self.n, int(now), e.data_ptr(),
                        self._rows[k].data_ptr(), self._hit[k].data_ptr(), None, None, out.data_ptr(),
                        mz[0], mz[1], wb, wbb, r.ls, r.cs, None, None, r.marks[kl][1] if b == b0 else None,
                        gb, ge, r.done[kl] if b == b1 - 1 else None, 2)
                _check(rc, "memory_layer_step")

        for gi in range(min(A, ngroups)):
            lookup_group(gi)
        for gi in range(ngroups):
            if gi + A < ngroups:
                lookup_group(gi + A)
            compute_group(gi)
        self.restart()


class StepGraph:
    """A fixed sequence of Memory-Layer batches enqueued once, as one HIP graph, through a native
    MemoryLayerPipeline: the same library calls in the same two-stream schedule with lookahead
    (batch t+1's lookup half before batch t's row half), captured from the compute stream, the
    lookup stream joining through the ring's fork event and rejoining at the end.  Replaying the
    graph runs the whole sequence with one host call: the eager schedule spends about 20 us of host
    time on every cross-stream wait, and two per batch make it host-bound.

    batches: list of (ids, now, e, out) per batch, in order, optionally followed by (evicted, stats,
    rows, hit): int64[n] evicted IDs and int64[6] stats written by the lookup as in
    mpzch_lookup_or_insert, and int64[n] rows / int8[n] hit buffers that receive copies of the batch's
    rows and hit mask (copied on the lookup stream while the ring slot still holds them).
    ahead: how many batches the lookup half runs ahead of the row half (at most depth - 1).  A wait on
    another stream's event takes about 10 us to resolve when the event completes after the waiting
    queue reached it; with the lookup two batches ahead, the event the row half of batch t waits for
    completed a whole row pass earlier.
    group: when given, the graph captures the grouped schedule of MemoryLayerPipeline.run(batches,
    group, ahead) instead (ahead then counts groups): one cross-stream dependency per stream and group
    of batches rather than one per batch, which the graph's queues resolve faster (73.3-73.9 against
    75.5-76.1 us per batch for groups of 4).  (HIP events
    recorded inside a capture cannot be timed on this runtime, so the row pass is not timed inside a
    graph.)  Every `now` must stay valid when the
    graph runs: a graph is meant to be replayed once for the state it was captured for, or again only
    after that state has been restored (the MPZCH stamps must stay below every `now`)."""

    def __init__(self, pipe: MemoryLayerPipeline, batches, ahead=1, group=None):
        if not pipe.native:
            raise HLRError("StepGraph needs a native MemoryLayerPipeline")
        if pipe._ahead:
            raise HLRError("StepGraph: finish the batches looked up ahead first")
        r = pipe.ring
        ahead = int(ahead)
        if group is None and not 1 <= ahead < r.depth:
            raise HLRError(f"StepGraph: ahead must be in [1, depth - 1] = [1, {r.depth - 1}]")
        if group is not None:
            G = int(group)
            if G < 1 or ahead < 1 or r.depth % G != 0 or r.depth < (ahead + 2) * G:
                raise HLRError(f"StepGraph: need group >= 1, ahead >= 1 and depth a multiple of group, at least "
                               f"(ahead + 2) * group (depth {r.depth}, group {G}, ahead {ahead})")
        if not r.cs:
            raise HLRError("StepGraph: the legacy default stream cannot be captured; build the pipeline while a "
                           "non-default torch stream is current")
        h = r.hip
        self.hip, self.stream, self.pipe = h, r.cs, pipe
        self.graph = self.exec = None
        h.begin_capture(r.cs)
        try:
            if group is not None:
                pipe.run(batches, group=group, ahead=ahead)  # begins by ordering the lookup stream after cs
            else:
                pipe.restart()
                bs = [tuple(b) + (None,) * (8 - len(b)) for b in batches]

                def look(b):
                    ids, now, _, _, ev, st, rows_out, hit_out = b
                    k = pipe.prefetch(ids, now, evicted=ev, stats=st)
                    n = ids.numel()
                    if rows_out is not None:
                        h.copy_d2d(rows_out.data_ptr(), pipe.rows(k).data_ptr(), 8 * n, r.ls)
                    if hit_out is not None:
                        h.copy_d2d(hit_out.data_ptr(), pipe.hit(k).data_ptr(), n, r.ls)

                for b in bs[:ahead]:
                    look(b)
                for k, (ids, now, e, out, ev, st, _, _) in enumerate(bs):
                    if k + ahead < len(bs):
                        look(bs[k + ahead])
                    pipe.step(ids, now, e, out=out, evicted=ev, stats=st)
            join = h.event()
            h.record(join, r.ls)
            h.wait(r.cs, join)
        finally:
            self.graph = h.end_capture(r.cs)
        self.exec = h.instantiate(self.graph)
        pipe.restart()

    def replay(self):
        """Runs the sequence on the compute stream; the pipeline's lookup stream is then ordered after it
        (and its ring restarted), so eager batches may follow."""
        self.hip.launch_graph(self.exec, self.stream)
        self.pipe.restart()

    def __del__(self):
        try:
            self.hip.destroy_graph(self.graph, self.exec)
        except Exception:
            pass


class RunGraph:
    """A pipeline's grouped schedule (MemoryLayerPipeline.run or EMAPipeline.run with the same batches,
    group and ahead) captured once as one HIP graph from the compute stream, every lookup stream joining
    back at the end; replay() runs it.  The graph's queues resolve the cross-stream dependencies of the
    schedule faster than the same calls enqueued eagerly (a CS3 step 182.8 against 187.0-187.6 us, same
    box).  As for StepGraph, the batches' inputs and outputs must stay valid and the state must be fit
    for the recorded `now` values (or the step order of an EMA) when the graph is replayed."""

    def __init__(self, pipe, batches, group=4, ahead=1):
        rings = list(getattr(pipe, "rings", None) or [pipe.ring])
        r0 = pipe.ring
        if not r0.cs:
            raise HLRError("RunGraph: the legacy default stream cannot be captured; build the pipeline while a "
                           "non-default torch stream is current")
        h = r0.hip
        self.hip, self.stream, self.pipe = h, r0.cs, pipe
        self.graph = self.exec = None
        h.begin_capture(r0.cs)
        try:
            pipe.run(batches, group=group, ahead=ahead)
            for r in rings:
                join = h.event()
                h.record(join, r.ls)
                h.wait(r0.cs, join)
        finally:
            self.graph = h.end_capture(r0.cs)
        self.exec = h.instantiate(self.graph)
        pipe.restart()

    def replay(self):
        """Runs the schedule on the compute stream; the lookup streams are then ordered after it."""
        self.hip.launch_graph(self.exec, self.stream)
        self.pipe.restart()

    def __del__(self):
        try:
            self.hip.destroy_graph(self.graph, self.exec)
        except Exception:
            pass


class HashedTablesPipeline:
    """Hashed tables (row = mix(key) mod rows): gather + duplicate-summed SGD per table.

    lookup stream:  hashed_rows -> writeback_plan(SGD_SUM), table by table
    compute stream: gather_rows -> writeback_apply(SGD_SUM, lr), table by table
    With batch=False there is one ring per table, so a table's next batch may plan while other
    tables apply.  With batch=True (the default; distinct tables of one dim) the tables go in groups
    of `group` (at most eight), one ring per group: the lookup stream makes the group's rows, then
    its plans; the compute stream waits once for the rows, gathers table by table, waits once for
    the plans and applies the whole group in one writeback_apply_batch call (one kernel launch per
    group instead of one per table; the long duplicate chains of the group's tables overlap).  mark is then
    called with ("apply", -1 - group index, 0 | 1).  Groups of four suit the 8 tables of [DLRM]:
    with all eight in one group the plan chains (many small kernels) wait behind the long gathers
    and applies of the group before."""

    def __init__(self, tables, n, depth=2, batch=True, group=4):
        self.tables, self.n = tables, n
        dev = tables[0].device
        self.batch = (bool(batch) and len({id(t) for t in tables}) == len(tables) and
                      len({t.shape[1] for t in tables}) == 1)
        g = max(1, min(int(group), 8)) if self.batch else 1
        self.groups = [list(range(i, min(i + g, len(tables)))) for i in range(0, len(tables), g)]
        first = _Ring(dev, depth, points=2)
        self.rings = [first] + [_Ring(dev, depth, points=2, lookup=first.lookup) for _ in
                                range((len(self.groups) if self.batch else len(tables)) - 1)]
        self._rows = [[torch.empty(n, dtype=torch.int64, device=dev) for _ in range(depth)] for _ in tables]
        self._ws = [[new_workspace(dev, writeback_workspace_size(t.shape[0], t.shape[1], n, WB_SGD_SUM))
                     for _ in range(depth)] for t in tables]
        if self.batch:
            from . import _WbApply
            self._lib = load_library()
            self._arr = [[(_WbApply * len(grp))() for _ in range(depth)] for grp in self.groups]
            for gi, grp in enumerate(self.groups):
                for k, arr in enumerate(self._arr[gi]):
                    for j, i in enumerate(grp):
                        t = tables[i]
                        _dev(t, "table", torch.float32)
                        need = self._lib.writeback_rows_workspace_size(t.shape[0], t.shape[1], n, WB_SGD_SUM)
                        w, wb = _own_ws(self._ws[i][k], need)
                        arr[j].table, arr[j].num_rows, arr[j].dim = t.data_ptr(), t.shape[0], t.shape[1]
                        arr[j].ws, arr[j].ws_bytes = w.value, wb

    def restart(self):
        for r in self.rings:
            r.restart()

    def rows(self, table, k):
        return self._rows[table][k]

    def step(self, keys, grads, lr, outs=None, mark=None):
        """keys[i], grads[i]: table i's keys (int64[n]) and gradients ([n, dim]); returns the gathered rows.
        mark: optional callable, called on the compute stream with ("gather" | "apply", table, 0 | 1)
        just before (0) and after (1) each gather and apply is enqueued."""
        mark = mark if mark is not None else (lambda tag: None)
        if self.batch:
            return self._step_batch(keys, grads, lr, outs, mark)
        ks = []
        for i, t in enumerate(self.tables):
            r = self.rings[i]
            k = r.begin_lookup()
            _on(r.lookup, keys[i])
            hashed_rows(keys[i], t.shape[0], out=self._rows[i][k], stream=r.ls)
            r.mark(k, 0)
            writeback_plan(t.shape[0], self._rows[i][k], self._ws[i][k], WB_SGD_SUM, stream=r.ls)
            r.mark(k, 1)
            ks.append(k)
        res = []
        for i, t in enumerate(self.tables):
            r, k = self.rings[i], ks[i]
            r.wait(k, 0)
            mark(("gather", i, 0))
            res.append(gather_rows(t, self._rows[i][k], None if outs is None else outs[i], stream=r.cs))
            mark(("gather", i, 1))
            r.wait(k, 1)
            mark(("apply", i, 0))
            writeback_apply(t, grads[i], self._ws[i][k], WB_SGD_SUM, lr, stream=r.cs)
            mark(("apply", i, 1))
            r.end_compute(k)
        return res

    def _step_batch(self, keys, grads, lr, outs, mark):
        ks = []
        for gi, grp in enumerate(self.groups):
            r = self.rings[gi]
            k = r.begin_lookup()
            for i in grp:
                _on(r.lookup, keys[i])
                hashed_rows(keys[i], self.tables[i].shape[0], out=self._rows[i][k], stream=r.ls)
            r.mark(k, 0)
            for i in grp:
                writeback_plan(self.tables[i].shape[0], self._rows[i][k], self._ws[i][k], WB_SGD_SUM, stream=r.ls)
            r.mark(k, 1)
            ks.append(k)
        res = []
        for gi, grp in enumerate(self.groups):
            r, k = self.rings[gi], ks[gi]
            r.wait(k, 0)
            for i in grp:
                mark(("gather", i, 0))
                res.append(gather_rows(self.tables[i], self._rows[i][k], None if outs is None else outs[i],
                                       stream=r.cs))
                mark(("gather", i, 1))
            arr = self._arr[gi][k]
            for j, i in enumerate(grp):
                g = grads[i]
                _dev(g, "grads", torch.float32)
                if g.numel() != self.n * self.tables[i].shape[1]:
                    raise ValueError(f"grads[{i}] must hold n x dim values")
                arr[j].src, arr[j].n, arr[j].lr = g.data_ptr(), self.n, float(lr)
            r.wait(k, 1)
            mark(("apply", -1 - gi, 0))
            rc = self._lib.writeback_apply_batch(len(grp), ctypes.cast(arr, ctypes.c_void_p), WB_SGD_SUM, r.cs)
            if rc != 0:
                _check(rc, "writeback_apply_batch")
            mark(("apply", -1 - gi, 1))
            r.end_compute(k)
        return res


class EMAPipeline:
    """EMA row updates of several tables per batch (CS3: CTS on positives, CMS on all).

    lookup streams: the plan of every update of the batch
    compute stream: ema_update_apply for every update
    `tables` fixes, per update, the table and its row count; step() takes the rows, masks and values
    of each update.  A masked update whose rows tensor is also the rows of an unmasked update of a
    table with as many rows (CTS beside CMS on the same user or item IDs) gets its plan cut out of
    that update's plan (ema_update_plan_subset: no second sort), unless derive=False.  Plans are made
    unmasked first; when every update has its own table the applies follow the plans' order (updates
    of different tables are independent), else the order given.

    Updates keyed by different rows tensors have independent plans (CS3: the user-keyed ones and the
    item-keyed ones); with lookup_streams = 2 they are planned on two lookup streams at once.  A plan
    is a chain of short, latency-bound kernels, so two chains side by side take about as long as one.
    With batch=True (distinct tables of one dim, at most four) all the applies of a batch are one
    ema_update_apply_batch call once every plan is ready: their long dependent chains then run side by
    side instead of one update after another; mark is then called with ("apply", -1, 0 | 1).

    With pairs=True the tables come in pairs (tables[2k], tables[2k + 1]: a user-keyed and an item-keyed
    cache with the same rule, as CS3's CTS and CMS pairs), at most four pairs of one dim; updates 2k and
    2k + 1 of every batch take the same mask tensor (or None) and the same (a, b).  Each pair is planned by
    one sort of both updates' positions (ema_update_plan_pair; with derive, a masked pair whose rows tensors
    are those of an unmasked pair of the same tables' sizes is cut out of that pair's plan, on that pair's
    lookup stream; other pairs go round-robin over the lookup streams), and all pairs are applied by one
    ema_update_apply_pairs launch: half the plan launches of the unpaired schedule."""

    def __init__(self, tables, n, depth=2, derive=True, lookup_streams=2, batch=True, pairs=False):
        self.tables, self.n, self.derive = tables, n, derive
        dev = tables[0].device
        self.pairs = bool(pairs)
        self._lookup_streams = lookup_streams
        if self.pairs:
            self._init_pairs(tables, n, depth, dev)
            return
        self.rings = [_Ring(dev, depth, points=len(tables)) for _ in range(max(1, int(lookup_streams)))]
        self.ring = self.rings[0]
        self._ws = [[new_workspace(dev, ema_workspace_size(t.shape[0], t.shape[1], n)) for t in tables]
                    for _ in range(depth)]
        self._distinct = len({id(t) for t in tables}) == len(tables)
        # one launch for all the applies of a batch (ema_update_apply_batch): distinct tables of one dim
        self.batch = bool(batch) and self._distinct and len(tables) <= 4 and len({t.shape[1] for t in tables}) == 1
        # the plan calls and the batch go straight to the library (a step is enqueued often enough that the
        # binding's per-call checks and conversions show up in its host time): workspace pointers per slot
        self._lib = load_library()
        need = [self._lib.ema_update_rows_workspace_size(t.shape[0], t.shape[1], n) for t in tables]
        self._wsp = [[_own_ws(w, need[i]) for i, w in enumerate(slot)] for slot in self._ws]
        self._wsp = [[(p.value, b) for p, b in slot] for slot in self._wsp]
        if self.batch:
            from . import _EmaApply
            self._arr = [(_EmaApply * len(tables))() for _ in range(depth)]
            for k, arr in enumerate(self._arr):
                for i, t in enumerate(tables):
                    _dev(t, "table", torch.float32)
                    arr[i].table, arr[i].num_rows, arr[i].dim = t.data_ptr(), t.shape[0], t.shape[1]
                    arr[i].ws, arr[i].ws_bytes = self._wsp[k][i]

    def _init_pairs(self, tables, n, depth, dev):
        from . import _EmaApplyPair
        P = len(tables) // 2
        if len(tables) % 2 or not 1 <= P <= 4:
            raise HLRError("pairs=True needs an even number of tables, at most eight")
        if len({id(t) for t in tables}) != len(tables) or len({t.shape[1] for t in tables}) != 1:
            raise HLRError("pairs=True needs distinct tables of one dim")
        for t in tables:
            _dev(t, "table", torch.float32)
        self._distinct, self.batch, self._np = True, True, P
        self.rings = [_Ring(dev, depth, points=1) for _ in range(max(1, int(self._lookup_streams)))]
        self.ring = self.rings[0]
        self._lib = load_library()
        D = tables[0].shape[1]
        need = [self._lib.ema_update_pair_workspace_size(tables[2 * k].shape[0], tables[2 * k + 1].shape[0], D, n)
                for k in range(P)]
        if min(need) == 0:
            raise HLRError("pair sizes out of range (rows of a pair below 2^31 - 1, 2n within the batch limit)")
        self._ws = [[new_workspace(dev, need[k]) for k in range(P)] for _ in range(depth)]
        self._wsp = [[_own_ws(w, need[k]) for k, w in enumerate(slot)] for slot in self._ws]
        self._wsp = [[(p.value, b) for p, b in slot] for slot in self._wsp]
        self._arr = [(_EmaApplyPair * P)() for _ in range(depth)]
        for k, arr in enumerate(self._arr):
            for j in range(P):
                t0, t1 = tables[2 * j], tables[2 * j + 1]
                arr[j].table0, arr[j].num_rows0 = t0.data_ptr(), t0.shape[0]
                arr[j].table1, arr[j].num_rows1 = t1.data_ptr(), t1.shape[0]
                arr[j].dim = D
                arr[j].ws, arr[j].ws_bytes = self._wsp[k][j]

    def _pair_sources(self, rows, masks, coeffs):
        """Per pair, the unmasked pair its plan is cut from (or None), and the planning order."""
        P, T = self._np, self.tables
        for k in range(P):
            if masks[2 * k] is not masks[2 * k + 1]:
                raise HLRError(f"updates {2 * k} and {2 * k + 1} form a pair and take the same mask")
            if tuple(coeffs[2 * k]) != tuple(coeffs[2 * k + 1]):
                raise HLRError(f"updates {2 * k} and {2 * k + 1} form a pair and take the same (a, b)")
            if rows[2 * k].numel() != rows[2 * k + 1].numel():
                raise HLRError(f"updates {2 * k} and {2 * k + 1} form a pair and take as many positions")
        src = [None] * P
        if self.derive:
            for k in range(P):
                if masks[2 * k] is None:
                    continue
                for j in range(P):
                    if (masks[2 * j] is None and rows[2 * j] is rows[2 * k] and rows[2 * j + 1] is rows[2 * k + 1]
                            and T[2 * j].shape[0] == T[2 * k].shape[0] and T[2 * j + 1].shape[0] == T[2 * k + 1].shape[0]):
                        src[k] = j
                        break
        order = [k for k in range(P) if masks[2 * k] is None] + [k for k in range(P) if masks[2 * k] is not None]
        return src, order

    def _pair_chains(self, src):
        """Lookup stream of each pair: pairs with a plan of their own round-robin over the lookup streams, a
        pair cut out of another pair's plan on that pair's stream (it reads that plan)."""
        chain, nxt = [0] * self._np, 0
        for k in range(self._np):
            if src[k] is None:
                chain[k] = nxt % len(self.rings)
                nxt += 1
        for k in range(self._np):
            if src[k] is not None:
                chain[k] = chain[src[k]]
        return chain

    def _pair_plan(self, k, rows, masks, src, slot, ls):
        T, lib, wsp = self.tables, self._lib, self._wsp[slot]
        U, I = T[2 * k].shape[0], T[2 * k + 1].shape[0]
        n = rows[2 * k].numel()
        if src[k] is not None:
            rc = lib.ema_update_plan_subset(U + I, masks[2 * k].data_ptr(), 2 * n, wsp[src[k]][0], wsp[src[k]][1],
                                            wsp[k][0], wsp[k][1], ls)
        else:
            m = masks[2 * k]
            rc = lib.ema_update_plan_pair(U, rows[2 * k].data_ptr(), I, rows[2 * k + 1].data_ptr(),
                                          None if m is None else m.data_ptr(), n, wsp[k][0], wsp[k][1], ls)
        _check(rc, "ema pair plan")

    def _pair_apply(self, rows, vals, coeffs, slot, cs):
        arr = self._arr[slot]
        for k in range(self._np):
            arr[k].vals0, arr[k].vals1 = vals[2 * k].data_ptr(), vals[2 * k + 1].data_ptr()
            arr[k].n = rows[2 * k].numel()
            arr[k].a, arr[k].b = coeffs[2 * k][0], coeffs[2 * k][1]
        _check(self._lib.ema_update_apply_pairs(self._np, ctypes.addressof(arr), cs), "ema_update_apply_pairs")

    def _pair_step(self, rows, masks, vals, coeffs, mark):
        src, order = self._pair_sources(rows, masks, coeffs)
        chain = self._pair_chains(src)
        used = sorted(set(chain))
        seen = {}
        self._check_ids(rows, masks, seen)
        self._check_vals(rows, vals)
        ks = {c: self.rings[c].begin_lookup() for c in used}
        k = ks[used[0]]
        for c in used:
            _on(self.rings[c].lookup, *seen.values())
        for j in order:
            self._pair_plan(j, rows, masks, src, k, self.rings[chain[j]].ls)
        for c in used:
            self.rings[c].mark(k, 0)
        for c in used:
            self.rings[c].wait(k, 0)
        _on(self.ring.compute, *vals)
        mark(("apply", -1, 0))
        self._pair_apply(rows, vals, coeffs, k, self.ring.cs)
        mark(("apply", -1, 1))
        for r in self.rings:  # every ring advances each step, so their slots stay in step
            r.end_compute(k)

    def restart(self):
        for r in self.rings:
            r.restart()

    def _sources(self, rows, masks):
        """For each update, the unmasked update its plan is cut from (or None), and the planning order."""
        src = [None] * len(self.tables)
        if self.derive:
            for i, m in enumerate(masks):
                if m is None:
                    continue
                for j, mj in enumerate(masks):
                    if mj is None and rows[j] is rows[i] and self.tables[j].shape[0] == self.tables[i].shape[0]:
                        src[i] = j
                        break
        order = [i for i in range(len(masks)) if masks[i] is None] + \
                [i for i in range(len(masks)) if masks[i] is not None]
        return src, order

    def _chains(self, rows):
        """Lookup stream of each update: updates with the same rows tensor share one (a cut plan
        reads its source plan), distinct rows tensors go round-robin over the lookup streams."""
        keys = {}
        return [keys.setdefault(id(r), len(keys)) % len(self.rings) for r in rows]

    def _check_ids(self, rows, masks, seen):
        """Checks rows and masks; each distinct tensor once (seen: id -> tensor, filled in)."""
        if len(rows) != len(self.tables) or len(masks) != len(self.tables):
            raise HLRError(f"expected rows and masks of {len(self.tables)} updates")
        for i, (x, m) in enumerate(zip(rows, masks)):
            if x.numel() > self.n:
                raise HLRError(f"rows of update {i} has more than {self.n} elements")
            for t, name, dt, cnt in ((x, "rows", torch.int64, x.numel()), (m, "mask", torch.uint8, x.numel())):
                if t is not None and id(t) not in seen:
                    seen[id(t)] = t
                    if not (t.is_cuda and t.dtype == dt and t.is_contiguous() and t.numel() == cnt):
                        raise HLRError(f"{name} of update {i} must be a contiguous GPU {dt} tensor of {cnt} elements")

    def _check_vals(self, rows, vals):
        D = self.tables[0].shape[1]
        for i, v in enumerate(vals):
            if not (v.is_cuda and v.dtype == torch.float32 and v.is_contiguous() and v.numel() == rows[i].numel() * D):
                raise HLRError(f"vals of update {i} must be a contiguous GPU float32 tensor of n x {D} elements")

    def _plan(self, i, rows, masks, src, k, ls):
        """Enqueues the plan of update i of a batch into slot k on lookup stream ls."""
        t, lib, wsp = self.tables[i], self._lib, self._wsp[k]
        n = rows[i].numel()
        if src[i] is not None:
            rc = lib.ema_update_plan_subset(t.shape[0], masks[i].data_ptr(), n, wsp[src[i]][0], wsp[src[i]][1],
                                            wsp[i][0], wsp[i][1], ls)
        else:
            rc = lib.ema_update_plan(t.shape[0], rows[i].data_ptr(), None if masks[i] is None else
                                     masks[i].data_ptr(), n, wsp[i][0], wsp[i][1], ls)
        _check(rc, "ema plan")

    def step(self, rows, masks, vals, coeffs, mark=None):
        """rows[i], masks[i] (or None), vals[i], coeffs[i] = (a, b) for update i of tables[i].
        mark: optional callable, called on the compute stream with ("apply", i, 0 | 1) just
        before and after each apply is enqueued."""
        mark = mark if mark is not None else (lambda tag: None)
        if self.pairs:
            self._pair_step(rows, masks, vals, coeffs, mark)
            return
        src, order = self._sources(rows, masks)
        chain = self._chains(rows)
        used = sorted(set(chain))
        ks = {c: self.rings[c].begin_lookup() for c in used}
        k = ks[used[0]]
        seen = {}
        self._check_ids(rows, masks, seen)
        for c in used:
            _on(self.rings[c].lookup, *seen.values())
        lib = self._lib
        for i in order:
            r = self.rings[chain[i]]
            self._plan(i, rows, masks, src, k, r.ls)
            r.mark(k, i)
        cs = self.ring.cs
        if self.batch:
            for i in order:
                self.rings[chain[i]].wait(k, i)
            arr = self._arr[k]
            self._check_vals(rows, vals)
            for i in range(len(self.tables)):
                arr[i].vals, arr[i].n, arr[i].a, arr[i].b = vals[i].data_ptr(), rows[i].numel(), coeffs[i][0], coeffs[i][1]
            _on(self.ring.compute, *vals)
            mark(("apply", -1, 0))
            _check(lib.ema_update_apply_batch(len(self.tables), ctypes.addressof(arr), cs), "ema_update_apply_batch")
            mark(("apply", -1, 1))
            for r in self.rings:
                r.end_compute(k)
            return
        for i in (order if self._distinct else range(len(self.tables))):
            t = self.tables[i]
            a, b = coeffs[i]
            self.rings[chain[i]].wait(k, i)
            mark(("apply", i, 0))
            ema_update_apply(t, vals[i], a, b, self._ws[k][i], stream=cs)
            mark(("apply", i, 1))
        for r in self.rings:  # every ring advances each step, so their slots stay in step
            r.end_compute(k)

    def run(self, batches, group=4, ahead=1, apply_events=None):
        """Enqueues a known sequence of batches with one cross-stream wait per stream per group of `group`
        batches (the schedule of MemoryLayerPipeline.run): each lookup stream enqueues its plans of a group
        back to back and records one event after the last; the compute stream waits once for each such
        event, runs the group's batched applies back to back and records one event after the last.  The
        plans run `ahead` groups ahead of the applies, so a stream normally reaches a wait whose event has
        completed (free), and the host enqueues two waits per lookup stream and group instead of two per
        stream and batch (a wait plus the launch after it costs the host about 20 us, more than a launch).

        Needs batch=True (one apply launch per batch).  Ring slots: batch b uses slot b mod depth, so a
        group's plans reuse the slots of the group depth / group groups back and wait for that group's
        applies: depth must be a multiple of `group`, at least (ahead + 2) * group.  batches:
        (rows, masks, vals, coeffs) per batch, as step() takes them.  apply_events: optional list of
        (begin, end) HIP event pairs, one per group (or None), recorded on the compute stream around the
        group's applies.  Returns after enqueueing; the lookup streams are then ordered after everything
        enqueued so far (restart())."""
        if not self.batch:
            raise HLRError("run() needs batch=True (distinct tables of one dim, at most four)")
        G, A, D = int(group), int(ahead), self.ring.depth
        if G < 1 or A < 1 or D % G != 0 or D < (A + 2) * G:
            raise HLRError(f"run(): need group >= 1, ahead >= 1 and depth a multiple of group, at least "
                           f"(ahead + 2) * group (depth {D}, group {G}, ahead {A})")
        seen, plans = {}, []
        for b, x in enumerate(batches):
            if len(x) != 4:
                raise HLRError(f"batch {b}: expected (rows, masks, vals, coeffs)")
            rows, masks, vals, coeffs = x
            self._check_ids(rows, masks, seen)
            if len(vals) != len(self.tables) or len(coeffs) != len(self.tables):
                raise HLRError(f"batch {b}: expected vals and coeffs of {len(self.tables)} updates")
            self._check_vals(rows, vals)
            for v in vals:
                seen[id(v)] = v
            if self.pairs:
                src, order = self._pair_sources(rows, masks, coeffs)
                plans.append((src, order, self._pair_chains(src)))
            else:
                src, order = self._sources(rows, masks)
                plans.append((src, order, self._chains(rows)))
        if apply_events is not None and len(apply_events) < (len(batches) + G - 1) // G:
            raise HLRError("apply_events needs one entry per group")
        self.restart()
        r0, h, lib = self.ring, self.ring.hip, self._lib
        for c, r in enumerate(self.rings):  # the caller's tensors, registered once with each stream using them
            _on(r.lookup, *(t for t in seen.values() if t.dtype != torch.float32))
        _on(r0.compute, *(t for t in seen.values() if t.dtype == torch.float32))
        ngroups = (len(batches) + G - 1) // G

        def last(gi):  # slot of the group's last batch: its events are the group's
            return (min(len(batches), gi * G + G) - 1) % D

        def streams(gi):
            return sorted({c for b in range(gi * G, min(len(batches), gi * G + G)) for c in plans[b][2]})

        def lookup_group(gi):
            b0, b1 = gi * G, min(len(batches), gi * G + G)
            kl = last(gi)
            used = streams(gi)
            if b0 >= D:  # released by the full group depth / group groups back (its last slot's done event)
                for c in used:
                    h.wait(self.rings[c].ls, r0.done[(b0 + G - 1) % D])
            for b in range(b0, b1):
                rows, masks, _, _ = batches[b]
                src, order, chain = plans[b]
                if self.pairs:
                    for i in order:
                        self._pair_plan(i, rows, masks, src, b % D, self.rings[chain[i]].ls)
                    continue
                for i in order:
                    self._plan(i, rows, masks, src, b % D, self.rings[chain[i]].ls)
            for c in used:
                self.rings[c].mark(kl, 0)

        def compute_group(gi):
            b0, b1 = gi * G, min(len(batches), gi * G + G)
            kl = last(gi)
            for c in streams(gi):
                self.rings[c].wait(kl, 0)
            ev = apply_events[gi] if apply_events is not None else None
            if ev is not None:
                h.record(ev[0], r0.cs)
            for b in range(b0, b1):
                rows, _, vals, coeffs = batches[b]
                if self.pairs:
                    self._pair_apply(rows, vals, coeffs, b % D, r0.cs)
                    continue
                arr = self._arr[b % D]
                for i in range(len(self.tables)):
                    arr[i].vals, arr[i].n = vals[i].data_ptr(), rows[i].numel()
                    arr[i].a, arr[i].b = coeffs[i][0], coeffs[i][1]
                _check(lib.ema_update_apply_batch(len(self.tables), ctypes.addressof(arr), r0.cs),
                       "ema_update_apply_batch")
            if ev is not None:
                h.record(ev[1], r0.cs)
            h.record(r0.done[kl], r0.cs)

        for gi in range(min(A, ngroups)):
            lookup_group(gi)
        for gi in range(ngroups):
            if gi + A < ngroups:
                lookup_group(gi + A)
            compute_group(gi)
        self.restart()


class RESPublisher:
    """Raw Embedding Streaming, GPU side ("Memory Layer: Train the In-Model Cache for Recommendation
    Models", sec. 2): training's fresh rows are copied out while they are in HBM, deduplicated,
    quantised and pushed to serving together with the ID map and its metadata at intervals.

    Per batch (compute stream, after the Writeback apply): the rows the batch wrote are added once
    each to a written-row set (writeback_plan_rows + mark_rows; with a native pipeline the batch runs
    as the one-call step's two halves and memory_layer_step_mark_written reads the rows from the
    step's row grouping).  Every `every` batches a publish:
      compute stream: quantise the set's rows to int8 (quantize_rows_int8, per-row min-max) into a
                      device staging slot, keep the row list and count beside it, clear the set;
      lookup stream:  at that batch's boundary (after its MPZCH step, before the next one) copy
                      identity and stamps into a device snapshot slot (a consistent, step-aligned
                      snapshot);
      copy stream:    copy the snapshot and the row count to pinned host memory; the staged rows of a
                      publish are copied once its count has reached the host, at the next publish (or
                      at flush()), so no GPU stream ever waits for the host.
    Two slots alternate; each is reused only after its copies finished.  on_publish(packet), if given,
    receives each publish as host numpy arrays once complete (the host then waits for that copy).
    every = 0 publishes only on publish_now()."""

    def __init__(self, pipe, every, on_publish=None, max_rows=None):
        dev = pipe.values.device
        C, D = pipe.values.shape
        self.C, self.D, self.every, self.on_publish = C, D, int(every), on_publish
        # staging rows per publish: a batch writes at most n rows; with publish_now() only, max_rows
        # bounds the rows written between two publishes (a publish with more raises at the host)
        cap = min(C, self.every * pipe.n) if self.every > 0 else C
        self.cap = cap if max_rows is None else min(cap, int(max_rows))
        cap = self.cap
        self.copy = torch.cuda.Stream(dev)
        self.cps = self.copy.cuda_stream
        self.hip = hip()
        self._lib = load_library()
        i64 = dict(dtype=torch.int64, device=dev)
        self.flags = torch.zeros(C, dtype=torch.int32, device=dev)
        self.lst = torch.empty(C, **i64)
        self.lst_count = torch.zeros(1, **i64)
        self.plan_rows = torch.empty(pipe.n, **i64)
        self.plan_count = torch.zeros(1, **i64)
        self.st_q = [torch.empty((cap, D), dtype=torch.int8, device=dev) for _ in range(2)]
        self.st_sc = [torch.empty(cap, dtype=torch.float32, device=dev) for _ in range(2)]
        self.st_bi = [torch.empty(cap, dtype=torch.float32, device=dev) for _ in range(2)]
        self.st_rows = [torch.empty(cap, **i64) for _ in range(2)]
        self.st_cnt = [torch.zeros(1, **i64) for _ in range(2)]
        self.snap = [(torch.empty_like(pipe.identity), torch.empty_like(pipe.stamps)) for _ in range(2)]
        pin = dict(pin_memory=True)
        self.h_cnt = [torch.zeros(1, dtype=torch.int64, **pin) for _ in range(2)]
        self.h_snap = [(torch.empty(C, dtype=torch.int64, **pin), torch.empty(C, dtype=torch.int64, **pin))
                       for _ in range(2)]
        self.h_q = [torch.empty((cap, D), dtype=torch.int8, **pin) for _ in range(2)]
        self.h_sc = [torch.empty(cap, dtype=torch.float32, **pin) for _ in range(2)]
        self.h_bi = [torch.empty(cap, dtype=torch.float32, **pin) for _ in range(2)]
        self.h_rows = [torch.empty(cap, dtype=torch.int64, **pin) for _ in range(2)]
        ev = self.hip.event
        self.ev_staged = [ev() for _ in range(2)]      # compute: slot staged
        self.ev_snapped = [ev() for _ in range(2)]     # lookup: snapshot taken
        self.ev_snap_out = [ev() for _ in range(2)]    # copy: snapshot and count on the host
        self.ev_rows_out = [ev() for _ in range(2)]    # copy: staged rows on the host
        self.t = 0          # batches seen
        self.p = 0          # publishes started
        self.pending = None  # (slot, step) whose rows still have to be copied out
        self.steps = [None, None]

    def _publishing(self):
        return self.every > 0 and (self.t + 1) % self.every == 0

    def publish_now(self, pipe):
        """Publishes the rows written so far at the current batch boundary (between steps)."""
        s = self.p % 2
        if self.p >= 2:
            self.hip.wait(pipe.ring.ls, self.ev_snap_out[s])
        with torch.cuda.stream(pipe.ring.lookup):
            self.snap[s][0].copy_(pipe.identity)
            self.snap[s][1].copy_(pipe.stamps)
        self.hip.record(self.ev_snapped[s], pipe.ring.ls)
        self.hip.wait(pipe.ring.cs, self.ev_snapped[s])  # the batch boundary on both streams
        self.t -= 1
        self._publish(pipe)
        self.t += 1

    def after_lookup(self, pipe):
        """Lookup stream, after this batch's MPZCH step: snapshot identity and stamps on publishing batches."""
        if not self._publishing():
            return
        s, ls = self.p % 2, pipe.ring.ls
        if self.p >= 2:
            self.hip.wait(ls, self.ev_snap_out[s])
        ident, stamps = self.snap[s]
        with torch.cuda.stream(pipe.ring.lookup):
            ident.copy_(pipe.identity)
            stamps.copy_(pipe.stamps)
        self.hip.record(self.ev_snapped[s], ls)

    def after_apply(self, pipe, plan_ws):
        """Compute stream, after this batch's Writeback apply."""
        cs = pipe.ring.cs
        writeback_plan_rows(self.C, pipe.n, plan_ws, out_rows=self.plan_rows, out_count=self.plan_count, stream=cs)
        mark_rows(self.plan_rows, self.C, self.flags, self.lst, self.lst_count, count=self.plan_count, stream=cs)
        if self._publishing():
            self._publish(pipe)
        self.t += 1

    def after_native_apply(self, pipe, k, n):
        """Compute stream, after the compute half of a one-call step in ring slot k (n positions): the rows
        its row pass wrote join the set, read from the slot's row grouping."""
        cs = pipe.ring.cs
        wb, wbb = pipe._wb[k]
        _check(self._lib.memory_layer_step_mark_written(wb, wbb, int(n), pipe.n, self.C, self.flags.data_ptr(),
                                                        self.lst.data_ptr(), self.lst_count.data_ptr(), cs),
               "memory_layer_step_mark_written")
        if self._publishing():
            self._publish(pipe)
        self.t += 1

    def _publish(self, pipe):
        s, cs = self.p % 2, pipe.ring.cs
        if self.p >= 2:
            self.hip.wait(cs, self.ev_rows_out[s])
        with torch.cuda.stream(pipe.ring.compute):
            quantize_rows_int8(pipe.values, self.lst[:self.cap], count=self.lst_count,
                               out=(self.st_q[s], self.st_sc[s], self.st_bi[s]), stream=cs)
            self.st_rows[s].copy_(self.lst[:self.cap])
            self.st_cnt[s].copy_(self.lst_count)
        clear_marks(self.lst, self.lst_count, self.C, self.flags, stream=cs)
        self.hip.record(self.ev_staged[s], cs)
        self.hip.wait(self.cps, self.ev_staged[s])
        self.hip.wait(self.cps, self.ev_snapped[s])
        with torch.cuda.stream(self.copy):
            self.h_cnt[s].copy_(self.st_cnt[s], non_blocking=True)
            self.h_snap[s][0].copy_(self.snap[s][0], non_blocking=True)
            self.h_snap[s][1].copy_(self.snap[s][1], non_blocking=True)
        self.hip.record(self.ev_snap_out[s], self.cps)
        self.steps[s] = self.t
        if self.pending is not None:
            self._copy_rows(*self.pending)
        self.pending = (s, self.t)
        self.p += 1

    def _copy_rows(self, s, step):
        """Copies publish slot s's staged rows to the host (its count is already there)."""
        # the count was copied at that publish; wait for that copy (long done in steady state)
        self._host_wait(self.ev_snap_out[s])
        c = int(self.h_cnt[s][0])
        if c > self.cap:
            raise RuntimeError(f"publish of {c} rows exceeds the staging capacity {self.cap}: raise max_rows "
                               "or publish more often")
        with torch.cuda.stream(self.copy):
            if c > 0:
                self.h_q[s][:c].copy_(self.st_q[s][:c], non_blocking=True)
                self.h_sc[s][:c].copy_(self.st_sc[s][:c], non_blocking=True)
                self.h_bi[s][:c].copy_(self.st_bi[s][:c], non_blocking=True)
                self.h_rows[s][:c].copy_(self.st_rows[s][:c], non_blocking=True)
        self.hip.record(self.ev_rows_out[s], self.cps)
        if self.on_publish is not None:
            self._host_wait(self.ev_rows_out[s])
            self.on_publish({"step": step, "rows": self.h_rows[s][:c].numpy().copy(),
                             "q": self.h_q[s][:c].numpy().copy(), "scale": self.h_sc[s][:c].numpy().copy(),
                             "bias": self.h_bi[s][:c].numpy().copy(),
                             "identity": self.h_snap[s][0].numpy().copy(),
                             "stamps": self.h_snap[s][1].numpy().copy()})

    def _host_wait(self, e):
        self.hip.synchronize(e)

    def flush(self):
        """Completes the last publish's row copy (call after the last batch)."""
        if self.pending is not None:
            self._copy_rows(*self.pending)
            self.pending = None
