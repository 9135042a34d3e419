#!/usr/bin/env python3
"""Benchmark of the embedding-cache hot path on one MI355X.

Workload (the Memory-Layer scale cache): capacity 4,194,304 rows x 512 fp32
(8 GiB) with int64 identity and LRU stamps, 8 probes; each step merges a
32,768-ID training batch and a 32,768-ID candidate-pool batch drawn Zipf(1.05)
over a 20M-ID universe plus 0.5% never-seen IDs; item-tower vectors
e ~ N(0, 0.1).  The table is prefilled (universe inserted coldest first,
untimed) so eviction is active.

One step = mpzch_lookup_or_insert (lookup, pin, insert, LRU evict, zero-fill)
-> gather_rows (the model reads M[i]) -> writeback_rows(last occurrence wins,
lr = 1, in-batch dedup inside).  Inputs are resident in HBM before timing.

Prints one JSON line.  `value` is positions (rows) per second of the whole
step; `roofline` is the row pass ml_fused (gather and Writeback in one pass over
the batch's rows): its algorithmic bytes per launch over its mean launch time,
taken with HIP events on the compute stream, against 8 TB/s; `step_hbm` is the
whole step's algorithmic bytes over the step time; `cpu_baseline` is the CPU
oracle doing the same steps on one host core (bounded sample).  Other
workloads (--workload serving | dlrm | cs3 | dedup | res | keystore |
hbm-ceiling) print their own line of the same shape.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
# The captured graph runs the grouped schedule: the lookups of GRAPH_GROUP batches back to back, GRAPH_AHEAD
# groups ahead of the row passes (73.3-73.4 us per batch; groups of 4 one ahead 73.7-73.9, of 8 73.5-73.8;
# one cross-stream dependency per batch, lookups 1 batch ahead 76.0-76.1; same box)
GRAPH_GROUP = 4
GRAPH_AHEAD = 2
PMC_FILE = os.path.join(ROOT, "profiles", "ml_fused_memory_layer_pmc.json")


class HipTimer:
    """HIP events created with hipEventDisableSystemFence (timing only: no cache writeback/invalidate on
    record), recorded on the stream the kernels are launched on."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.pairs = []

    def event(self):
        e = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.ct.c_uint(self.DISABLE_SYSTEM_FENCE))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        return e

    def record(self, e, stream):
        rc = self.hip.hipEventRecord(e, self.ct.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_s(self, a, b):
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value * 1e-3


def src_sha(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def row_pass_sha():
    """Source hash of the Memory-Layer row pass and the plan it reads (the kernel the counters describe)."""
    h = hashlib.sha256()
    for f in ("mlstep.hip", "mlwork.hpp"):
        h.update(open(os.path.join(ROOT, "hashed_lookup_row_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--depth", type=int, default=3,
                    help="ring depth of the two-stream schedule (grouped: at least (ahead + 2) * group)")
    ap.add_argument("--schedule", default="graph", choices=["grouped", "graph", "eager"],
                    help="Memory Layer: grouped = the lookup halves of a group of batches back to back, one "
                         "cross-stream wait per stream per group (MemoryLayerPipeline.run); graph = batch by "
                         "batch with lookahead, captured as one HIP graph and replayed; eager = batch by batch "
                         "with lookahead, call by call.  CS3: eager = step by step; otherwise grouped "
                         "(EMAPipeline.run, plans a group ahead)")
    ap.add_argument("--group", type=int, default=4, help="grouped schedule: batches per group")
    ap.add_argument("--ahead", type=int, default=1, help="grouped schedule: groups the lookups run ahead")
    ap.add_argument("--no-lookahead", dest="lookahead", action="store_false",
                    help="eager: enqueue each batch's lookup with its own row traffic instead of one batch ahead")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--e-pool", type=int, default=16, help="distinct e batches cycled through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time budget for the CPU baseline")
    ap.add_argument("--ema-lookup-streams", type=int, default=2,
                    help="cs3: lookup streams the EMA plans run on (independent plans side by side)")
    ap.add_argument("--no-dlrm-batch", dest="dlrm_batch", action="store_false",
                    help="DLRM: one ring and one SGD apply launch per table instead of one batched apply")
    ap.add_argument("--dlrm-group", type=int, default=4, help="DLRM: tables per batched SGD apply")
    ap.add_argument("--ema-derive", default="auto", choices=["auto", "yes", "no"],
                    help="CS3: cut the CTS plans out of the CMS plans (yes) or sort them on their own (no); auto: "
                         "no with pairs (the two pair plans then run on two lookup streams), yes without")
    ap.add_argument("--no-ema-pairs", dest="ema_pairs", action="store_false",
                    help="CS3: plan each of the four updates on its own instead of the user- and item-keyed update "
                         "of each rule by one sort (EMAPipeline pairs)")
    ap.add_argument("--no-ema-batch", dest="ema_batch", action="store_false",
                    help="cs3: one apply launch per update instead of ema_update_apply_batch")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM counters)")
    ap.add_argument("--scale", type=float, default=1.0, help="shrink capacity/universe/batch (testing only)")
    ap.add_argument("--workload", default="memory-layer",
                    choices=["memory-layer", "serving", "dlrm", "cs3", "dedup", "res", "keystore", "hbm-ceiling"],
                    help="memory-layer (default, the headline) or one of the other rows' workloads")
    ap.add_argument("--ceiling-gib", default="1,2,4,8",
                    help="hbm-ceiling: buffer sizes in GiB (comma-separated)")
    ap.add_argument("--ceiling-kinds", default="read,write,copy,read-nt,write-nt,copy-nt",
                    help="hbm-ceiling: which sweeps to time")
    ap.add_argument("--op-events", action="store_true",
                    help="also time lookup and writeback separately (events between every call)")
    return ap.parse_args()


def copy_calibration(torch):
    dev = torch.device("cuda:0")
    nbytes = 1 << 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    t = min(ts)
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "copy_gbs": 2 * nbytes / t / 1e9}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration(torch)
        return
    sys.path.insert(0, ROOT)
    if args.workload != "memory-layer":
        {"serving": run_serving, "dlrm": run_dlrm, "cs3": run_cs3, "dedup": run_dedup,
         "res": run_res, "keystore": run_keystore, "hbm-ceiling": run_hbm_ceiling}[args.workload](args)
        return
    import hashed_lookup_row_amd as hlr
    import synth
    from hashed_lookup_row_amd.pipeline import MemoryLayerPipeline, StepGraph

    hlr.load_library()
    dev = torch.device("cuda:0")
    cfg = synth.MEMORY_LAYER
    if args.scale != 1.0:
        s = args.scale
        cfg = synth.scaled_memory_layer(capacity=int(cfg.capacity * s) // 8 * 8, universe=int(cfg.universe * s),
                                        batch=max(64, int(cfg.batch * s)), steps=cfg.steps)
    C, P, D, n = cfg.capacity, cfg.probes, cfg.dim, cfg.batch
    K, W = args.steps, args.warmup
    R = D * 4

    # ---------------------------------------------------------------- inputs
    # step t uses stream[t]: W warm-up steps, K timed headline steps, K steps timed by events (roofline),
    # K one-stream steps, one stats step
    t0 = time.time()
    prefill = synth.prefill_batches(cfg)
    stream, fc = [], 0
    for t in range(1, W + 3 * K + 3):
        ids, fc = synth.mpzch_step_ids(cfg, t, fc)
        stream.append(ids)
    print(f"[bench] generated inputs in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    identity = torch.full((C,), -1, dtype=torch.int64, device=dev)
    stamps = torch.full((C,), -1, dtype=torch.int64, device=dev)
    values = torch.zeros((C, D), dtype=torch.float32, device=dev)
    ids_dev = [torch.from_numpy(x).to(dev) for x in stream]
    npool = max(1, min(args.e_pool, W + K))
    e_pool = [synth.normal_rows(n, D, cfg.e_std, cfg.config, t + 1, device=dev) for t in range(npool)]
    rows_buf = torch.empty(n, dtype=torch.int64, device=dev)
    hit_buf = torch.empty(n, dtype=torch.int8, device=dev)
    stats = torch.zeros(6, dtype=torch.int64, device=dev)
    out = torch.empty((n, D), dtype=torch.float32, device=dev)

    # prefill (untimed): every slot receives an ID; the table starts at zero
    for k, batch in enumerate(prefill, start=1):
        hlr.mpzch_lookup_or_insert(identity, stamps, None, P, torch.from_numpy(batch).to(dev), k, insert=True,
                                   out_rows=rows_buf, out_hit=hit_buf)
    torch.cuda.synchronize()
    base_now = len(prefill)
    print(f"[bench] prefilled {len(prefill)} batches; load {(identity >= 0).float().mean().item():.4f}",
          file=sys.stderr, flush=True)

    timer = HipTimer()
    # a non-default compute stream (a HIP graph cannot be captured on the legacy default stream)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    torch.cuda.set_stream(side)
    cur = torch.cuda.current_stream(dev).cuda_stream
    G, A = args.group, args.ahead
    depth = args.depth
    if args.schedule != "eager":  # grouped (and the graph's): a multiple of the group, at least (ahead + 2) groups
        depth = max(depth, (A + 2) * G, (GRAPH_AHEAD + 2) * GRAPH_GROUP if args.schedule == "graph" else 0)
        depth = (depth + G - 1) // G * G
        if args.schedule == "graph":
            depth = (depth + GRAPH_GROUP - 1) // GRAPH_GROUP * GRAPH_GROUP
    pipe = MemoryLayerPipeline(identity, stamps, values, P, n, depth=depth)

    def piped_step(t, evs=None, ahead=None):
        # one library call per half batch (memory_layer_step): the lookup half of batch `ahead` (the next
        # one) is enqueued before the row traffic of batch t; evs: timing events around the gather
        if ahead is not None:
            pipe.prefetch(ids_dev[ahead], base_now + 1 + ahead)
        pipe.step(ids_dev[t], base_now + 1 + t, e_pool[t % npool], out=out, gather_events=evs)

    def serial_step(t, evs=None, stats_out=None):
        if evs is not None:
            timer.record(evs[0], cur)
        hlr.mpzch_lookup_or_insert(identity, stamps, values, P, ids_dev[t], base_now + 1 + t, insert=True,
                                   out_rows=rows_buf, out_hit=hit_buf, out_stats=stats_out)
        if evs is not None:
            timer.record(evs[1], cur)
        hlr.gather_rows(values, rows_buf, out=out)
        if evs is not None:
            timer.record(evs[2], cur)
        hlr.writeback_rows(values, rows_buf, e_pool[t % npool])
        if evs is not None:
            timer.record(evs[3], cur)

    # the lookup state before the first batch, for an untimed replay of the same lookups after the timed
    # regions (it gives each batch's insert count: rows the gather reads as zero instead of loading)
    id_snap, st_snap = identity.clone(), stamps.clone()
    la = args.lookahead or args.schedule != "eager"

    def two_stream(first, timed_evs, mode):
        """Batches first .. first+K-1 in the two-stream schedule `mode`, timed on the compute stream; returns
        (total seconds, host enqueue seconds, wall seconds)."""
        start, stop = timer.event(), timer.event()
        batches = [(ids_dev[first + k], base_now + 1 + first + k, e_pool[(first + k) % npool], out)
                   for k in range(K)]
        if mode == "graph":
            graph = StepGraph(pipe, batches, ahead=GRAPH_AHEAD, group=GRAPH_GROUP)  # captured, not run
            torch.cuda.synchronize()
            wall0 = time.perf_counter()
            timer.record(start, cur)
            graph.replay()
            timer.record(stop, cur)
        elif mode == "grouped":
            # timed_evs: group -> (begin, end), recorded before the group's first and after its last row pass
            gevs = None
            if timed_evs:
                gevs = [None] * K
                for g, (eb, ee) in timed_evs.items():
                    b0, b1 = g * G, min(K, g * G + G) - 1
                    gevs[b0] = (eb, ee if b1 == b0 else None)
                    if b1 != b0:
                        gevs[b1] = (None, ee)
            torch.cuda.synchronize()
            wall0 = time.perf_counter()
            timer.record(start, cur)
            pipe.run(batches, group=G, ahead=A, gather_events=gevs)
            timer.record(stop, cur)
        else:
            torch.cuda.synchronize()
            wall0 = time.perf_counter()
            timer.record(start, cur)
            if la:
                pipe.prefetch(ids_dev[first], base_now + 1 + first)
            for k in range(K):
                piped_step(first + k, timed_evs.get(k) if timed_evs else None,
                           ahead=first + k + 1 if la and k + 1 < K else None)
            timer.record(stop, cur)
        enqueue = time.perf_counter() - wall0
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        return timer.elapsed_s(start, stop), enqueue, wall

    # warm-up (eager), ending with no batch looked up ahead
    if la:
        pipe.prefetch(ids_dev[0], base_now + 1)
    for t in range(W):
        piped_step(t, ahead=t + 1 if la and t + 1 < W else None)
    torch.cuda.synchronize()

    # the headline: batches W .. W+K-1 in the chosen two-stream schedule, no events inside.  The row pass is
    # then timed with HIP events on the compute stream over the next K batches (events inside a captured
    # graph cannot be timed on this runtime): with the grouped schedule (unless the headline is the eager
    # one), one event pair around each group's back-to-back row passes, whose span / group size is the mean
    # launch duration (markers around every single launch would add their own few us to each); eager:
    # around every EV_SAMPLE_ML-th row pass.  That leg is reported beside the headline
    total_s, enqueue, wall = two_stream(W, None, args.schedule)
    ev_mode = "eager" if args.schedule == "eager" else "grouped"
    if ev_mode == "grouped":
        evs = {g: [timer.event() for _ in range(2)] for g in range((K + G - 1) // G)}
        ev_count = {g: min(K, g * G + G) - g * G for g in evs}
        ev_batches = {g: list(range(g * G, g * G + ev_count[g])) for g in evs}
    else:
        evs = {k: [timer.event() for _ in range(2)] for k in range(0, K, EV_SAMPLE_ML)}
        ev_count = {k: 1 for k in evs}
        ev_batches = {k: [k] for k in evs}
    e_total, e_enqueue, _ = two_stream(W + K, evs, ev_mode)
    timed_leg = {"schedule": ev_mode, "ms_per_step": e_total / K * 1e3, "rows_per_s": n * K / e_total,
                 "host_enqueue_us_per_step": e_enqueue / K * 1e6}
    ev_first = W + K
    span_s = np.array([timer.elapsed_s(evs[g][0], evs[g][1]) for g in sorted(evs)])
    launches = np.array([ev_count[g] for g in sorted(evs)])
    gather_s = span_s / launches  # mean launch duration in each timed span
    gather_steps = np.array([b for g in sorted(evs) for b in ev_batches[g]])
    off = K

    # the same step as three calls on one stream, over the next K batches (reported beside the headline)
    sevs = {k: [timer.event() for _ in range(4)] for k in range(K)} if args.op_events else {}
    s_start, s_stop = timer.event(), timer.event()
    timer.record(s_start, cur)
    for k in range(K):
        serial_step(W + K + off + k, sevs.get(k))
    timer.record(s_stop, cur)
    torch.cuda.synchronize()
    serial_s = timer.elapsed_s(s_start, s_stop)
    per_op = np.array([[timer.elapsed_s(e[i], e[i + 1]) for i in range(3)] for e in sevs.values()]) \
        if args.op_events else None
    # one more step after the timed regions reports the optional MPZCH stats (hit rate, inserts, ...)
    serial_step(W + 2 * K + off, None, stats)
    torch.cuda.synchronize()
    # distinct rows per timed step (for algorithmic bytes): MPZCH gives every distinct valid ID its own
    # row and no two IDs share one, so u = distinct IDs minus those without a row (overflows and
    # invalid IDs, both 0 on this workload: see stats_after)
    nb = (ev_first - W) + K  # the headline batches, then (with --graph) the call-by-call batches timed by events
    us_all = np.array([np.unique(stream[W + k]).size for k in range(nb)], dtype=np.float64)
    us = us_all[:K]
    dup = 1.0 - us.mean() / n
    # rows the gather loads: distinct rows that were already stored (a row inserted by the batch reads as
    # zero and is not loaded); insert and overflow counts from the replay of the same lookups
    rstats = torch.zeros((W + nb, 6), dtype=torch.int64, device=dev)
    for t in range(W + nb):
        hlr.mpzch_lookup_or_insert(id_snap, st_snap, None, P, ids_dev[t], base_now + 1 + t, insert=True,
                                   out_rows=rows_buf, out_hit=hit_buf, out_stats=rstats[t])
    rst = rstats.cpu().numpy()[W:W + nb].astype(np.float64)
    u_read_all = us_all - rst[:, 1] - rst[:, 3]
    u_read = u_read_all[:K]
    del id_snap, st_snap
    # the row pass (gather + Writeback in one kernel), algorithmic bytes per batch as the method defines them:
    # the gather writes every position's row and reads every distinct row, the Writeback reads the row and e
    # at its last position and writes the row, plus the row index of every position: n*R + 4u*R + 8n
    row_bytes_all = n * R + 4 * us_all * R + 8 * n
    row_bytes = row_bytes_all[:K]
    # what this one-pass design must move: each stored row read once (rows the batch inserted read as zero),
    # e at the last position, every position's output and every distinct row written, and the plan it reads
    # (a 16-byte descriptor and a 4-byte position per position at most)
    design_bytes_all = n * R + u_read_all * R + 2 * us_all * R + 20 * n
    timed = (ev_first - W) + gather_steps  # indices of the event-timed batches in the arrays above
    row_gbs = float(row_bytes_all[timed].sum() / span_s.sum() / 1e9)
    design_gbs = float(design_bytes_all[timed].sum() / span_s.sum() / 1e9)
    step_bytes = row_bytes
    ms_per_step = total_s / K * 1e3
    value = n * K / total_s

    traffic = None
    if os.path.exists(PMC_FILE):
        pmc = json.load(open(PMC_FILE))
        if pmc.get("src_sha") == row_pass_sha():
            traffic = pmc.get("traffic_bytes_per_launch")

    GG, AA = (GRAPH_GROUP, GRAPH_AHEAD) if args.schedule == "graph" else (G, A)
    line = {
        "metric": "rows/s and achieved HBM GB/s (% of peak), 512-d fp32 lookup+writeback",
        "value": value,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic (seeded Zipf ID streams, N(0,0.1) item-tower vectors)",
        "config": {
            "workload": cfg.name,
            "capacity": C, "dim": D, "probes": P, "ids_per_step": n, "universe": cfg.universe,
            "zipf_s": cfg.zipf_s, "fresh_frac": cfg.fresh_frac, "prefilled": True,
            "step": "mpzch_lookup_or_insert + gather_rows + writeback_rows(last_wins, lr=1)",
            "schedule": ("two streams: lookup (MPZCH without values, whose last kernel groups the batch's positions "
                         "by row) beside compute (one pass over the batch's rows: gather and Writeback; rows the "
                         "lookup inserts read as zero), one library call per half batch; "
                         + (f"grouped: the lookup halves of {GG} batches back to back on the lookup stream, one "
                            f"event after them; the compute stream waits once per group, then runs the group's "
                            f"row passes back to back; lookups {AA} group(s) ahead, ring depth {depth}" +
                            ("; the K timed batches captured (untimed) as one HIP graph of those calls "
                             "(MemoryLayerPipeline.run inside StepGraph) and replayed once" if args.schedule == "graph"
                             else "; enqueued call by call (MemoryLayerPipeline.run)")
                            if args.schedule != "eager" else
                            (f"lookahead: batch t+1's lookup is enqueued before batch t's row traffic, ring depth "
                             f"{depth}" if la else f"batch t's lookup with its own row traffic, ring depth {depth}")
                            + "; enqueued call by call")),
        },
        "roofline": {
            "bound": "hbm", "kernel": "ml_fused<2> (gather + Writeback, one pass over the batch's rows)",
            "achieved": row_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": row_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": float(row_bytes_all[timed].mean()),
            "avg_launch_us": float(span_s.sum() / launches.sum() * 1e6),
            "timed_launches": int(launches.sum()),
            "design_bytes_per_launch": float(design_bytes_all[timed].mean()),
            "timed_in": (f"the next {K} batches in the grouped schedule (groups of {G}), one HIP event pair "
                         f"around each group's back-to-back row passes" if ev_mode == "grouped" else
                         f"the next {K} batches call by call, events around every {EV_SAMPLE_ML}rd row pass"),
            "design_frac": design_gbs / HBM_PEAK_GBS,
        },
        "step_hbm": {
            "algorithmic_bytes_per_step": float(step_bytes.mean()),
            "achieved_gbs": float(step_bytes.sum() / total_s / 1e9),
            "frac": float(step_bytes.sum() / total_s / 1e9 / HBM_PEAK_GBS),
        },
        "event_timed_leg": timed_leg,
        "one_stream": {"ms_per_step": serial_s / K * 1e3, "rows_per_s": n * K / serial_s,
                       "ops_us": ({"lookup_or_insert": float(per_op[:, 0].mean() * 1e6),
                                   "gather": float(per_op[:, 1].mean() * 1e6),
                                   "writeback": float(per_op[:, 2].mean() * 1e6)} if args.op_events else None)},
        "distinct_rows_per_step": float(us.mean()),
        "stored_rows_read_per_step": float(u_read.mean()),
        "dup_frac": float(dup),
        "hit_rate_after": None,
        "wall_s": wall,
        "host_enqueue_us_per_step": enqueue / K * 1e6,
    }
    st = stats.cpu().numpy()
    line["hit_rate_after"] = float(st[0] / n)
    line["stats_after"] = {"hits": int(st[0]), "inserts": int(st[1]), "evictions": int(st[2]),
                               "overflows": int(st[3]), "invalid": int(st[4]), "consistency_failures": int(st[5])}

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, prefill, stream, e_pool, npool, base_now, args.cpu_seconds, W)
    print(json.dumps(line), flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, prefill, stream, e_pool, npool, base_now, budget_s, W):
    """Times the CPU oracle (single-threaded C) on the same steps: a bounded sample, the process pinned to one
    core of its CPU set for the duration (os.sched_setaffinity, no re-exec), mean and median per step."""
    import numpy as np
    import oracle

    C, P, D, n = cfg.capacity, cfg.probes, cfg.dim, cfg.batch
    t0 = time.time()
    tab = oracle.MPZCHTable(C, P, D, with_values=False)
    for k, batch in enumerate(prefill, start=1):
        tab.step(batch, k, zero_fill=False)
    tab.values = np.empty((C, D), np.float32)
    tab.values.fill(0.0)  # touch every page before timing (inputs resident)
    setup = time.time() - t0
    e_host = {}
    for t in range(W, len(stream)):  # host copies of e before timing
        if t % npool not in e_host:
            e_host[t % npool] = e_pool[t % npool].cpu().numpy()
    allowed = sorted(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else []
    core = allowed[-1] if allowed else None
    if core is not None:
        os.sched_setaffinity(0, {core})
    per_step = []
    try:
        for t in range(W, len(stream)):
            e = e_host[t % npool]
            a = time.perf_counter()
            rows, hit, ev, st = tab.step(stream[t], base_now + 1 + t)
            tab.gather(rows)
            tab.writeback(rows, e)
            per_step.append(time.perf_counter() - a)
            if sum(per_step) >= budget_s:
                break
    finally:
        if core is not None:
            os.sched_setaffinity(0, set(allowed))
    spent, steps = float(sum(per_step)), len(per_step)
    return {"value": steps * n / spent, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} steps (steps {W + 1}..{W + steps} of the same stream, {n} IDs each) after an "
                      f"untimed oracle prefill ({setup:.1f}s); single-threaded C oracle, lookup+gather+writeback",
            "seconds": spent, "step_ms_mean": spent / steps * 1e3,
            "step_ms_median": float(np.median(per_step)) * 1e3,
            "rows_per_s_median_step": n / float(np.median(per_step)),
            "pinned_core": core, "cpu_model": cpu_model(), "host_nproc": os.cpu_count(),
            "cpus_allowed": len(allowed) or None}


# ----------------------------------------------------------------------------------------------
# Other rows of the path, measured on their own workloads (one JSON line each; not the headline).
def _line(metric, value, unit, K, W, ms, config, roof, extra):
    d = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": ms,
         "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "data": "synthetic", "config": config,
         "roofline": roof}
    d.update(extra)
    print(json.dumps(d), flush=True)


def _roof(name, nbytes, seconds, bound="hbm"):
    gbs = nbytes / seconds / 1e9
    return {"bound": bound, "kernel": name, "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes_per_launch": nbytes,
            "avg_launch_us": seconds * 1e6}


def _timed(timer, cur, fn, K):
    """Runs fn(k) for k < K with an event pair around each call; returns per-call seconds."""
    import numpy as np
    evs = [(timer.event(), timer.event()) for _ in range(K)]
    for k in range(K):
        timer.record(evs[k][0], cur)
        fn(k)
        timer.record(evs[k][1], cur)
    import torch
    torch.cuda.synchronize()
    return np.array([timer.elapsed_s(a, b) for a, b in evs])


def run_serving(args):
    """Serving read path: lookup-only MPZCH + int8 dequant + dot, 256 requests x 1024 candidates."""
    import numpy as np
    import torch
    import hashed_lookup_row_amd as hlr
    import synth
    dev = torch.device("cuda:0")
    cfg, sv = synth.MEMORY_LAYER, synth.SERVING
    C, P, D = sv.capacity, cfg.probes, sv.dim
    identity = torch.full((C,), -1, dtype=torch.int64, device=dev)
    stamps = torch.full((C,), -1, dtype=torch.int64, device=dev)
    for k, b in enumerate(synth.prefill_batches(cfg), start=1):
        hlr.mpzch_lookup_or_insert(identity, stamps, None, P, torch.from_numpy(b).to(dev), k)
    keys = synth.universe_keys(cfg.universe, cfg.config)
    ident = identity.cpu().numpy()
    cands = synth.serving_candidates(keys[np.isin(keys, ident[ident >= 0])], sv.requests, sv.cands, sv.zipf_s,
                                     sv.miss_frac)
    q, scale, bias = synth.int8_table(C, D, device=dev)
    user = synth.normal_rows(sv.requests, D, 1.0, 3, 0, device=dev)
    ids = torch.from_numpy(cands).to(dev)
    rows = torch.empty(ids.numel(), dtype=torch.int64, device=dev)
    hit = torch.empty(ids.numel(), dtype=torch.int8, device=dev)
    scores = torch.empty((sv.requests, sv.cands), dtype=torch.float32, device=dev)
    timer, cur = HipTimer(), torch.cuda.current_stream(dev).cuda_stream
    K, W = args.steps, args.warmup
    for _ in range(W):
        hlr.mpzch_lookup_or_insert(identity, None, None, P, ids, 0, insert=False, out_rows=rows, out_hit=hit)
        hlr.gather_dequant_score(q, scale, bias, rows, user, sv.cands, out=scores)
    for _ in range(W):
        hlr.mpzch_score(identity, P, ids, q, scale, bias, user, sv.cands, out=scores)
    # the step: lookup-only MPZCH and the score in one launch (mpzch_score); the two-call form is timed beside it
    t_fused = _timed(timer, cur, lambda k: hlr.mpzch_score(identity, P, ids, q, scale, bias, user, sv.cands,
                                                           out=scores), K)
    t_look = _timed(timer, cur, lambda k: hlr.mpzch_lookup_or_insert(identity, None, None, P, ids, 0, insert=False,
                                                                     out_rows=rows, out_hit=hit), K)
    t_score = _timed(timer, cur, lambda k: hlr.gather_dequant_score(q, scale, bias, rows, user, sv.cands,
                                                                    out=scores), K)
    r = rows.cpu().numpy()
    u = np.unique(r[r >= 0]).size
    u_ids = np.unique(cands).size
    n = r.size
    score_bytes = u * (D + 8) + 8 * n + 4 * n + sv.requests * D * 4
    look_bytes = 8 * n + u * 64 + 9 * n
    # one launch: the IDs, one 64-byte bucket per distinct ID, each distinct row once, the scores, the user vectors
    fused_bytes = 8 * n + u_ids * 64 + u * (D + 8) + 4 * n + sv.requests * D * 4
    step_s = float(np.median(t_fused))
    _line("candidate scores/s (lookup-only MPZCH + int8 dequant + dot)", n / step_s, "scores/s", K, W,
          step_s * 1e3, {"workload": sv.name, "requests": sv.requests, "cands": sv.cands, "dim": D, "capacity": C,
                         "step": "mpzch_score: lookup-only MPZCH and the int8 dequant-score in one launch"},
          _roof("score_kernel<2,2,2,ProbeIn8> (mpzch_score)", fused_bytes, step_s),
          {"dtype": "int8->fp64", "distinct_rows": int(u), "hit_rate": float((r >= 0).mean()),
           "ops_us": {"fused": step_s * 1e6, "lookup_only": float(np.median(t_look) * 1e6),
                      "score": float(np.median(t_score) * 1e6)},
           "two_calls": {"ms_per_step": float(np.median(t_look) + np.median(t_score)) * 1e3,
                         "score_roofline": _roof("score_kernel<2,2,2,RowsIn>", score_bytes, float(np.median(t_score))),
                         "lookup_roofline": _roof("mz_probe<8>", look_bytes, float(np.median(t_look)))},
           "score_valu_ops_per_s": float(3 * n * D / step_s)})


# Kernel times inside a timed region are taken with HIP events on every EV_SAMPLE-th step only: each event
# is a packet on the compute stream between kernels, and events around every kernel of every step add to
# the step they measure.
EV_SAMPLE = 4
EV_SAMPLE_ML = 3  # Memory Layer: coprime with the default group of 4, so the sampled row passes sit anywhere in a group


class _EventPool:
    """Timing events created before the timed region: creating HIP events inside it has stalled the GPU
    for tens of milliseconds now and then (the runtime growing its signal pool)."""

    def __init__(self, timer, count):
        self.free = [timer.event() for _ in range(count)]

    def take(self):
        if not self.free:
            raise RuntimeError("event pool exhausted: size it for the timed steps")
        return self.free.pop()


def _marker(timer, cur, store, pool):
    """A pipeline mark hook recording HIP events (from `pool`) on the compute stream into store[(op, i)]."""
    def mark(tag):
        op, i, edge = tag
        if edge == 0:
            store.setdefault((op, i), []).append([pool.take(), pool.take()])
        timer.record(store[(op, i)][-1][edge], cur)
    return mark


def _mean_s(timer, store, key):
    import numpy as np
    return float(np.mean([timer.elapsed_s(a, b) for a, b in store[key]]))


def run_dlrm(args):
    """DLRMv4-like: 8 hashed tables (120 GiB), per table hashed rows + gather + duplicate-summed SGD."""
    import numpy as np
    import torch
    import hashed_lookup_row_amd as hlr
    import synth
    from hashed_lookup_row_amd.pipeline import HashedTablesPipeline
    dev = torch.device("cuda:0")
    cfg = synth.DLRM
    D, n = cfg.dim, cfg.per_table
    R = D * 4
    tables = []
    t0 = time.time()
    for t, nr in enumerate(cfg.table_rows):
        x = torch.empty((nr, D), dtype=torch.float32, device=dev)
        synth.dlrm_fill_table(t, nr, D, x)
        tables.append(x)
        torch.cuda.synchronize()
        print(f"[bench] table {t} ({nr} x {D}) filled, {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    K, W = args.steps, args.warmup
    keys = [[torch.from_numpy(synth.dlrm_keys(cfg, t, s + 1)).to(dev) for t in range(8)] for s in range(2)]
    grads = [[synth.normal_rows(n, D, cfg.g_std, 4, 100 * s + t, device=dev) for t in range(8)] for s in range(2)]
    rows = [torch.empty(n, dtype=torch.int64, device=dev) for _ in range(8)]
    outs = [torch.empty((n, D), dtype=torch.float32, device=dev) for _ in range(8)]
    timer, cur = HipTimer(), torch.cuda.current_stream(dev).cuda_stream
    pipe = HashedTablesPipeline(tables, n, batch=args.dlrm_batch, group=args.dlrm_group)

    def serial_step(s):
        for t in range(8):
            hlr.hashed_rows(keys[s % 2][t], cfg.table_rows[t], out=rows[t])
            hlr.gather_rows(tables[t], rows[t], out=outs[t])
            hlr.writeback_rows(tables[t], rows[t], grads[s % 2][t], mode=hlr.WB_SGD_SUM, lr=cfg.lr)

    ev = {}
    for s in range(W):
        pipe.step(keys[s % 2], grads[s % 2], cfg.lr, outs)
    torch.cuda.synchronize()
    a, b = timer.event(), timer.event()
    pool = _EventPool(timer, K * 8 * 2 * 2)  # per step: 8 tables x (gather, apply) x 2 edges
    timer.record(a, cur)
    for s in range(K):
        pipe.step(keys[s % 2], grads[s % 2], cfg.lr, outs,
                  mark=_marker(timer, cur, ev, pool) if s % EV_SAMPLE == 0 else None)
    timer.record(b, cur)
    torch.cuda.synchronize()
    total = timer.elapsed_s(a, b)
    print(f"[bench] {K} pipelined steps: {total / K * 1e3:.3f} ms per step; one-stream leg next", file=sys.stderr,
          flush=True)
    c, d = timer.event(), timer.event()
    timer.record(c, cur)
    for s in range(K):
        serial_step(s)
    timer.record(d, cur)
    torch.cuda.synchronize()
    serial = timer.elapsed_s(c, d)
    # distinct rows per table, averaged over the two key sets the steps alternate between
    us = [float(np.mean([np.unique(hlr.hashed_rows(keys[s][t], cfg.table_rows[t]).cpu().numpy()).size
                         for s in range(2)])) for t in range(8)]
    g_bytes = sum(n * R + u * R + 8 * n for u in us)          # gather: write n rows, read u rows, indices
    s_bytes = sum(n * R + 2 * u * R + 8 * n for u in us)      # SGD: read n gradients, read+write u rows
    g_time = sum(_mean_s(timer, ev, ("gather", t)) for t in range(8))
    if pipe.batch:  # one writeback_apply_batch call per step: its time covers all 8 tables
        s_time = sum(_mean_s(timer, ev, ("apply", -1 - gi)) for gi in range(len(pipe.groups)))
    else:
        s_time = sum(_mean_s(timer, ev, ("apply", t)) for t in range(8))
    step_s = total / K
    _line("per-token rows/s (8 hashed tables: gather + duplicate-summed SGD)", 8 * n / step_s, "rows/s", K, W,
          step_s * 1e3, {"workload": cfg.name, "tables": 8, "rows_per_table": list(cfg.table_rows), "dim": D,
                         "keys_per_table": n, "zipf_s": cfg.zipf_s, "lr": cfg.lr,
                         "schedule": (f"two streams, tables in groups of {len(pipe.groups[0])}: per group the hashed "
                                      "rows, then the SGD plans (sort) on a lookup stream; on the compute stream the "
                                      "group's gathers, then one batched SGD apply for the group" if pipe.batch else
                                      "two streams: hashed rows + SGD plan (sort) on a lookup stream beside gather + "
                                      "SGD apply on the compute stream, table by table")},
          (_roof(f"writeback_apply_batch SGD_SUM, {len(pipe.groups[0])} tables per launch (sgd_apply_kernel)",
                 s_bytes / len(pipe.groups), s_time / len(pipe.groups))
           if pipe.batch else
           _roof("writeback_apply SGD_SUM (sgd_apply_kernel)", s_bytes / 8, s_time / 8)),
          {"dtype": "fp32", "distinct_rows_per_table": us,
           "gather_roofline": _roof("gather_kernel<128>", g_bytes / 8, g_time / 8),
           "step_hbm_gbs": (g_bytes + s_bytes) / step_s / 1e9,
           "ops_us_per_table": {"gather": float(g_time / 8 * 1e6), "sgd_apply": float(s_time / 8 * 1e6)},
           "one_stream": {"ms_per_step": serial / K * 1e3, "rows_per_s": 8 * n * K / serial}})


def run_cs3(args):
    """CS3 EMA caches: CTS on positives (c_user, c_item) and CMS on all pairs (s_user, s_item)."""
    import numpy as np
    import torch
    import hashed_lookup_row_amd as hlr
    import synth
    from hashed_lookup_row_amd.pipeline import EMAPipeline, RunGraph
    dev = torch.device("cuda:0")
    cfg = synth.CS3
    D, n = cfg.dim, cfg.batch
    R = D * 4
    names = ["c_user", "c_item", "s_user", "s_item"]
    sizes = {"c_user": cfg.users, "s_user": cfg.users, "c_item": cfg.items, "s_item": cfg.items}
    tabs = {k: torch.zeros((sizes[k], D), dtype=torch.float32, device=dev) for k in names}
    K, W = args.steps, args.warmup
    inp = []
    for s in range(2):
        ur, ir, y = synth.cs3_step(cfg, s + 1)
        inp.append([torch.from_numpy(x).to(dev) for x in (ur, ir, y)] +
                   [synth.normal_rows(n, D, 1.0, 5, s + 1, stream=k, device=dev) for k in (1, 2, 3)])
    # a non-default compute stream (a HIP graph cannot be captured on the legacy default stream)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    torch.cuda.set_stream(side)
    timer, cur = HipTimer(), torch.cuda.current_stream(dev).cuda_stream
    # (table, rows index, values index, masked, a, b) per update, in the order applied
    calls = [("c_user", 0, 3, True, cfg.cts_a, cfg.cts_b), ("c_item", 1, 4, True, cfg.cts_a, cfg.cts_b),
             ("s_user", 0, 5, False, cfg.cms_a, cfg.cms_b), ("s_item", 1, 5, False, cfg.cms_a, cfg.cms_b)]
    grouped = args.schedule != "eager" and args.ema_batch
    derive = {"yes": True, "no": False}.get(args.ema_derive, not args.ema_pairs)
    G, A = args.group, args.ahead
    pipe = EMAPipeline([tabs[c[0]] for c in calls], n, depth=(A + 2) * G if grouped else 2,
                       lookup_streams=args.ema_lookup_streams, batch=args.ema_batch, pairs=args.ema_pairs,
                       derive=derive)

    def step_args(s):
        x = inp[s % 2]
        return ([x[c[1]] for c in calls], [x[2] if c[3] else None for c in calls], [x[c[2]] for c in calls],
                [(c[4], c[5]) for c in calls])

    def piped_step(s, mark=None):
        pipe.step(*step_args(s), mark=mark)

    def serial_step(s):
        x = inp[s % 2]
        for name, ri, vi, masked, a, b in calls:
            hlr.ema_update_rows(tabs[name], x[ri], x[vi], x[2] if masked else None, a, b)

    ev = {}
    a, b = timer.event(), timer.event()
    if grouped:
        # the plans of a group run a group ahead of its applies; one event pair per group on the compute
        # stream around its back-to-back applies (apply time = span / batches in the group), the ends
        # giving per-group step times
        if W:
            pipe.run([step_args(s) for s in range(W)], group=G, ahead=A)
        torch.cuda.synchronize()
        ngroups = (K + G - 1) // G
        gev = [(timer.event(), timer.event()) for _ in range(ngroups)]
        todo = [step_args(W + s) for s in range(K)]
        timer.record(a, cur)
        h0 = time.perf_counter()
        pipe.run(todo, group=G, ahead=A, apply_events=gev)
        timer.record(b, cur)
        enqueue_s = time.perf_counter() - h0
        torch.cuda.synchronize()
        total = timer.elapsed_s(a, b)
        sizes = [min(G, K - g * G) for g in range(ngroups)]
        apply_s = [timer.elapsed_s(x, y) / sizes[g] for g, (x, y) in enumerate(gev)]
        step_ms = [timer.elapsed_s(gev[g - 1][1], gev[g][1]) / sizes[g] * 1e3 for g in range(1, ngroups)] or \
            [total / K * 1e3]
        if args.schedule == "graph":
            # the same schedule captured (untimed) as one HIP graph and replayed: the step time; the apply
            # times above come from the eagerly enqueued run (events inside a graph cannot be timed)
            event_leg_ms = total / K * 1e3
            graph = RunGraph(pipe, todo, group=G, ahead=A)
            torch.cuda.synchronize()
            ga, gb = timer.event(), timer.event()
            timer.record(ga, cur)
            h0 = time.perf_counter()
            graph.replay()
            timer.record(gb, cur)
            enqueue_s = time.perf_counter() - h0
            torch.cuda.synchronize()
            total = timer.elapsed_s(ga, gb)
    else:
        for s in range(W):
            piped_step(s)
        torch.cuda.synchronize()
        pool = _EventPool(timer, K * 4 * 2)  # per step: 4 applies x 2 edges
        # an event on the compute stream after every step: per-step times (median reported), and without them
        # this schedule has stalled for about 40 ms at the start of the timed region on some runs (a runtime
        # effect, seen as an idle GPU in kernel traces, never with these events)
        sev = [timer.event() for _ in range(K)]
        timer.record(a, cur)
        h0 = time.perf_counter()
        for s in range(K):
            piped_step(W + s, _marker(timer, cur, ev, pool) if s % EV_SAMPLE == 0 else None)
            timer.record(sev[s], cur)
        timer.record(b, cur)
        enqueue_s = time.perf_counter() - h0
        torch.cuda.synchronize()
        total = timer.elapsed_s(a, b)
        step_ms = [timer.elapsed_s(a if s == 0 else sev[s - 1], sev[s]) * 1e3 for s in range(K)]
    c, d = timer.event(), timer.event()
    timer.record(c, cur)
    for s in range(K):
        serial_step(W + K + s)
    timer.record(d, cur)
    torch.cuda.synchronize()
    serial = timer.elapsed_s(c, d)
    if grouped:
        per = {"batch": float(np.mean(apply_s))}
    else:
        per = ({"batch": _mean_s(timer, ev, ("apply", -1))} if pipe.batch else
               {calls[i][0]: _mean_s(timer, ev, ("apply", i)) for i in range(4)})
    x = inp[0]
    ur, ir, y = (t.cpu().numpy() for t in x[:3])
    m = int(y.sum())
    nb = {"c_user": m * R + 2 * np.unique(ur[y > 0]).size * R, "c_item": m * R + 2 * np.unique(ir[y > 0]).size * R,
          "s_user": n * R + 2 * np.unique(ur).size * R, "s_item": n * R + 2 * np.unique(ir).size * R}
    tot_bytes = sum(nb.values()) + 4 * 9 * n
    step_s = total / K
    if pipe.batch:
        roof = _roof(("ema_update_apply_pairs" if args.ema_pairs else "ema_update_apply_batch") +
                     " (the four updates: ema_apply_kernel + ema_combine_kernel)", sum(nb.values()), per["batch"])
        applies = "the four applies as one ema_update_apply_batch call"
    else:
        worst = max(per, key=lambda k: per[k])
        roof = _roof(f"ema_update_apply ({worst}: ema_apply_kernel + ema_combine_kernel)", nb[worst], per[worst])
        applies = "the four applies"
    _line("interaction pairs/s (CTS + CMS EMA row updates)", n / step_s, "pairs/s", K, W, step_s * 1e3,
          {"workload": cfg.name, "users": cfg.users, "items": cfg.items, "dim": D, "pairs": n,
           "schedule": (f"each rule's user- and item-keyed updates planned by one sort (CMS and CTS pair plans"
                        + (", CTS cut out of CMS by the label mask" if derive else ", each sorted on its own") +
                        f") on {args.ema_lookup_streams} lookup stream(s), beside the four applies as one "
                        "ema_update_apply_pairs call on the compute stream" if args.ema_pairs else
                        f"the EMA plans on {args.ema_lookup_streams} lookup stream(s) (user-keyed and item-keyed "
                        "plans side by side; CMS plans sorted, CTS plans "
                        + ("cut out of them by the label mask" if derive else "sorted on their own") +
                        f") beside {applies} on the compute stream") +
                       (f"; grouped: plans of {G} steps back to back, {A} group(s) ahead of the applies, one "
                        "cross-stream wait per stream per group (EMAPipeline.run)" if grouped else
                        "; step by step, plans one step ahead") +
                       ("; the K timed steps captured (untimed) as one HIP graph and replayed once (RunGraph); "
                        "apply times from the same schedule enqueued call by call" if grouped and
                        args.schedule == "graph" else "")},
          roof,
          {"dtype": "fp32", "step_hbm_gbs": tot_bytes / step_s / 1e9,
           "apply_us": {k: v * 1e6 for k, v in per.items()},
           "step_ms_median": float(np.median(step_ms)), "step_ms_max": float(np.max(step_ms)),
           "host_enqueue_us_per_step": enqueue_s / K * 1e6,
           "eager_grouped_ms_per_step": event_leg_ms if grouped and args.schedule == "graph" else None,
           "one_stream": {"ms_per_step": serial / K * 1e3, "pairs_per_s": n * K / serial},
           "top_user_occurrences": int(np.bincount(ur).max())})


def run_res(args):
    """Memory-Layer step with the Raw Embedding Streaming bookkeeping (each batch's written rows added to
    the publish set), then one publish of everything written in the timed batches: quantise to int8,
    snapshot identity/stamps at the batch boundary, copy both to pinned host memory."""
    import numpy as np
    import torch
    import hashed_lookup_row_amd as hlr
    import synth
    from hashed_lookup_row_amd.pipeline import MemoryLayerPipeline, RESPublisher
    from hashed_lookup_row_amd._hip import hip
    dev = torch.device("cuda:0")
    cfg = synth.MEMORY_LAYER
    C, P, D, n = cfg.capacity, cfg.probes, cfg.dim, cfg.batch
    # at most 50 timed batches between the two publishes: about 0.55M distinct rows are written in them
    K, W = min(args.steps, 50), args.warmup
    stream, fc = [], 0
    for t in range(1, W + K + 1):
        ids, fc = synth.mpzch_step_ids(cfg, t, fc)
        stream.append(ids)
    identity = torch.full((C,), -1, dtype=torch.int64, device=dev)
    stamps = torch.full((C,), -1, dtype=torch.int64, device=dev)
    values = torch.zeros((C, D), dtype=torch.float32, device=dev)
    prefill = synth.prefill_batches(cfg)
    for k, b in enumerate(prefill, start=1):
        hlr.mpzch_lookup_or_insert(identity, stamps, None, P, torch.from_numpy(b).to(dev), k)
    base = len(prefill)
    ids_dev = [torch.from_numpy(x).to(dev) for x in stream]
    e_pool = [synth.normal_rows(n, D, cfg.e_std, cfg.config, t + 1, device=dev) for t in range(8)]
    out = torch.empty((n, D), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    timer, cur = HipTimer(), torch.cuda.current_stream(dev).cuda_stream
    pipe = MemoryLayerPipeline(identity, stamps, values, P, n)
    pub = RESPublisher(pipe, 0, max_rows=1 << 20)
    for t in range(W):
        pipe.step(ids_dev[t], base + 1 + t, e_pool[t % 8], out=out, publisher=pub)
    pub.publish_now(pipe)  # clears the warm-up's rows (and warms the host copy path)
    pub.flush()
    torch.cuda.synchronize()
    pub.copy.synchronize()
    a, b = timer.event(), timer.event()
    timer.record(a, cur)
    for k in range(K):
        t = W + k
        pipe.step(ids_dev[t], base + 1 + t, e_pool[t % 8], out=out, publisher=pub)
    timer.record(b, cur)
    torch.cuda.synchronize()
    total = timer.elapsed_s(a, b)
    # one publish of the rows the K timed batches wrote; quantiser timed on the compute stream and the
    # host copies (snapshot + count, then the rows) on the copy stream
    h = hip()
    qa, qb, ca, cb = h.event(True), h.event(True), h.event(True), h.event(True)
    h.record(qa, cur)
    pub.publish_now(pipe)
    h.record(qb, cur)
    h.record(ca, pub.cps)
    pub.flush()
    h.record(cb, pub.cps)
    torch.cuda.synchronize()
    pub.copy.synchronize()
    u = int(pub.h_cnt[(pub.p - 1) % 2][0])
    pub_s = h.elapsed_s(qa, qb)
    copy_s = h.elapsed_s(qa, cb)
    qbytes = u * (D * 4 + D + 8 + 8) + u * 8 * 2
    host_bytes = u * (D + 16) + 16 * C + 8
    step_s = total / K
    _line("rows/s of the Memory-Layer step with RES bookkeeping (written-row set per batch)", n / step_s, "rows/s",
          K, W, step_s * 1e3, {"workload": cfg.name + "+res", "capacity": C, "dim": D, "ids_per_step": n},
          _roof("publish on the compute stream (quantize_rows_int8 + staging copies)", qbytes, pub_s),
          {"dtype": "fp32->int8", "published_rows": u, "publish_gpu_us": pub_s * 1e6,
           "host_copy": {"bytes": host_bytes, "ms_from_publish_start": copy_s * 1e3,
                         "GBps": host_bytes / copy_s / 1e9}})


def run_keystore(args):
    """The Memory-Layer ID stream (65,536 IDs per batch, Zipf(1.05) over 20M keys + 0.5% fresh) through
    the decoupled key store: key store from 2^20 slots, grown by rehash (keys only) whenever it could
    pass half full; value store of up to 4Mi rows x 512 fp32 in chunks of 65,536 rows, 2Mi rows at the
    start and grown a chunk at a time as rows fill (new rows zero-filled, stamped and counted)."""
    import numpy as np
    import torch
    import hashed_lookup_row_amd as hlr
    import synth
    from hashed_lookup_row_amd.keystore import DynamicKeyStore
    dev = torch.device("cuda:0")
    cfg = synth.MEMORY_LAYER
    C, D, n = cfg.capacity, cfg.dim, cfg.batch
    K, W = args.steps, args.warmup
    stream, fc = [], 0
    for t in range(1, W + K + 1):
        ids, fc = synth.mpzch_step_ids(cfg, t, fc)
        stream.append(ids)
    ids_dev = [torch.from_numpy(x).to(dev) for x in stream]
    store = DynamicKeyStore(D, C, dev, key_cap=1 << 20, chunk_shift=16, initial_rows=C // 2)
    rows = torch.empty(n, dtype=torch.int64, device=dev)
    hit = torch.empty(n, dtype=torch.int8, device=dev)
    stats = torch.zeros(4, dtype=torch.int64, device=dev)
    for t in range(W):
        store.step(ids_dev[t], t + 1, out_rows=rows, out_hit=hit)
    torch.cuda.synchronize()
    timer, cur = HipTimer(), torch.cuda.current_stream(dev).cuda_stream
    r0 = store.rehashes
    a, b = timer.event(), timer.event()
    timer.record(a, cur)
    for k in range(K):
        t = W + k
        store.step(ids_dev[t], t + 1, out_rows=rows, out_hit=hit, out_stats=stats if k == K - 1 else None)
    timer.record(b, cur)
    torch.cuda.synchronize()
    total = timer.elapsed_s(a, b)
    st = stats.cpu().numpy()
    used = int(store.next_row.cpu()[0])
    # one rehash of the final key store into one twice as large (keys and row indices only), timed alone
    ra, rb = timer.event(), timer.event()
    timer.record(ra, cur)
    hlr.dks_rehash(store.keys, store.krows, 2 * store.keys.numel())
    timer.record(rb, cur)
    torch.cuda.synchronize()
    rehash_s = timer.elapsed_s(ra, rb)
    cap = store.keys.numel()
    step_s = total / K
    probe_bytes = n * (8 + 64 + 8 + 8 + 1 + 8)  # id, key line, row index, out row, hit, stamp per position
    _line("IDs/s through the decoupled key store (lookup-or-insert, growth by rehash)", n / step_s, "ids/s", K, W,
          step_s * 1e3, {"workload": "memory-layer ID stream, decoupled key store", "value_rows": C, "dim": D,
                         "ids_per_step": n, "key_slots_final": cap},
          _roof("dks_lookup_or_insert (all kernels)", probe_bytes, step_s),
          {"dtype": "int64", "rows_in_use": used, "rehashes_timed": store.rehashes - r0,
           "last_step_stats": {"hits": int(st[0]), "inserts": int(st[1]), "overflows": int(st[2]),
                               "invalid": int(st[3])},
           "rehash": {"from_slots": cap, "to_slots": 2 * cap, "us": rehash_s * 1e6,
                      "bytes_moved": cap * 16 + 2 * cap * 16},
           "value_store": {"chunks": len(store.values.chunks), "rows_held": store.values.capacity,
                           "chunk_rows": store.values.rows_per_chunk}})


def run_dedup(args):
    """Standalone dedup_ids on the Memory-Layer ID stream (65,536 int64 IDs per call)."""
    import numpy as np
    import torch
    import hashed_lookup_row_amd as hlr
    import synth
    dev = torch.device("cuda:0")
    cfg = synth.MEMORY_LAYER
    K, W = args.steps, args.warmup
    ids = [torch.from_numpy(synth.mpzch_step_ids(cfg, t + 1, 0)[0]).to(dev) for t in range(8)]
    n = cfg.batch
    uq = torch.empty(n, dtype=torch.int64, device=dev)
    lp = torch.empty(n, dtype=torch.int64, device=dev)
    inv = torch.empty(n, dtype=torch.int64, device=dev)
    nu = torch.empty(1, dtype=torch.int64, device=dev)
    timer, cur = HipTimer(), torch.cuda.current_stream(dev).cuda_stream
    for k in range(W):
        hlr.dedup_ids(ids[k % 8], uq, lp, inv, nu)
    t = _timed(timer, cur, lambda k: hlr.dedup_ids(ids[k % 8], uq, lp, inv, nu), K)
    u = int(nu.item())
    nbytes = 8 * n + 16 * u + 8 * n  # keys in; unique + last position out; inverse out
    _line("IDs deduplicated/s (dedup_ids, last occurrence wins)", n / float(np.median(t)), "ids/s", K, W,
          float(np.median(t)) * 1e3, {"workload": "memory-layer ID stream", "ids": n},
          _roof("dedup_ids (radix sort + segments, all kernels)", nbytes, float(np.median(t))),
          {"dtype": "int64", "distinct": u})


def run_hbm_ceiling(args):
    """Measured HBM ceiling: hand-written read-only, write-only and copy sweeps (ordinary and non-temporal
    accesses) over buffers of 1-8 GiB, each launch timed with HIP events on the stream it runs on."""
    import ctypes
    import statistics
    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "hashed_lookup_row_amd", "libhlr_bwprobe.so"))
    lib.hlr_bwprobe.restype = ctypes.c_int
    lib.hlr_bwprobe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                ctypes.c_void_p, ctypes.c_void_p]
    lib.hlr_bwprobe_sink_words.restype = ctypes.c_int64
    lib.hlr_bwprobe_sink_words.argtypes = [ctypes.c_int64]
    dev = torch.device("cuda:0")
    timer, cur = HipTimer(), torch.cuda.current_stream(dev).cuda_stream
    sizes = [int(float(x) * (1 << 30)) for x in args.ceiling_gib.split(",")]
    kinds = args.ceiling_kinds.split(",")
    big = max(sizes)
    src = torch.empty(big // 4, dtype=torch.float32, device=dev).uniform_()
    dst = torch.empty(big // 4, dtype=torch.float32, device=dev)
    sink = torch.empty(lib.hlr_bwprobe_sink_words(big), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    code = {"read": 0, "write": 1, "copy": 2}
    reps = max(3, args.steps if args.steps < 50 else 10)
    out = []
    for nbytes in sizes:
        for kind in kinds:
            base, nt = kind.split("-")[0], kind.endswith("-nt")
            evs = [(timer.event(), timer.event()) for _ in range(reps)]
            for w in range(2):  # untimed warm-up launches
                rc = lib.hlr_bwprobe(code[base], int(nt), src.data_ptr(), dst.data_ptr(), nbytes, sink.data_ptr(), cur)
                if rc:
                    raise RuntimeError(f"hlr_bwprobe failed ({rc})")
            for a, b in evs:
                timer.record(a, cur)
                lib.hlr_bwprobe(code[base], int(nt), src.data_ptr(), dst.data_ptr(), nbytes, sink.data_ptr(), cur)
                timer.record(b, cur)
            torch.cuda.synchronize()
            ts = [timer.elapsed_s(a, b) for a, b in evs]
            moved = 2 * nbytes if base == "copy" else nbytes
            rec = {"kind": kind, "gib": nbytes / (1 << 30), "bytes_moved": moved,
                   "us_median": statistics.median(ts) * 1e6, "us_min": min(ts) * 1e6,
                   "gbs_median": moved / statistics.median(ts) / 1e9, "gbs_best": moved / min(ts) / 1e9}
            out.append(rec)
            print(json.dumps(rec), flush=True)
    best = {k: max(r["gbs_median"] for r in out if r["kind"] == k) for k in kinds}
    print(json.dumps({"metric": "HBM ceiling of hand-written streaming kernels (median over launches)",
                      "unit": "GB/s", "per_kind_best_median": best, "peak": HBM_PEAK_GBS,
                      "reps": reps}), flush=True)


if __name__ == "__main__":
    main()
