"""Seeded synthetic inputs for the embedding-cache workloads.

This module only draws inputs: item-ID streams, item-tower vectors, gradients,
EMA update vectors, int8 serving tables and user vectors.  It holds none of the
cache's own arithmetic (no hashing, probing, deduplication or row update); the
oracle and the HIP path both consume what it returns, and neither is imported
here.

Distributions follow the workloads the pages describe:
  * skewed item popularity (a few IDs take most lookups: MP-Rec explainer,
    "Why it works"; DLRMv4 review, skew paragraph) is drawn as Zipf(s) over a
    finite universe of ranks 1..N, P(k) proportional to k**-s, sampled by
    inverse CDF on the exact finite pmf;
  * the Memory Layer batch merges a labelled training batch with an unlabelled
    candidate-pool batch (Memory Layer page, section 2, Multi-Table Training);
  * never-seen fresh IDs stand for newly posted content (Memory Layer page,
    section 1) and are negative keys -2, -3, ... that no universe key equals.
The public datasets the pages measure on are not available; these streams take
only their sizes and skew.
"""
from __future__ import annotations

import dataclasses
import functools
from typing import Optional

import numpy as np

try:  # torch is only needed for device-resident tensors
    import torch
except Exception:  # pragma: no cover - torch is present in every supported image
    torch = None

EMPTY = -1
MI = 1 << 20


# --------------------------------------------------------------------------- rng
def rng(config: int, step: int, stream: int = 0) -> np.random.Generator:
    """numpy PCG64 generator for (config, step, stream); fully reproducible."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 + config, step % (1 << 64), stream])))


def torch_gen(device, config: int, step: int, stream: int = 0):
    """torch generator on `device`, seeded from (config, step, stream)."""
    seed = int(np.random.SeedSequence([2000 + config, step % (1 << 64), stream]).generate_state(1, dtype=np.uint64)[0] >> 1)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


# ------------------------------------------------------------------------- zipf
@functools.lru_cache(maxsize=8)
def _zipf_cdf(n: int, s: float) -> np.ndarray:
    k = np.arange(1, n + 1, dtype=np.float64)
    w = k ** (-s)
    c = np.cumsum(w)
    c /= c[-1]
    return c


def zipf_ranks(g: np.random.Generator, n_universe: int, s: float, size: int) -> np.ndarray:
    """0-based ranks (0 = most popular) drawn from Zipf(s) over n_universe ranks."""
    c = _zipf_cdf(int(n_universe), float(s))
    u = g.random(size)
    r = np.searchsorted(c, u, side="right")
    return np.minimum(r, n_universe - 1).astype(np.int64)


def zipf_pmf(n_universe: int, s: float) -> np.ndarray:
    k = np.arange(1, n_universe + 1, dtype=np.float64)
    w = k ** (-s)
    return w / w.sum()


def expected_distinct(n_universe: int, s: float, draws: int) -> float:
    """E[#distinct] of `draws` i.i.d. Zipf(s) ranks: sum_k 1-(1-p_k)^draws."""
    p = zipf_pmf(n_universe, s)
    return float(np.sum(-np.expm1(draws * np.log1p(-p))))


@functools.lru_cache(maxsize=4)
def universe_keys(n_universe: int, config: int) -> np.ndarray:
    """n_universe distinct non-negative int64 item IDs; index = popularity rank."""
    g = rng(config, -1, 99)
    keys = np.empty(0, dtype=np.int64)
    while keys.size < n_universe:
        draw = g.integers(0, np.iinfo(np.int64).max, size=int(n_universe * 1.05) + 16, dtype=np.int64)
        keys = np.unique(np.concatenate([keys, draw]))
    keys = keys[:n_universe]
    return keys[g.permutation(n_universe)]


def insert_fresh(g: np.random.Generator, ids: np.ndarray, frac: float, counter: int) -> tuple[np.ndarray, int]:
    """Replace round(frac*n) seeded positions by fresh IDs -2-counter, -3-counter, ..."""
    n = ids.size
    m = int(round(frac * n))
    if m == 0:
        return ids, counter
    pos = g.choice(n, size=m, replace=False)
    pos.sort()
    out = ids.copy()
    out[pos] = -2 - (counter + np.arange(m, dtype=np.int64))
    return out, counter + m


# ---------------------------------------------------------------------- configs
@dataclasses.dataclass(frozen=True)
class MPZCHConfig:
    """A Memory-Layer style cache workload (tiny and full-scale variants)."""
    name: str
    config: int
    capacity: int
    probes: int
    dim: int
    universe: int
    zipf_s: float
    batch: int            # positions per step (training + candidate-pool halves)
    steps: int
    e_std: float
    fresh_frac: float = 0.0
    prefill: bool = False  # insert the universe coldest-first before step 1
    split_halves: bool = False

    @property
    def table_bytes(self) -> int:
        return self.capacity * self.dim * 4


TINY = MPZCHConfig("tiny-mpzch-4096x64", 1, 4096, 8, 64, 10_000, 1.1, 1024, 100, 1.0)
MEMORY_LAYER = MPZCHConfig("memory-layer-4Mx512", 2, 4 * MI, 8, 512, 20_000_000, 1.05, 65_536, 200, 0.1,
                           fresh_frac=0.005, prefill=True, split_halves=True)


def scaled_memory_layer(capacity: int = 16_384, universe: int = 80_000, batch: int = 4_096, steps: int = 4,
                        dim: int = 512) -> MPZCHConfig:
    """Memory-Layer workload shrunk for oracle-speed tests (same skew, fresh rate, prefill)."""
    return MPZCHConfig(f"memory-layer-scaled-{capacity}x{dim}", 2, capacity, 8, dim, universe, 1.05, batch, steps,
                       0.1, fresh_frac=0.005, prefill=True, split_halves=True)


def mpzch_step_ids(cfg: MPZCHConfig, step: int, fresh_counter: int = 0) -> tuple[np.ndarray, int]:
    """IDs for one step (step >= 1).  Memory Layer: training half then candidate-pool half."""
    g = rng(cfg.config, step, 0)
    keys = universe_keys(cfg.universe, cfg.config)
    if cfg.split_halves:
        half = cfg.batch // 2
        a = keys[zipf_ranks(g, cfg.universe, cfg.zipf_s, half)]
        b = keys[zipf_ranks(g, cfg.universe, cfg.zipf_s, cfg.batch - half)]
        ids = np.concatenate([a, b])
    else:
        ids = keys[zipf_ranks(g, cfg.universe, cfg.zipf_s, cfg.batch)]
    if cfg.fresh_frac > 0:
        ids, fresh_counter = insert_fresh(g, ids, cfg.fresh_frac, fresh_counter)
    return ids.astype(np.int64), fresh_counter


def mpzch_stream(cfg: MPZCHConfig, steps: int) -> list[np.ndarray]:
    out, c = [], 0
    for t in range(1, steps + 1):
        ids, c = mpzch_step_ids(cfg, t, c)
        out.append(ids)
    return out


def prefill_batches(cfg: MPZCHConfig) -> list[np.ndarray]:
    """Universe keys coldest rank first, cut into batches of cfg.batch (untimed warm start)."""
    keys = universe_keys(cfg.universe, cfg.config)[::-1]
    return [np.ascontiguousarray(keys[i:i + cfg.batch]) for i in range(0, keys.size, cfg.batch)]


def normal_rows(n: int, dim: int, std: float, config: int, step: int, stream: int = 1, device="cpu"):
    """float32 [n, dim] ~ N(0, std) as a torch tensor on `device`."""
    g = torch_gen(device, config, step, stream)
    x = torch.randn((n, dim), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def normal_rows_np(n: int, dim: int, std: float, config: int, step: int, stream: int = 1) -> np.ndarray:
    g = rng(config, step, stream)
    return (g.standard_normal((n, dim), dtype=np.float32) * np.float32(std)).astype(np.float32)


# ------------------------------------------------------------- serving (int8)
@dataclasses.dataclass(frozen=True)
class ServingConfig:
    name: str
    capacity: int
    dim: int
    requests: int
    cands: int
    zipf_s: float
    miss_frac: float


SERVING = ServingConfig("serving-int8-4Mx512-256x1024", 4 * MI, 512, 256, 1024, 1.05, 0.005)


def int8_table(capacity: int, dim: int, config: int = 3, device="cpu"):
    """Row-quantised serving table stand-in: int8 codes, per-row fp32 scale and bias.

    Codes are rounded N(0, 42) clipped to [-128, 127] (the spread a min-max code
    of a Gaussian row has); scale ~ 0.6/255*(1+U(-.1,.1)); bias ~ N(0, 0.005).
    """
    g = torch_gen(device, config, 0, 7)
    q = torch.empty((capacity, dim), dtype=torch.int8, device=device)
    chunk = max(1, (64 * MI) // dim)
    for r0 in range(0, capacity, chunk):
        r1 = min(capacity, r0 + chunk)
        x = torch.randn((r1 - r0, dim), generator=g, device=device, dtype=torch.float32).mul_(42.0)
        q[r0:r1] = x.round_().clamp_(-128, 127).to(torch.int8)
    scale = ((torch.rand((capacity,), generator=g, device=device) - 0.5) * 0.2 + 1.0) * (0.6 / 255.0)
    bias = torch.randn((capacity,), generator=g, device=device) * 0.005
    return q, scale.float().contiguous(), bias.float().contiguous()


def serving_candidates(resident_ids_by_rank: np.ndarray, requests: int, cands: int, s: float, miss_frac: float,
                       config: int = 3) -> np.ndarray:
    """[requests*cands] candidate IDs: Zipf(s) over resident IDs (hottest first) + fresh misses."""
    g = rng(config, 0, 3)
    n = requests * cands
    r = zipf_ranks(g, resident_ids_by_rank.size, s, n)
    ids = resident_ids_by_rank[r].astype(np.int64)
    ids, _ = insert_fresh(g, ids, miss_frac, 0)
    return ids


# --------------------------------------------------------- DLRMv4-like tables
@dataclasses.dataclass(frozen=True)
class DLRMConfig:
    name: str
    table_rows: tuple
    dim: int
    users: int
    seq: int
    zipf_s: float
    g_std: float
    lr: float

    @property
    def per_table(self) -> int:
        return self.users * self.seq


DLRM = DLRMConfig("dlrmv4-8tables-120GiB", tuple(r * MI for r in (24, 4, 5, 6, 6, 5, 5, 5)), 512, 64, 2048, 1.2,
                  1e-3, 0.01)


def dlrm_keys(cfg: DLRMConfig, table: int, step: int) -> np.ndarray:
    """Per-token item keys of one table for one step: Zipf(s) ranks over a universe of rows_t keys."""
    g = rng(4, step, 10 + table)
    n_univ = cfg.table_rows[table]
    # universe keys of table t: rank k -> a fixed seeded 63-bit key (distinctness not required:
    # these tables use the hashing trick, collisions allowed)
    ranks = zipf_ranks(g, n_univ, cfg.zipf_s, cfg.per_table)
    salt = np.int64(0x1234_5678 + 7919 * table)
    # key = odd multiplier * (rank+1) + salt, kept non-negative: a bijection of rank, not a hash
    keys = ((ranks + 1) * np.int64(0x5851_F42D) + salt) & np.int64(0x7FFF_FFFF_FFFF_FFFF)
    return keys.astype(np.int64)


def dlrm_initial_rows(table: int, rows, dim: int, device="cpu"):
    """Closed-form initial table content, exact in fp32 and cheap to regenerate anywhere.

    value(t, r, d) = (((r*2654435761 + d*40503 + t*1000003) mod 2^20) - 2^19) * 2^-27
    """
    if not torch.is_tensor(rows):
        rows = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=device)
    rows = rows.to(device=device, dtype=torch.int64)
    d = torch.arange(dim, device=device, dtype=torch.int64)
    v = (rows[:, None] * 2654435761 + d[None, :] * 40503 + table * 1000003) % (1 << 20)
    return (v - (1 << 19)).to(torch.float32) * (2.0 ** -27)


def dlrm_fill_table(table: int, num_rows: int, dim: int, out):
    """Fill device tensor `out` [num_rows, dim] with dlrm_initial_rows in chunks."""
    chunk = max(1, (32 * MI) // dim)
    for r0 in range(0, num_rows, chunk):
        r1 = min(num_rows, r0 + chunk)
        rows = torch.arange(r0, r1, device=out.device, dtype=torch.int64)
        out[r0:r1] = dlrm_initial_rows(table, rows, dim, device=out.device)


# ------------------------------------------------------------------ CS3 EMA
@dataclasses.dataclass(frozen=True)
class CS3Config:
    name: str
    users: int
    items: int
    dim: int
    batch: int
    user_s: float
    item_s: float
    pos_rate: float
    cts_a: float = 0.99
    cts_b: float = 0.01
    cms_a: float = 0.95
    cms_b: float = 0.05


CS3 = CS3Config("cs3-ema-1Mx128-2Mx128", 1 * MI, 2 * MI, 128, 262_144, 1.1, 1.05, 0.05)


@functools.lru_cache(maxsize=4)
def _perm(n: int, salt: int) -> np.ndarray:
    return rng(5, -1, salt).permutation(n).astype(np.int64)


def cs3_step(cfg: CS3Config, step: int):
    """(user_rows, item_rows, y) for one step; rank -> row through a seeded permutation."""
    g = rng(5, step, 0)
    ur = zipf_ranks(g, cfg.users, cfg.user_s, cfg.batch)
    ir = zipf_ranks(g, cfg.items, cfg.item_s, cfg.batch)
    y = (g.random(cfg.batch) < cfg.pos_rate).astype(np.uint8)
    return _perm(cfg.users, 1)[ur], _perm(cfg.items, 2)[ir], y
