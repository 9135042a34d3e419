"""Mutation tests of the oracle's pins (CPU).

Each case plants one plausible mistake in a copy of oracle/oracle.c (a
dropped term, a wrong sign, constant, comparison or index, a step done in
the wrong order), builds the copy as the oracle is built, and runs the pin
suite (tests/test_oracle_pins.py) against it in a subprocess: at least one
pin must fail.  An unmodified copy built the same way must pass, which shows
that the harness itself is sound.  The mistakes are planted in the oracle,
on the CPU; the GPU path is not involved.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, text in oracle.c, replacement).  Each text must occur exactly once.
MUTANTS = [
    # hash and buckets (SplitMix64 finaliser, bucket = mix mod count)
    ("mix64: first shift 31", "z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;",
     "z = (z ^ (z >> 31)) * 0xbf58476d1ce4e5b9ULL;"),
    ("mix64: second multiplier wrong", "* 0x94d049bb133111ebULL;", "* 0x94d049bb133111edULL;"),
    ("bucket: hash shifted before the modulus",
     "return (int64_t)(orc_mix64((uint64_t)id) % (uint64_t)num_buckets);",
     "return (int64_t)((orc_mix64((uint64_t)id) >> 1) % (uint64_t)num_buckets);"),
    ("hashed rows: modulus rows - 1",
     "rows[i] = (int64_t)(orc_mix64((uint64_t)ids[i]) % (uint64_t)num_rows);",
     "rows[i] = (int64_t)(orc_mix64((uint64_t)ids[i]) % (uint64_t)(num_rows > 1 ? num_rows - 1 : 1));"),
    # MPZCH lookup / insert / LRU
    ("mpzch: phase-1 probes start at the bucket, not bucket * probes",
     "const int64_t base = orc_bucket(ids[i], nb) * probes;", "const int64_t base = orc_bucket(ids[i], nb);"),
    ("mpzch: a hit does not pin its slot", "if (insert) stamps[base + j] = now;", "(void)0;"),
    ("mpzch: a lookup-only call pins too", "if (insert) stamps[base + j] = now;", "stamps[base + j] = now;"),
    ("mpzch: evicts the most recently used slot",
     "(best < 0 || stamps[base + j] < stamps[base + best])", "(best < 0 || stamps[base + j] > stamps[base + best])"),
    ("mpzch: stamp ties go to the highest probe index",
     "(best < 0 || stamps[base + j] < stamps[base + best])", "(best < 0 || stamps[base + j] <= stamps[base + best])"),
    ("mpzch: slots pinned by this batch may be evicted", "if (stamps[base + j] < now && ",
     "if (stamps[base + j] <= now && "),
    ("mpzch: missed IDs inserted in key order, not first-occurrence order",
     "qsort(first, (size_t)f, sizeof(orc_pair), cmp_pos_first);", "(void)cmp_pos_first;"),
    ("mpzch: inserted rows not zero-filled",
     "if (values) memset(values + s * dim, 0, (size_t)dim * sizeof(float));", "(void)0;"),
    ("mpzch: overflows not counted", "if (best < 0) { st[3]++; continue; }", "if (best < 0) { continue; }"),
    ("mpzch: evicted reports the new ID", "evicted[first[k].pos] = old;", "evicted[first[k].pos] = id;"),
    ("mpzch: invalid IDs not counted", "if (ids[i] == ORC_EMPTY) { st[4]++; continue; }\n        const int64_t base",
     "if (ids[i] == ORC_EMPTY) { continue; }\n        const int64_t base"),
    # gather and dedup
    ("gather: a miss reads row 0",
     "out[i * dim + d] = rows[i] < 0 ? 0.0f : table[rows[i] * dim + d];",
     "out[i * dim + d] = table[(rows[i] < 0 ? 0 : rows[i]) * dim + d];"),
    ("dedup: first occurrence kept", "last_pos[u] = p[k].pos; /* positions",
     "if (k == 0 || p[k].key != p[k - 1].key) last_pos[u] = p[k].pos; /* positions"),
    # Writeback
    ("writeback: gradient added", "            w[d] = w[d] - g;\n", "            w[d] = w[d] + g;\n"),
    ("writeback: first occurrence wins", "if (k + 1 < m && p[k + 1].key == p[k].key) continue;",
     "if (k > 0 && p[k - 1].key == p[k].key) continue;"),
    ("writeback: gradient taken as e - M", "const float g = w[d] - src[d];", "const float g = src[d] - w[d];"),
    # SGD with summed duplicates
    ("sgd: first gradient dropped", "float s = g[p[k0].pos * dim + d];", "float s = 0.0f;"),
    ("sgd: sum in descending batch order",
     "float s = g[p[k0].pos * dim + d];\n            for (int64_t k = k0 + 1; k < k1; ++k) s = s + g[p[k].pos * dim + d];",
     "float s = g[p[k1 - 1].pos * dim + d];\n            for (int64_t k = k1 - 2; k >= k0; --k) s = s + g[p[k].pos * dim + d];"),
    ("sgd: learning rate dropped", "            const float step = lr * s;\n            w[d] = w[d] - step;",
     "            const float step = s;\n            w[d] = w[d] - step;"),
    # L2 alignment
    ("l2: factor 2 dropped", "float s = 2.0f * diff;", "float s = diff;"),
    ("l2: step added", "w[d] = before - step;", "w[d] = before + step;"),
    ("l2: later gradients at the first target",
     "diff = before - e[p[k].pos * dim + d];", "diff = before - e[p[k0].pos * dim + d];"),
    # EMA
    ("ema: a and b swapped", "const float x = a * t[d];\n            const float y = b * v[d];",
     "const float x = b * t[d];\n            const float y = a * v[d];"),
    ("ema: mask ignored", "if (rows[i] < 0 || (mask && !mask[i])) continue;", "if (rows[i] < 0) continue;"),
    ("ema: decay applied to the new value", "t[d] = x + y;", "t[d] = a * (x + y);"),
    # int8 quantisation
    ("quantize: scale over 256 steps", "range / 255.0f", "range / 256.0f"),
    ("quantize: bias offset 127 scales", "const float offset = 128.0f * scale;", "const float offset = 127.0f * scale;"),
    ("quantize: truncation instead of round-to-nearest-even", "rintf(centred / scale)", "truncf(centred / scale)"),
    # dequant-score
    ("score: bias dropped",
     "(double)qtable[row * dim + d] * (double)scale[row] + (double)bias[row];",
     "(double)qtable[row * dim + d] * (double)scale[row];"),
    ("score: a miss scores the bias row 0", "if (row < 0) { out[r * cands + c] = 0.0f; continue; }",
     "if (row < 0) { out[r * cands + c] = (float)bias[0]; continue; }"),
    # decoupled key store
    ("key store: a hit does not stamp its row", "if (insert) stamps[rows[i]] = now;", "(void)0;"),
    ("key store: only hits are counted", "if (rows[i] >= 0) counts[rows[i]]++;",
     "if (rows[i] >= 0 && hit[i]) counts[rows[i]]++;"),
    ("key store: linear probing skips a slot", "s = (s + 1) % key_cap;", "s = (s + 2) % key_cap;"),
    ("ema: step evaluated in fp64, rounded once",
     "const float x = a * t[d];\n            const float y = b * v[d];\n            t[d] = x + y;",
     "const double x = (double)a * t[d];\n            const double y = (double)b * v[d];\n            t[d] = (float)(x + y);"),
    ("ema: rows outside the table accepted",
     "if (rows[i] < -1 || rows[i] >= num_rows) return ORC_EINVAL;\n    for (int64_t i = 0; i < n; ++i) {\n        if (rows[i] < 0 || (mask",
     "(void)0;\n    for (int64_t i = 0; i < n; ++i) {\n        if (rows[i] < 0 || (mask"),
    ("sgd: lr applied to every gradient",
     "float s = g[p[k0].pos * dim + d];\n            for (int64_t k = k0 + 1; k < k1; ++k) s = s + g[p[k].pos * dim + d];\n"
     "            const float step = lr * s;",
     "float s = lr * g[p[k0].pos * dim + d];\n            for (int64_t k = k0 + 1; k < k1; ++k) s = s + lr * g[p[k].pos * dim + d];\n"
     "            const float step = s;"),
    ("score: fp32 accumulation", "double acc = 0.0;", "float acc = 0.0f;"),
    ("score: user element shifted", "acc += x * (double)user[r * dim + d];",
     "acc += x * (double)user[r * dim + (d + 1) % dim];"),
    ("writeback: row set to e without the update", "            w[d] = w[d] - g;\n", "            (void)g; w[d] = src[d];\n"),
    ("dedup: keys ordered as unsigned",
     "if (x->key != y->key) return x->key < y->key ? -1 : 1;\n    if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;\n"
     "    return 0;\n}\n\nstatic int cmp_pos_first",
     "if (x->key != y->key) return (uint64_t)x->key < (uint64_t)y->key ? -1 : 1;\n"
     "    if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;\n    return 0;\n}\n\nstatic int cmp_pos_first"),
    ("quantize: symmetric scale", "const float range = hi - lo;",
     "const float range = 2.0f * (fabsf(hi) > fabsf(lo) ? fabsf(hi) : fabsf(lo));"),
    ("quantize: clamp at 126", "(v > 127.0f ? 127.0f : v)", "(v > 126.0f ? 126.0f : v)"),
    ("l2: gradient at the partly updated row", "diff = before - e[p[k].pos * dim + d];",
     "diff = (before - lr * s) - e[p[k].pos * dim + d];"),
    ("mpzch: inserts not stamped", "            identity[s] = id;\n            stamps[s] = now;", "            identity[s] = id;"),
    ("mpzch: a hit's row recorded as its bucket's first slot", "                rows[i] = base + j;\n                hit[i] = 1;",
     "                rows[i] = base;\n                hit[i] = 1;"),
    ("key store: new keys stamped now - 1", "            krows[slot] = r;\n            stamps[r] = now;",
     "            krows[slot] = r;\n            stamps[r] = now - 1;"),
    ("key store: overflow one row early", "if (*next_row >= max_rows || slot < 0) { st[2]++; continue; }",
     "if (*next_row >= max_rows - 1 || slot < 0) { st[2]++; continue; }"),
    ("key store: overflowed keys counted as inserted", "if (*next_row >= max_rows || slot < 0) { st[2]++; continue; }",
     "if (*next_row >= max_rows || slot < 0) { st[1]++; continue; }"),
]


def _build(text: str, out: str) -> None:
    c = out[:-3] + ".c"
    with open(c, "w") as f:
        f.write(text)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", c,
                           "-o", out, "-lm"])


def _run_pins(lib: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, HLR_ORACLE_LIBRARY=lib)
    return subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"], cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=300)


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


def test_every_planted_mistake_fails_a_pin(source, tmp_path):
    texts = [("unmodified", source)]
    for name, old, new in MUTANTS:
        assert source.count(old) == 1, f"mutant {name!r}: its text no longer occurs exactly once in oracle.c"
        texts.append((name, source.replace(old, new, 1)))
    libs = []
    for k, (name, text) in enumerate(texts):
        lib = str(tmp_path / f"oracle_m{k}.so")
        _build(text, lib)
        libs.append(lib)
    workers = max(1, min(8, (os.cpu_count() or 2)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(_run_pins, libs))
    base = results[0]
    assert base.returncode == 0, "the unmodified copy must pass every pin:\n" + base.stdout[-2000:]
    # returncode 1: pytest ran and a pin failed (a crash or a usage error is not a catch)
    survivors = [name for (name, _), r in zip(texts[1:], results[1:]) if r.returncode != 1]
    assert not survivors, "planted mistakes that no pin caught (or that crashed the run): " + ", ".join(survivors)
