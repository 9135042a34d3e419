"""Builds libhlr.so (HIP, gfx950) in-tree with hipcc.

Every translation unit is compiled with:
  --offload-arch=gfx950            MI355X (CDNA4), wave64
  -ffp-contract=off                no FMA contraction: each fp32 operation of
                                   the row updates rounds on its own
  -fno-gpu-flush-denormals-to-zero keep fp32 denormals (IEEE results)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                   no packed fp32 instructions
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libhlr.so")
# streaming kernels for the benchmark's HBM-ceiling mode, a library of their own
PROBE_SOURCES = ["bwprobe.hip"]
PROBE_LIB = os.path.join(HERE, "libhlr_bwprobe.so")

SOURCES = ["capi.hip", "mpzch.hip", "gather.hip", "dedup.hip", "writeback.hip", "ema.hip", "score.hip", "quantize.hip", "publish.hip", "keystore.hip", "mlstep.hip", "step.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas", "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    jobs = min(len(srcs), max(1, (os.cpu_count() or 4)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


def asm(src: str, out: str | None = None) -> str:
    """Device assembly of one source (for inspection of code built here)."""
    out = out or os.path.join(BUILD, os.path.splitext(src)[0] + ".s")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = [HIPCC, *FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    subprocess.check_call(cmd)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
