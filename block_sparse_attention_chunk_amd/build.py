"""Build libbsa.so (HIP, gfx950) in-tree with hipcc, and the benchmark's
bandwidth-ceiling kernel libbsa_ceiling.so.

    python -m block_sparse_attention_chunk_amd.build [--jobs N]

Every source compiles on a CPU-only machine (hipcc cross-compiles for the
gfx950 target); the shared library lands next to this file.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libbsa.so")
# the benchmark's bandwidth-ceiling kernel, a library of its own
CEILING_SRC = "ceiling.hip"
CEILING_LIB = os.path.join(HERE, "libbsa_ceiling.so")

SOURCES = ["api.cpp", "meta.hip", "score.hip", "select.hip", "router.hip", "decode.hip", "select_decode.hip", "tile_prefill.hip"]
ARCH = "gfx950"
# Packed fp32 vector ops stay off: the compiler keeps plain v_fma_f32 / v_mul_f32.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-munsafe-fp-atomics", "-Wno-unused-result", "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, src + ".o")
    cmd = [hipcc()] + HIP_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc()] + HIP_FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES + [CEILING_SRC]))
    _link(objs[:-1], LIB, verbose)
    _link(objs[-1:], CEILING_LIB, verbose)
    return LIB


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(lib)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    a = ap.parse_args(argv)
    build(a.jobs, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
