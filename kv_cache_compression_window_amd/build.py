"""Build ``libkvc.so`` for gfx950 in-tree with hipcc.

Usage: ``python -m kv_cache_compression_window_amd.build`` (or ``build()``).
Objects go to ``_build/`` at the repository root; the library is written next
to this file, where ``binding`` loads it.  Every HIP source is compiled with
packed fp32 instructions disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libkvc.so")
BENCH_DIR = os.path.join(CSRC, "bench")
BENCH_LIB_PATH = os.path.join(HERE, "libkvc_bench.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, folder: str = CSRC) -> str:
    path = os.path.join(folder, src)
    obj = os.path.join(BUILD_DIR, os.path.basename(folder) + "_" + src + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, *COMMON, *DEVICE, "-x", "hip", "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
    noise = "is not a recognized feature for this target"
    msg = "\n".join(line for line in (r.stdout + r.stderr).splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def _link(objs, path):
    tmp = path + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", *DEVICE, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    shutil.move(tmp, path)


def build(verbose: bool = True) -> str:
    """Compile every source and link libkvc.so (and bench.py's libkvc_bench.so,
    the hardware-ceiling kernels); returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    bench_srcs = sorted(f for f in os.listdir(BENCH_DIR) if f.endswith(".hip"))
    jobs = max(1, min(len(srcs) + len(bench_srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
        bench_objs = list(ex.map(lambda f: _compile(f, BENCH_DIR), bench_srcs))
    _link(objs, LIB_PATH)
    _link(bench_objs, BENCH_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources, {BENCH_LIB_PATH} from {len(bench_srcs)}")
    return LIB_PATH


if __name__ == "__main__":
    build()
