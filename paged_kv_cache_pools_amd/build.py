"""Build libpkv.so (HIP, gfx950) in place: hipcc per source, then one link.
With --debug-bounds the same sources build libpkv_debug.so with
PKV_DEBUG_BOUNDS defined (kernels record the first out-of-range index they
clamp; see pkv_debug_status in include/pkv.h).

usage: python -m paged_kv_cache_pools_amd.build [--jobs N] [--debug-bounds]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpkv.so")
BUILD_DEBUG = os.path.join(HERE, "_build_debug")
LIB_DEBUG = os.path.join(HERE, "libpkv_debug.so")
SOURCES = ["pkv_api.cpp", "pool.cpp", "store.hip", "decode.hip", "prefill.hip", "copy.hip",
           "mixed.hip", "cascade.hip", "probe.hip"]

ARCH = "gfx950"
# Packed fp32 arithmetic is switched off for every device pass; the host pass
# warns that it does not know the feature, which is harmless.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall"]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src: str, debug: bool = False) -> str:
    out_dir = BUILD_DEBUG if debug else BUILD
    os.makedirs(out_dir, exist_ok=True)
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    extra = ["-DPKV_DEBUG_BOUNDS"] if debug else []
    cmd = [_hipcc(), *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(x for x in r.stderr.splitlines() if noise not in x)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(jobs: int = 4, verbose: bool = True, debug: bool = False) -> str:
    lib = LIB_DEBUG if debug else LIB
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, debug), SOURCES))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--debug-bounds", action="store_true")
    args = ap.parse_args()
    build(args.jobs, debug=args.debug_bounds)
