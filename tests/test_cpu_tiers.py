"""CPU tiers that need no GPU: every HIP source compiles for gfx950, and the
fp64 oracle and the host code of libpkv run clean under the address and
undefined-behaviour sanitizers.

- The oracle is built with gcc and -fsanitize=address,undefined and runs every
  pin (tests/run_pins.py) in a child process with the sanitizer runtimes
  preloaded (put in front of whatever LD_PRELOAD already holds).  A copy with a
  planted heap overflow must be caught, which shows the sanitizer is live.
- The host code of libpkv (pkv_api.cpp: argument checks, work split and
  workspace sizing of every entry point; pool.cpp: the block pool; the table
  helpers) is built with g++ under the same sanitizers, with the kernel
  launchers replaced by stubs (tests/sanitize/launch_stubs.cpp), and driven by
  tests/sanitize/host_driver.cpp: rejected and accepted calls of every entry
  point, random tables, random pool operation streams.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "paged_kv_cache_pools_amd", "csrc")
ORACLE_SRC = os.path.join(ROOT, "oracle", "pkv_oracle.c")
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _sanitizer_env():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    env = dict(os.environ)
    pre = [asan, ubsan] + ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else [])
    env["LD_PRELOAD"] = ":".join(pre)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


def _build_oracle(src, out):
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
           *SAN, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)


def _run_pins(lib, env):
    return subprocess.run([sys.executable, os.path.join(HERE, "run_pins.py"), lib], env=env,
                          capture_output=True, text=True, timeout=900)


def test_oracle_pins_under_sanitizers(tmp_path):
    env = _sanitizer_env()
    lib = str(tmp_path / "libpkv_oracle_san.so")
    _build_oracle(ORACLE_SRC, lib)
    r = _run_pins(lib, env)
    assert r.returncode == 0 and "FAILED: none" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]


def test_oracle_sanitizer_catches_a_planted_overflow(tmp_path):
    """The per-thread score buffer one element short: the first decode with a
    context of two or more tokens writes past it, and the run must fail with
    an AddressSanitizer report."""
    env = _sanitizer_env()
    src = open(ORACLE_SRC).read()
    old = ("double *scores = malloc(sizeof(double) * (size_t)(w->max_context_len > 0 ? "
           "w->max_context_len : 1));")
    assert src.count(old) == 1
    bad = tmp_path / "pkv_oracle.c"
    bad.write_text(src.replace(old, "double *scores = malloc(sizeof(double) * (size_t)"
                                    "(w->max_context_len > 1 ? w->max_context_len - 1 : 1));"))
    shutil.copy(os.path.join(ROOT, "oracle", "pkv_oracle.h"), tmp_path / "pkv_oracle.h")
    lib = str(tmp_path / "libpkv_oracle_bad.so")
    _build_oracle(str(bad), lib)
    r = _run_pins(lib, env)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-3000:]


def test_host_library_under_sanitizers(tmp_path):
    hip_inc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")
    if not os.path.isdir(os.path.join(hip_inc, "hip")):
        pytest.skip("HIP headers not installed")
    exe = str(tmp_path / "host_driver")
    srcs = [os.path.join(CSRC, "pkv_api.cpp"), os.path.join(CSRC, "pool.cpp"),
            os.path.join(HERE, "sanitize", "launch_stubs.cpp"),
            os.path.join(HERE, "sanitize", "host_driver.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", hip_inc,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0 and "0 check(s) failed" in r.stdout, r.stdout + r.stderr[-4000:]
    assert "runtime error" not in r.stderr, r.stderr[-4000:]


def test_hip_sources_compile_for_gfx950(tmp_path):
    """Every HIP and C++ source of libpkv compiles for gfx950 (device code
    included), so a source that no longer builds fails here, not only on a GPU
    machine."""
    from paged_kv_cache_pools_amd import build as hip_build

    hipcc = hip_build._hipcc()
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not installed")

    def compile_one(src):
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [hipcc, *hip_build.COMMON, *lang, "-c", os.path.join(CSRC, src), "-o",
               str(tmp_path / (src + ".o"))]
        r = subprocess.run(cmd, capture_output=True, text=True)
        return src, r.returncode, r.stderr

    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(compile_one, hip_build.SOURCES))
    failed = [(s, e[-3000:]) for s, rc, e in results if rc != 0]
    assert not failed, failed
    assert sorted(hip_build.SOURCES) == sorted(
        f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp"))), "a source is not built"
