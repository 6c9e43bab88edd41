"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The CPU oracle (oracle/kv4_oracle.c) and the host side of libkv4 (argument
checks, sizes and offsets, workspace carving, the capacity model, the
allocation-free entry point's checks) are rebuilt with clang's sanitizers
into a temporary directory, and the CPU test suite runs against those builds
in a child process with the sanitizer runtime preloaded.  Any out-of-bounds
access, use after free or undefined behaviour aborts the child.  Device code
is not instrumented (the sanitizer flags apply to the host pass only), and
nothing here needs a GPU.
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _runtime():
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return rt[-1] if rt else None


def _build(out):
    from int4_kv_cache_amd import build as kb

    lib_oracle = os.path.join(out, "liboracle_san.so")
    subprocess.run(["/opt/rocm/llvm/bin/clang", "-std=c11", "-O1", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", "-fno-fast-math", *SAN, "-o", lib_oracle,
                    os.path.join(ROOT, "oracle", "kv4_oracle.c"), "-lm"], check=True, capture_output=True)
    host_san = [f for flag in SAN for f in ("-Xarch_host", flag)]

    def compile_one(src):
        obj = os.path.join(out, os.path.splitext(src)[0] + ".o")
        r = subprocess.run([kb.HIPCC, *kb.CFLAGS, *host_san, "-c", os.path.join(kb.CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, kb.SOURCES))
    lib_kv4 = os.path.join(out, "libkv4_san.so")
    r = subprocess.run([kb.HIPCC, f"--offload-arch={kb.ARCH}", "-shared", "-fPIC", "-o", lib_kv4, *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return lib_oracle, lib_kv4


@pytest.mark.slow
def test_cpu_suite_under_asan_and_ubsan(tmp_path):
    rt = _runtime()
    if rt is None:
        pytest.skip("clang's sanitizer runtime is not installed")
    lib_oracle, lib_kv4 = _build(str(tmp_path))
    env = dict(os.environ, KV4_ORACLE_LIB=lib_oracle, KV4_LIB=lib_kv4, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    # -s: a sanitizer report goes to the child's stderr, not into a test's capture
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-s",
                        "-m", "not gpu and not slow", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    tail = (r.stdout[-3000:] + "\n" + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "Sanitizer" not in r.stdout + r.stderr, tail
