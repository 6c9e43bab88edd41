"""Build libkv4.so (gfx950) in-tree with hipcc.

    python -m int4_kv_cache_amd.build

Every source under csrc/ is compiled as HIP for gfx950 and linked into
int4_kv_cache_amd/libkv4.so.  Flags: -O3, IEEE fp32 divide (the quantizer's
rounding decisions depend on it), no fast-math, and packed-FP32 instruction
generation disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkv4.so")
SOURCES = ["api.cpp", "append.hip", "decode.hip", "probe.hip"]
ARCH = os.environ.get("KV4_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math", "-ffp-contract=fast",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    # hipcc warns that the host pass does not know the packed-fp32 feature: harmless
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
