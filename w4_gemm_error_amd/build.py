"""Build libw4ec.so (HIP, gfx950) in-tree with hipcc.

    python -m w4_gemm_error_amd.build

Every source under csrc/ is compiled separately (in parallel) and linked
into ``w4_gemm_error_amd/libw4ec.so``.  All device code is built with
packed-FP32 instructions disabled.
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
OBJ_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libw4ec.so")
ARCH = os.environ.get("W4EC_OFFLOAD_ARCH", "gfx950")

SOURCES = ["api.cpp", "quant_pack.hip", "decode.hip", "prefill.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON_FLAGS
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in line and "is not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build()
