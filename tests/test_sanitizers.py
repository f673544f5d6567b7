"""CPU code under AddressSanitizer and UndefinedBehaviorSanitizer.

* The float64 oracle's pins (tests/test_oracle.py) run again in a child
  process with the oracle built instrumented (W4EC_ORACLE_SANITIZE=1) and the
  ASan runtime preloaded into the interpreter.
* The library's host side -- argument validation, launch plans and workspace
  sizing in api.cpp -- is compiled for the host only, instrumented, and
  driven by tests/host_san/abi_checks.cpp over invalid arguments and a sweep
  of valid shapes, with stub launchers that check each plan against the
  workspace the caller sized (no GPU involved).

Device code is never instrumented (the sanitizer flags apply to the host
compilation only).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "w4_gemm_error_amd", "csrc")
BUILD = os.path.join(ROOT, "tests", "host_san", "_build")


def _libasan():
    try:
        path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                              check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_ubsan():
    asan = _libasan()
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    env = dict(os.environ, W4EC_ORACLE_SANITIZE="1", LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"),
                          "-q", "-x", "-p", "no:cacheprovider"], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "AddressSanitizer" not in tail and "runtime error" not in tail, tail


def test_host_layer_under_asan_ubsan():
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    if not os.path.exists(hipcc) and shutil.which("hipcc") is None:
        pytest.skip("hipcc is not installed")
    hipcc = hipcc if os.path.exists(hipcc) else "hipcc"
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "abi_checks")
    cmd = [hipcc, "-x", "hip", "--cuda-host-only", "-O1", "-g", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-std=c++17",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(ROOT, "tests", "host_san", "abi_checks.cpp"), os.path.join(CSRC, "api.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0", HIP_VISIBLE_DEVICES=""))
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "abi checks ok" in run.stdout
