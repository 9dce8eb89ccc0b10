"""Host code under the address and undefined-behaviour sanitizers (CPU only).

* la_api.cpp -- every argument check, workspace size and launch plan of the
  C ABI -- is built with g++ -fsanitize=address,undefined together with
  stand-in launchers that launch nothing (tests/hostcheck/stub_launchers.cpp)
  and driven through every entry point by tests/hostcheck/abi_driver.cpp:
  valid shapes, invalid arguments, huge sizes and a sweep of random shapes.
* oracle/lao.c is built with the same sanitizers and the oracle's pins
  (tests/test_oracle_pins.py) run against that build.
Any sanitizer report aborts the run and fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "hostcheck")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not available")


def test_abi_host_path_under_sanitizers(tmp_path):
    _need("g++")
    if not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("HIP headers not available")
    exe = tmp_path / "abi_driver"
    cmd = (["g++", "-std=c++17", "-O1"] + SAN +
           ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
            "-I", os.path.join(ROOT, "include"),
            "-I", os.path.join(ROOT, "long_sequence_causal_amd", "csrc"),
            os.path.join(ROOT, "long_sequence_causal_amd", "csrc", "la_api.cpp"),
            os.path.join(HERE, "stub_launchers.cpp"), os.path.join(HERE, "abi_driver.cpp"),
            "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
            "-o", str(exe)])
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "0 failures" in r.stdout


def test_oracle_pins_under_sanitizers(tmp_path):
    _need("gcc")
    lib = tmp_path / "liblao_san.so"
    cmd = (["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off"] + SAN +
           [os.path.join(ROOT, "oracle", "lao.c"), "-o", str(lib), "-lm"])
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("libasan not found")
    env = dict(os.environ, LAO_LIB=str(lib), LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",  # the interpreter's own allocations
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    which = subprocess.run([sys.executable, "-c", "from oracle import lao; lao._load(); print(lao._LIB)"],
                           capture_output=True, text=True, env=env, cwd=ROOT, timeout=120)
    assert which.stdout.strip() == str(lib), which.stdout + which.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    print(r.stdout[-3000:], r.stderr[-3000:])
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr
