"""Build liblinattn.so for gfx950 with hipcc, in-tree.

    python -m long_sequence_causal_amd.build

compiles every source under ``csrc/`` (objects in ``_build/``) and links
``long_sequence_causal_amd/liblinattn.so``.  hipcc cross-compiles for gfx950
without a GPU present.  Packed-fp32 instruction selection is disabled for all
device code (-packed-fp32-ops).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblinattn.so")
ARCH = "gfx950"

SOURCES = ["la_fwd.hip", "la_scan.hip", "la_gate.hip", "la_tangent.hip", "la_step.hip",
           "la_noalloc.hip", "la_api.cpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False) -> str:
    """Compile all sources (in parallel) and link the shared library."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [cc] + _flags() + ["-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    errors = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if p.returncode != 0:
            errors.append(f"{src}:\n" + "\n".join(lines))
        elif verbose and lines:
            print("\n".join(lines))
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n\n".join(errors))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
