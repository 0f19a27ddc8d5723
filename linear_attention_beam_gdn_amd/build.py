"""Build libonela.so (the C-ABI library of the OneLA GDN decode step) and
libonela_probes.so (the measurement probes of bench.py) for gfx950.

Run `python -m linear_attention_beam_gdn_amd.build`. It always recompiles and
writes the library next to this file, so it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libonela.so")
PROBE_LIB = os.path.join(PKG, "libonela_probes.so")   # measurement probes of bench.py

ARCH = "gfx950"
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 instructions stay off (they are generated from float code
    # otherwise); the host pass warns that it does not know the feature
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
SOURCES = ["onela_kernels.hip", "onela_api.cpp", "fullstate_kernels.hip", "fullstate_api.cpp",
           "replay_kernels.hip", "replay_api.cpp", "prefill_kernels.hip", "prefill_api.cpp"]
PROBE_SOURCES = ["probes.hip"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libonela.so")
    return path


def _link(cc, sources, lib, verbose):
    objs = []
    for src in sources:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        _run([cc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = lib + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Build libonela.so (the decode path) and libonela_probes.so (bench probes)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    _link(cc, SOURCES, LIB, verbose)
    _link(cc, PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose=True))
