"""Build tests/host_asan/abi_driver: the C-ABI driver and the library's host
sources (*_api.cpp) compiled with AddressSanitizer on the host side only
(each -fsanitize= after -Xarch_host; the GPU code is the regular build's),
linked with the kernel objects of the regular build. Run by the repository's
build entry point after the library; the GPU test runs the binary."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "linear_attention_beam_gdn_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
OUT_DIR = os.path.join(BUILD, "host_asan")
DRIVER = os.path.join(HERE, "abi_driver")
API_SOURCES = ["onela_api.cpp", "fullstate_api.cpp", "replay_api.cpp", "prefill_api.cpp"]
KERNEL_OBJECTS = ["onela_kernels.o", "fullstate_kernels.o", "replay_kernels.o", "prefill_kernels.o"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def build(hipcc: str) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for src in API_SOURCES + [os.path.join(HERE, "abi_driver.cpp")]:
        path = src if os.path.isabs(src) else os.path.join(CSRC, src)
        obj = os.path.join(OUT_DIR, os.path.splitext(os.path.basename(path))[0] + ".o")
        _run([hipcc, *flags, *SAN, "-c", path, "-o", obj])
        objs.append(obj)
    kernels = [os.path.join(BUILD, o) for o in KERNEL_OBJECTS]
    missing = [k for k in kernels if not os.path.exists(k)]
    if missing:
        raise RuntimeError(f"kernel objects missing (build the library first): {missing}")
    tmp = DRIVER + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", *SAN, "-o", tmp, *objs, *kernels])
    os.replace(tmp, DRIVER)
    return DRIVER


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host-ASan build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
