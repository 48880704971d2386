"""Compile the gfx950 HIP library ``liblora_mi355x.so`` in-tree.

    python -m lora_adapter_application_amd.build

The library is the C ABI of ``include/lora_mi355x.h``: the runtime
(``csrc/lora_runtime.cpp``), the low-rank kernels (``csrc/lora_kernels.hip``)
and the saved-module kernels (``csrc/lora_saved.hip``).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "liblora_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, "lora_kernels.hip"), os.path.join(CSRC, "lora_saved.hip"),
           os.path.join(CSRC, "lora_runtime.cpp")]

# Packed-fp32 instructions stay disabled for device code (the host pass warns
# that it does not know the feature; that is harmless).
HIPCC_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
               "-Wall", "-Wno-unused-result",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", INCLUDE]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Always recompile; returns the path of the shared library."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
