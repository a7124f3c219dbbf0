"""Build libmoe.so (HIP kernels for gfx950 + the C ABI) in the package directory.

Run ``python -m expert_offloaded_routed_amd._build`` or call ``build()``.  hipcc cross-compiles
for gfx950 on a machine without a GPU.
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
LIB = os.path.join(PKG, "libmoe.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")

HIP_SOURCES = ["moe_kernels.hip", "moe_dcache.hip", "moe_formats.hip"]
HOST_SOURCES = ["moe_api.cpp", "moe_pack.cpp", "moe_cache.cpp", "moe_cold.cpp", "moe_stage.cpp"]

# Packed fp32 instructions are kept out of every kernel (the compiler would otherwise form
# v_pk_* from scalar float code).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)


def kernel_source_sha() -> str:
    """Hash of the device sources (kernels and the headers they include)."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def build(verbose: bool = False) -> str:
    """Compile every source and link libmoe.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    common = ["-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC, "-Wall"]
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        _run([hipcc, "-x", "hip", "--offload-arch=gfx950", *common, *DEVICE_FLAGS, "-c",
              os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        _run([hipcc, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, *common, "-ffp-contract=off", "-pthread", "-c",
              os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-pthread", "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
