"""Build libpa.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m paged_kv_cache_121_amd.build            # or build() from Python

Every HIP translation unit under csrc/ is compiled to an object in
``_build/`` (in parallel), then linked into ``paged_kv_cache_121_amd/libpa.so``.
The benchmark's HBM read-rate probe (``read_probe.hip`` beside bench.py) is
built into ``libpa_probe.so`` next to it, apart from the library.  All device
code is compiled with packed-fp32 instructions disabled.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa.so")
PROBE_SRC = os.path.join(ROOT, "read_probe.hip")
PROBE_LIB = os.path.join(ROOT, "libpa_probe.so")
ARCH = "gfx950"

SOURCES = ["pa_api.hip", "cache_ops.hip", "decode.hip", "prefill.hip"]  # HIP: device and host code
HOST_SOURCES = ["block_manager.cpp"]                      # host-only C++ (g++)
ROCM_INCLUDE = "/opt/rocm/include"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (a ROCm toolchain is required to build libpa.so)")


def _compile(src: str, hipcc: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    if src.endswith(".cpp"):
        cxx = shutil.which("g++") or "g++"
        cmd = [cxx, "-O3", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}", f"-I{CSRC}",
               f"-I{ROCM_INCLUDE}", "-c", os.path.join(CSRC, src), "-o", obj]
    else:
        cmd = [hipcc, *COMMON_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile and link libpa.so; returns its path.  Always rebuilds."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = list(extra_flags or [])
    sources = SOURCES + HOST_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(sources), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, extra), sources))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_probe(hipcc, extra, verbose)
    return LIB


def build_probe(hipcc: str, extra: list[str], verbose: bool = False) -> str:
    """libpa_probe.so: the benchmark's HBM read-rate probe."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc, *COMMON_FLAGS, *extra, "-shared", PROBE_SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for read_probe.hip:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}")
    return PROBE_LIB


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
