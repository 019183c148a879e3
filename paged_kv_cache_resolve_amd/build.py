"""Build libpagedkv.so in-tree for gfx950 with hipcc.

    python -m paged_kv_cache_resolve_amd.build [-v]

Objects go to paged_kv_cache_resolve_amd/_build/, the library to
paged_kv_cache_resolve_amd/libpagedkv.so, and the HBM read-ceiling probe
(a measurement helper with its own small ABI, include/pagedkv_probe.h) to
paged_kv_cache_resolve_amd/libpagedkv_probe.so.  Every call recompiles.
Importing the package does not load the library, so this module runs on a
tree where it has not been built yet.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libpagedkv.so")
PROBE_LIB_PATH = os.path.join(HERE, "libpagedkv_probe.so")
PROBE_SOURCES = ["probe/read_ceiling.hip"]

SOURCES = [
    "api.cpp",
    "launch_cache.cpp",
    "block_manager.cpp",
    "copy_kernels.hip",
    "decode_mfma.hip",
    "decode_generic.hip",
    "decode_merge.hip",
]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# Packed fp32 VALU instructions are kept out of the generated code.  MFMA
# results are kept in VGPRs (the decode kernel rescales its accumulator with
# VALU ops every chunk; AGPR accumulators would need copies both ways).
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0].replace("/", "_") + ".o")
    cmd = [HIPCC, *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs, path: str, verbose: bool) -> None:
    tmp = path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(path)} failed:\n{r.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(min(len(srcs), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:len(SOURCES)], LIB_PATH, verbose)
    _link(objs[len(SOURCES):], PROBE_LIB_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
