"""The library's host code (pool handles, free-block stack, block manager,
argument validation) under AddressSanitizer, UndefinedBehaviorSanitizer and
LeakSanitizer: a copy of the library is built with the sanitizers on its host
side only (device code is compiled as usual and never launched), and a C++
driver (host_sanitizer_driver.cpp) runs random manager traffic, detaches
managers by destroying their pool first, and feeds bad arguments to the entry
points.  CPU only; skipped where hipcc is missing."""

from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from conftest import ROOT

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CSRC = os.path.join(ROOT, "paged_kv_cache_resolve_amd", "csrc")
SOURCES = ["api.cpp", "launch_cache.cpp", "block_manager.cpp", "copy_kernels.hip",
           "decode_mfma.hip", "decode_generic.hip", "decode_merge.hip"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_code_is_sanitizer_clean(tmp_path):
    common = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC, *SAN]

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        r = subprocess.run([HIPCC, *common, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True, timeout=900)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    lib = str(tmp_path / "libpagedkv_san.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, "-o", lib, *objs],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = str(tmp_path / "driver")
    r = subprocess.run([HIPCC, "-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include"), *SAN,
                        "-x", "c++", os.path.join(ROOT, "tests", "host_sanitizer_driver.cpp"),
                        "-x", "none", lib, "-o", exe, f"-Wl,-rpath,{tmp_path}"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "0 failures" in r.stdout
