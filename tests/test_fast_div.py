"""The kernels divide token indices by the block size and workgroup indices
by the virtual KV head count with a host-computed multiplier and shift
(make_fast_div in internal.h): a C++ driver (fast_div_check.cpp) checks the
quotient the kernels form against integer division for every divisor up to
8192 over the index range they use.  CPU only."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

from conftest import ROOT

GXX = shutil.which("g++")


@pytest.mark.skipif(GXX is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not available")
def test_fast_division_is_exact(tmp_path):
    exe = str(tmp_path / "fast_div_check")
    r = subprocess.run([GXX, "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
                        "-I", os.path.join(ROOT, "include"),
                        "-I", os.path.join(ROOT, "paged_kv_cache_resolve_amd", "csrc"),
                        os.path.join(ROOT, "tests", "fast_div_check.cpp"), "-o", exe],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:]
    assert " 0 failures" in r.stdout
