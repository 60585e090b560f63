"""The fused kernel divides by launch constants (team size, queries per sequence, compress
ratio, ring rows, dim quads, block size) with host-computed multipliers.  This CPU test
builds the host side of that arithmetic (the same inline functions the kernel uses) and
checks it against ordinary integer division."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc missing")
def test_fast_division_matches_integer_division(tmp_path):
    exe = str(tmp_path / "fastdiv_check")
    src = os.path.join(ROOT, "tests", "host", "fastdiv_check.cpp")
    r = subprocess.run([HIPCC if os.path.exists(HIPCC) else "hipcc", "-O2", "-std=c++17", "-x", "hip",
                        "--offload-arch=gfx950", "-o", exe, src], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "fastdiv ok" in r.stdout, r.stdout + r.stderr
