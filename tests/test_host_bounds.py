"""Host-side check of the bound arithmetic of the push work lists (CPU only).

The registration of nonzero vector blocks counts one entry per leader; with
an x_idx that is not strictly increasing a block can have several leaders, so
the raw count can reach 16 nb.  tests/host_checks/meta_bounds.cpp compiles the
library's own meta.h for the host and checks that the count the kernels use
is clamped to the list's capacity and that a pushing call that enumerates its
chunks from the list never exceeds the LDS prefix array (PUSH_LIST_MAX).
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not found")
def test_push_list_bounds_host(tmp_path):
    src = os.path.join(HERE, "host_checks", "meta_bounds.cpp")
    exe = str(tmp_path / "meta_bounds")
    hipcc = HIPCC if os.path.exists(HIPCC) else shutil.which("hipcc")
    r = subprocess.run([hipcc, "--offload-host-only", "-x", "hip", "-std=c++17", "-O1", src, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not found")
def test_offset_limits_host(tmp_path):
    src = os.path.join(HERE, "host_checks", "offset_bounds.cpp")
    exe = str(tmp_path / "offset_bounds")
    hipcc = HIPCC if os.path.exists(HIPCC) else shutil.which("hipcc")
    r = subprocess.run([hipcc, "--offload-host-only", "-x", "hip", "-std=c++17", "-O1", src, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 failures" in r.stdout
