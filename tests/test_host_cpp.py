"""Host-side C++ checks of library internals that the C ABI does not expose, compiled with
hipcc in host mode and run on the CPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunked_tp_overlap_amd", "csrc")


def _hipcc():
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_tile_aligned_units(tmp_path):
    exe = tmp_path / "tile_aligned_units_check"
    cmd = [_hipcc(), "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(ROOT, "tests", "cpp", "tile_aligned_units_check.cpp"),
           os.path.join(CSRC, "ub_plan.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok"), res.stdout


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_tile_of(tmp_path):
    """The workgroup -> tile map of the device-side chunk loop covers every tile once."""
    exe = tmp_path / "tile_of_check"
    cmd = [_hipcc(), "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(ROOT, "tests", "cpp", "tile_of_check.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok"), res.stdout
