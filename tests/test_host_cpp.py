"""Host-side C++ checks of library internals and of the C ABI's argument checking, compiled
as plain host C++ (no device code) with AddressSanitizer and UndefinedBehaviorSanitizer and
run on the CPU: the tile cut of the device-side chunk loop, the workgroup -> tile map, and
the C ABI's host code (ub_api.cpp, ub_plan.cpp) with its device launchers stubbed out."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunked_tp_overlap_amd", "csrc")
CPP = os.path.join(ROOT, "tests", "cpp")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _cxx():
    for c in (os.path.join(ROCM, "lib", "llvm", "bin", "clang++"), shutil.which("clang++")):
        if c and os.path.exists(c):
            return c
    return None


def _build_and_run(tmp_path, name, sources, libs=(), timeout=300, hip=False):
    """hip: the sources include device code (compiled for gfx950 too), so the sanitizers
    are given to the host compilation only."""
    exe = tmp_path / name
    lang = ["-x", "hip", "--offload-arch=gfx950"] if hip else ["-x", "c++", "-D__HIP_PLATFORM_AMD__"]
    san = [f for s in SAN for f in ("-Xarch_host", s)] if hip else SAN
    cmd = [_cxx(), *lang, "-std=c++17", "-O1", "-g", *san,
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *sources, "-o", str(exe)]
    if libs:
        cmd += ["-L", os.path.join(ROCM, "lib"), *libs, f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=timeout, env=ENV)
    assert res.returncode == 0, (res.stdout + res.stderr)[-4000:]
    assert res.stdout.startswith("ok"), res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-4000:]
    return res.stdout


@pytest.mark.skipif(_cxx() is None, reason="clang++ not available")
def test_tile_aligned_units(tmp_path):
    _build_and_run(tmp_path, "tile_aligned_units_check",
                   [os.path.join(CPP, "tile_aligned_units_check.cpp"), os.path.join(CSRC, "ub_plan.cpp")])


@pytest.mark.skipif(_cxx() is None, reason="clang++ not available")
def test_tile_of(tmp_path):
    """The workgroup -> tile map of the device-side chunk loop covers every tile once."""
    _build_and_run(tmp_path, "tile_of_check", [os.path.join(CPP, "tile_of_check.cpp")],
                   libs=("-lamdhip64",), hip=True)


@pytest.mark.skipif(_cxx() is None, reason="clang++ not available")
def test_segmentation_choice(tmp_path):
    """choose_segmentation over the workloads' shapes and random ones: deterministic, from
    the priced segment counts, inside the row range on 64-row boundaries, on a built tile,
    within the 64 MiB of partials the scratch sizing promises; none for batched launches."""
    out = _build_and_run(tmp_path, "segmentation_check",
                         [os.path.join(CPP, "segmentation_check.cpp"), os.path.join(CSRC, "gemm_bf16.hip"),
                          os.path.join(CSRC, "ub_plan.cpp")],
                         libs=("-lamdhip64",), hip=True, timeout=600)
    checks, segmented = map(int, out.split()[1:3])
    assert checks == 6000 and segmented > 100


@pytest.mark.skipif(_cxx() is None, reason="clang++ not available")
def test_abi_argument_paths_under_sanitizers(tmp_path):
    """The C ABI's argument checks, state handling and messages, and a randomized sweep of
    arguments through every entry point, with no sanitizer report (the device launchers
    are stubs; calls that pass the checks stop at the first HIP call, with no GPU here)."""
    out = _build_and_run(tmp_path, "abi_args_check",
                         [os.path.join(CSRC, "ub_api.cpp"), os.path.join(CSRC, "ub_plan.cpp"),
                          os.path.join(CPP, "kernel_stubs.cpp"), os.path.join(CPP, "abi_args_check.cpp")],
                         libs=("-lamdhip64", "-lrocprofiler-sdk-roctx"))
    assert int(out.split()[1]) > 5000
