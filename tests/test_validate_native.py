"""The C ABI's argument validation compiled on its own with the system C++
compiler and no HIP header (a host-only translation unit), run on the CPU
(also under the address and undefined-behaviour sanitizers where the
toolchain has them)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "acoustic_wave_propagation_amd", "csrc")


def _build_and_run(tmp_path, extra):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "validate_check")
    cmd = [cxx, "-std=c++17", "-O1", "-Wall", "-Werror", *extra,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "validate.cpp"),
           os.path.join(ROOT, "tests", "native", "validate_check.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return r, exe


def test_validation_without_hip(tmp_path):
    r, exe = _build_and_run(tmp_path, [])
    assert r.returncode == 0, r.stderr
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "validate ok" in out.stdout


def test_validation_under_sanitizers(tmp_path):
    r, exe = _build_and_run(tmp_path, ["-fsanitize=address,undefined",
                                       "-fno-sanitize-recover=all"])
    if r.returncode != 0:
        pytest.skip("sanitizers unavailable: " + r.stderr[-200:])
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stdout + out.stderr
