"""Host logic of the Jacobi ping-pong: the split of the sweeps into fused
passes (acoustic_wave_propagation_amd/csrc/pass_plan.h), compiled with the
host C++ compiler and checked exhaustively -- no GPU, no HIP."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "acoustic_wave_propagation_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "native", "pass_plan_check.cpp")


def test_pass_plans(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "pass_plan_check")
    subprocess.run([cxx, "-std=c++17", "-O1", "-Wall", "-I", CSRC, SRC, "-o",
                    exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 bad" in r.stdout
    # 10 sweeps with up to six fused at the measured costs: two passes of
    # five (2 x 2.176 < 2.696 + 1.842; the result stays in buffer 0)
    assert "10 sweeps, up to 6 fused: 5 5" in r.stdout, r.stdout
