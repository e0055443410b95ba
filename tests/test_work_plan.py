"""Host logic of the launch geometry: the z chunking of a streamed box and the
map from a workgroup id back to its tile and chunk
(acoustic_wave_propagation_amd/csrc/work_plan.h, the same code the kernels
run), compiled with the host C++ compiler and checked exhaustively over a
grid of shapes -- no GPU, no HIP."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "acoustic_wave_propagation_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "native", "work_plan_check.cpp")


def test_work_plans_cover_the_box(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "work_plan_check")
    subprocess.run([cxx, "-std=c++17", "-O2", "-Wall", "-I", CSRC, SRC, "-o",
                    exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert ", 0 bad" in r.stdout
    # some plans of the grid take the mixed chunking
    mixed = int(r.stdout.split("(")[-1].split(" mixed")[0])
    assert mixed > 0
    # Worked by hand: uniform chunking is best at 5 chunks of 103 planes
    # (ceil(1520/256) = 6 rounds of 115 = 690); the mixed plan streams 256
    # whole columns (one round of 524) and the other 48 columns in 5 chunks
    # of 103 (240 workgroups, one round of 115): 639 < 690.
    assert ("plan(512 planes, 304 tiles, cap 256, fill 12, min 16): nwg 496, "
            "A 256 tiles x 512, B 5 chunks of 103") in r.stdout, r.stdout
    # equal chunks: 512 planes in 4 chunks of 128 (not 132 + 132 + 132 + 116)
    assert "plan(512 planes, 64 tiles, cap 256): nwg 256, 4 chunks of 128" \
        in r.stdout, r.stdout
