"""Build libstencil3d.so in-tree with hipcc for gfx950.

    python -m acoustic_wave_propagation_amd.build

All HIP code is compiled with packed-fp32 instructions disabled; the library
links only the HIP runtime.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libstencil3d.so")
SOURCES = ["star2p5d.hip", "sweeps_fused.hip", "wave2.hip", "validate.cpp", "api.cpp"]
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-variable", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every HIP source into LIB (always recompiles)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES],
           "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (r.returncode, out))
    if verbose and out:
        print(out, flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
