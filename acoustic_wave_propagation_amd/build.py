"""Build libstencil3d.so in-tree with hipcc for gfx950.

    python -m acoustic_wave_propagation_amd.build

Each source is compiled to an object of its own (in parallel), then the
objects are linked into the shared library.  All HIP code is compiled with
packed-fp32 instructions disabled; the library links only the HIP runtime.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libstencil3d.so")
OBJDIR = os.path.join(PKG, "_build")
SOURCES = ["star2p5d.hip", "sweeps_fused.hip", "wave2.hip", "noalloc.hip",
           "validate.cpp", "api.cpp"]
# copy kernels with the stencil's memory walk, for measuring its ceiling
# (bench.py --ceilings); a library of their own
WALK_SOURCE = "walk_copy.hip"
WALK_LIB = os.path.join(PKG, "libwalkcopy.so")
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-variable", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _clean(text: str) -> str:
    return "\n".join(l for l in text.splitlines()
                     if "packed-fp32-ops" not in l and l.strip())


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    return r.returncode, _clean(r.stdout + r.stderr)


def build(verbose: bool = False, extra_flags=(), jobs: int | None = None) -> str:
    """Compile every source into LIB (always recompiles)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    os.makedirs(OBJDIR, exist_ok=True)
    tag = "%d" % os.getpid()
    objs = [os.path.join(OBJDIR, os.path.splitext(s)[0] + ".%s.o" % tag)
            for s in SOURCES]
    walk_obj = os.path.join(OBJDIR, "walk_copy.%s.o" % tag)
    cmds = [[hipcc(), *FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-c",
             os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES + [WALK_SOURCE], objs + [walk_obj])]
    jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    try:
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(lambda c: _run(c, verbose), cmds))
        for (rc, out), s in zip(results, SOURCES + [WALK_SOURCE]):
            if rc != 0:
                raise RuntimeError("hipcc failed on %s (%d):\n%s" % (s, rc, out))
            if verbose and out:
                print(out, flush=True)
        tmp = LIB + ".tmp" + tag
        rc, out = _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC",
                        *objs, "-Wl,-rpath," + os.path.join(rocm, "lib"),
                        "-o", tmp], verbose)
        if rc != 0:
            raise RuntimeError("link failed (%d):\n%s" % (rc, out))
        os.replace(tmp, LIB)
        rc, out = _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", walk_obj,
                        "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", tmp], verbose)
        if rc != 0:
            raise RuntimeError("link failed (%d):\n%s" % (rc, out))
        os.replace(tmp, WALK_LIB)
    finally:
        for o in objs + [walk_obj]:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
