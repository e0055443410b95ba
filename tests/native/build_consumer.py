"""Compile tests/native/abi_consumer.c (a plain C99 program that links
libstencil3d.so and the HIP runtime's C API) next to its source.

    python tests/native/build_consumer.py
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_consumer.c")
EXE = os.path.join(HERE, "abi_consumer")


def build() -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    pkg = os.path.join(ROOT, "acoustic_wave_propagation_amd")
    cmd = [cc, "-std=c99", "-O1", "-Wall", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(rocm, "include"), SRC, "-L", pkg, "-lstencil3d",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath," + pkg, "-Wl,-rpath," + os.path.join(rocm, "lib"),
           "-o", EXE + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build())
    sys.exit(0)
