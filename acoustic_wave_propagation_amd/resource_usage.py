"""Per-kernel register, LDS and occupancy figures of the library's gfx950
code objects, from the compiler's resource-usage remarks (no GPU needed).

    python -m acoustic_wave_propagation_amd.resource_usage > profiles/kernel_resources.md

Compiles each HIP source of the library for the device only, with the same
flags as the build, and prints a markdown table: one row per instantiated
kernel (demangled and shortened), with VGPRs, AGPRs, SGPRs, scratch (spills),
LDS bytes per workgroup and the waves per SIMD the registers allow.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
import tempfile

from .build import CSRC, FLAGS, INCLUDE, hipcc

SOURCES = ["star2p5d.hip", "sweeps_fused.hip", "wave2.hip"]
FIELDS = {
    "VGPRs": "vgprs", "AGPRs": "agprs", "TotalSGPRs": "sgprs",
    "ScratchSize [bytes/lane]": "scratch", "Occupancy [waves/SIMD]": "occupancy",
    "LDS Size [bytes/block]": "lds", "VGPRs Spill": "vgpr_spill",
}


def _remarks(src: str):
    flags = [f for f in FLAGS if f not in ("-shared", "-fPIC")]
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [hipcc(), *flags, "--cuda-device-only", "-c", "-I", INCLUDE,
               "-I", CSRC, os.path.join(CSRC, src), "-o",
               os.path.join(tmp, "k.o"), "-Rpass-analysis=kernel-resource-usage"]
        r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(r.stderr)
    kernels, cur = [], None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: (?:\s*)([^:]+?): (.*?) \[-Rpass-analysis", line)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2).strip()
        if key == "Function Name":
            cur = {"name": val}
            kernels.append(cur)
        elif cur is not None and key in FIELDS:
            cur[FIELDS[key]] = val
    return kernels


def _demangle(names):
    tool = shutil.which("c++filt")
    if tool is None:
        return names
    r = subprocess.run([tool], input="\n".join(names), capture_output=True,
                       text=True)
    out = r.stdout.splitlines()
    return out if len(out) == len(names) else names


def _short(name: str) -> str:
    name = re.sub(r"\bst::", "", name)
    name = re.sub(r"\(.*\)$", "", name)
    return name.replace("float", "f32").replace("double", "f64")


def main(argv=None):
    rows = []
    for src in SOURCES:
        ks = _remarks(src)
        for k, dn in zip(ks, _demangle([k["name"] for k in ks])):
            if "kernel" not in dn:
                continue
            rows.append((src, _short(dn), k))
    print("# Kernel resources (gfx950)\n")
    print("Command: `python -m acoustic_wave_propagation_amd.resource_usage`"
          " (device-only compile of each source with the library's flags and"
          " `-Rpass-analysis=kernel-resource-usage`).\n")
    print("| source | kernel | VGPRs | AGPRs | SGPRs | scratch B/lane | "
          "LDS B | waves/SIMD |")
    print("|---|---|---|---|---|---|---|---|")
    for src, name, k in rows:
        print("| %s | `%s` | %s | %s | %s | %s | %s | %s |" % (
            src, name, k.get("vgprs", "?"), k.get("agprs", "?"),
            k.get("sgprs", "?"), k.get("scratch", "?"), k.get("lds", "?"),
            k.get("occupancy", "?")))
    return 0


if __name__ == "__main__":
    sys.exit(main())
