"""Build the HIP libraries in-tree for gfx950: libqlinear.so (the library)
and libqlprobe.so (the benchmark's HBM read-bandwidth probe).

Usage: python -m bit_group_quantized_amd.build   (or build() from Python)
Each source is compiled in parallel with hipcc, then linked into a shared
library next to this file.  Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libqlinear.so"
SOURCES = ["gemv.hip", "gemm.hip", "route.hip", "misc.hip", "codecs.hip", "noalloc.hip", "capi.cpp"]
PROBE_NAME = "libqlprobe.so"
PROBE_SOURCES = ["readprobe.hip"]
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # Keep the compiler from forming packed-fp32 instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def _hipcc() -> str:
    cand = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libqlinear")
    return cand


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _link(hipcc, sources, name, tmp):
    objs, cmds = [], []
    for src in sources:
        obj = os.path.join(tmp, name + "." + src + ".o")
        objs.append(obj)
        cmds.append([hipcc, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj])
    return objs, cmds


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    out = os.path.join(PKG, LIB_NAME)
    with tempfile.TemporaryDirectory(prefix="qlbuild_") as tmp:
        libs = [(out, *_link(hipcc, SOURCES, LIB_NAME, tmp)),
                (os.path.join(PKG, PROBE_NAME), *_link(hipcc, PROBE_SOURCES, PROBE_NAME, tmp))]
        cmds = [c for _, _, cs in libs for c in cs]
        with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
            logs = list(ex.map(_run, cmds))
        for path, objs, _ in libs:
            tmp_lib = path + ".tmp"
            _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, *objs])
            os.replace(tmp_lib, path)
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
        print(f"built {out} and {PROBE_NAME}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
