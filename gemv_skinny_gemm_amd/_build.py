"""Builds the gfx950 shared libraries in-tree with hipcc.

libskinny_gemm.so          the C-ABI library (kernels + host entry points)
synth/libskinny_synth.so   the GPU twin of the seeded input generator (test and
                           benchmark data only; shares no code with the library)
probe/libskinny_probe.so   an arithmetic-free streaming read, the HBM read
                           ceiling bench.py reports beside the library's rate
"""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(PKG, "csrc")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for every device compile.
COMMON = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-command-line-argument", f"-I{INCLUDE}"]

LIBS = {
    "libskinny_gemm.so": [os.path.join(CSRC, "skinny_gemm.hip")],
    os.path.join("synth", "libskinny_synth.so"): [os.path.join(PKG, "synth", "synth_gpu.hip")],
    os.path.join("probe", "libskinny_probe.so"): [os.path.join(PKG, "probe", "stream_read.hip")],
}


def lib_path(name: str) -> str:
    return os.path.join(PKG, name)


def build_lib(name: str, verbose: bool = False) -> str:
    srcs = LIBS[name]
    out = lib_path(name)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *COMMON, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {name}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> list[str]:
    return [build_lib(n, verbose) for n in LIBS]


if __name__ == "__main__":
    for p in build_all(verbose=True):
        print("built", p)
