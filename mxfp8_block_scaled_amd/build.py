"""Builds libmxfp8.so, the gfx950 HIP library behind include/mxfp8.h, in-tree.

    python -m mxfp8_block_scaled_amd.build

Every call recompiles (hipcc cross-compiles for gfx950; no GPU is needed).
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmxfp8.so")
# the same sources built with MX_CYCLE_STAMPS: the GEMM kernels also record per-block
# cycle stamps (bench.py --cycle-stamps); never loaded by the library's own callers
STAMPS_LIB = os.path.join(HERE, "libmxfp8_stamps.so")
SOURCES = ["abi.cpp", "cast.hip", "gemm.hip", "pad.hip", "convert.hip", "probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep packed-fp32 VALU forms out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
    "-I" + os.path.join(ROOT, "include"),
]


def build(verbose=False, stamps=False):
    """Builds libmxfp8.so, or with stamps=True the instrumented libmxfp8_stamps.so."""
    lib = STAMPS_LIB if stamps else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC] + FLAGS + (["-DMX_CYCLE_STAMPS"] if stamps else []) + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    # every kernel launched from host code must have its host stub defined in the
    # library; a template whose host-side instantiation failed leaves it undefined
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in nm.stdout.splitlines() if "_ZN2mx" in ln]
    if missing:
        raise RuntimeError("libmxfp8.so would have undefined kernel symbols: " + ", ".join(missing))
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, stamps="--stamps" in sys.argv))
