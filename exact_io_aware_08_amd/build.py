"""Build libfa_fwd.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m exact_io_aware_08_amd.build [--isa DIR]

Compiles with hipcc for --offload-arch=gfx950 only.  Packed-fp32 VALU
instructions are disabled on the device pass (-packed-fp32-ops); the host
pass prints a harmless "not a recognized feature" warning for it.
``--isa DIR`` also keeps the device assembly there for inspection.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfa_fwd.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["fa_fwd_kernel.hip", "fa_bwd_kernel.hip", "fa_api.cpp"]
ARCH = "gfx950"

DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-fno-honor-nans"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"),
                 "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build)")


def build(isa_dir: str | None = None, verbose: bool = False) -> str:
    """Compile every source into LIB_PATH; return the path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
           "-shared", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}",
           f"-I{CSRC}", *DEVICE_FLAGS]
    if isa_dir:
        os.makedirs(isa_dir, exist_ok=True)
        cmd += ["-save-temps"]
    cmd += [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=isa_dir or PKG, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--isa", default=None, help="keep device assembly here")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.isa, a.verbose))


if __name__ == "__main__":
    main()
