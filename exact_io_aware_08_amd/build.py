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
SOURCES = ["fa_fwd_kernel.hip", "fa_fp8_kernel.hip", "fa_bwd_kernel.hip", "fa_noalloc.hip",
           "fa_api.cpp"]
ARCH = "gfx950"

DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-fno-honor-nans"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"),
                 "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build)")


# Per-file device flags.  The backward kernels keep their MFMA accumulators
# in the VGPR form of the instructions (the register allocator then puts the
# long-lived dK/dV accumulators in AGPRs without copying them back and forth
# every loop trip); the forward kernels are faster with the default.
FILE_FLAGS = {"fa_bwd_kernel.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def build(isa_dir: str | None = None, verbose: bool = False, csrc: str = CSRC,
          out: str = LIB_PATH, extra_flags=()) -> str:
    """Compile every source (one object each, in parallel) and link them
    into ``out``; return the path."""
    import tempfile
    base = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{csrc}",
            *DEVICE_FLAGS, *extra_flags]
    if isa_dir:
        os.makedirs(isa_dir, exist_ok=True)
        base += ["-save-temps"]
    noise = "is not a recognized feature for this target"

    def run(cmds, cwd):
        procs = [(c, subprocess.Popen(c, cwd=cwd, stdout=subprocess.PIPE,
                                      stderr=subprocess.PIPE, text=True)) for c in cmds]
        for c, pr in procs:
            _, stderr = pr.communicate()
            err = "\n".join(l for l in stderr.splitlines() if noise not in l)
            if verbose:
                print(" ".join(c), flush=True)
            if pr.returncode != 0:
                raise RuntimeError(f"hipcc failed ({pr.returncode}):\n{err}")
            if err.strip() and verbose:
                print(err, file=sys.stderr)

    with tempfile.TemporaryDirectory() as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        run([base + FILE_FLAGS.get(s, []) + ["-c", os.path.join(csrc, s), "-o", o]
             for s, o in zip(SOURCES, objs)], isa_dir or tmpdir)
        tmp = out + ".tmp"
        # -z defs: a kernel whose host pass failed leaves its launch stub
        # undefined, which must stop the build rather than the first load
        run([[hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", *objs,
              "-o", tmp]], tmpdir)
        os.replace(tmp, out)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--isa", default=None, help="keep device assembly here")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.isa, a.verbose))


if __name__ == "__main__":
    main()
