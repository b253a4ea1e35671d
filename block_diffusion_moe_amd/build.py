"""Build libbdmoe.so (HIP, gfx950) in-tree with hipcc.

    python -m block_diffusion_moe_amd.build

Compiles every csrc/*.hip into one shared library next to this file, and
csrc/calib/*.hip (the copy kernel that calibrates HBM traffic counters)
into a second one.  The
library links the HIP runtime by soname (libamdhip64.so.7), so inside a
process that has imported torch it binds to the runtime torch already
loaded: one runtime, one set of streams and device pointers.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libbdmoe.so")
CAL_LIB = os.path.join(HERE, "libbdmcal.so")   # counter-calibration copy kernel
ARCH = os.environ.get("BDM_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-result",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile the library to `out` (and the calibration library beside the
    default one).  `defines` are extra -D macros (kernel tuning knobs); the
    defaults are the tuned ones."""
    _compile(sources(), out, defines, verbose)
    if out == LIB:
        _compile(sorted(glob.glob(os.path.join(CSRC, "calib", "*.hip"))), CAL_LIB, (), verbose)
    return out


def _compile(srcs, out, defines, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], f"-I{INCLUDE}", f"-I{CSRC}", *srcs,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    with tempfile.TemporaryDirectory() as td:
        env = dict(os.environ, TMPDIR=td)
        r = subprocess.run(cmd, capture_output=True, text=True, env=env)
    errs = [ln for ln in (r.stderr or "").splitlines()
            if "packed-fp32-ops" not in ln or "error" in ln.lower()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs), file=sys.stderr)
    os.replace(tmp, out)


if __name__ == "__main__":
    print(build(verbose=True))
