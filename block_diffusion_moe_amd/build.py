"""Build libbdmoe.so (HIP, gfx950) in-tree with hipcc.

    python -m block_diffusion_moe_amd.build

Compiles every csrc/*.hip into one shared library next to this file, the
same sources with device-side bounds checks (BDM_DEBUG_BOUNDS=1) into
libbdmoe_debug.so, and csrc/calib/*.hip (the copy kernel that calibrates
HBM traffic counters) into a third one.  The
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
DEBUG_LIB = os.path.join(HERE, "libbdmoe_debug.so")   # bounds-checked build
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
    """Compile the library to `out` (and, beside the default one, the
    bounds-checked debug library and the calibration library; the three
    compiles run side by side).  `defines` are extra -D macros (kernel tuning
    knobs); the defaults are the tuned ones."""
    jobs = [(sources(), out, tuple(defines))]
    if out == LIB:
        jobs.append((sources(), DEBUG_LIB, ("BDM_DEBUG_BOUNDS=1",)))
        jobs.append((sorted(glob.glob(os.path.join(CSRC, "calib", "*.hip"))), CAL_LIB, ()))
    with tempfile.TemporaryDirectory() as td:
        procs = [_start(srcs, o, d, verbose, td) for srcs, o, d in jobs]
        errors = [e for e in (_finish(p, verbose) for p in procs) if e]
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
    return out


def _start(srcs, out, defines, verbose, tmpdir):
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], f"-I{INCLUDE}", f"-I{CSRC}", *srcs,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    env = dict(os.environ, TMPDIR=tmpdir)
    proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                            env=env)
    return proc, tmp, out


def _finish(job, verbose):
    proc, tmp, out = job
    _, err = proc.communicate()
    errs = [ln for ln in (err or "").splitlines()
            if "packed-fp32-ops" not in ln or "error" in ln.lower()]
    if proc.returncode != 0:
        return f"{out}:\n" + "\n".join(errs)
    if verbose and errs:
        print("\n".join(errs), file=sys.stderr)
    os.replace(tmp, out)
    return ""


if __name__ == "__main__":
    print(build(verbose=True))
