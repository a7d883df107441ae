"""Build the library in-tree with hipcc for gfx950 (one shared object, all
kernels): libdflash.so, and libdflash_checked.so, the same sources with the
device-data precondition checks compiled in (DFLASH_DEVICE_CHECKS=1)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdflash.so")
LIB_CHECKED = os.path.join(HERE, "libdflash_checked.so")
SOURCES = ["block_attn.hip", "vocab_rows.hip", "context_fuse.hip", "select_path.hip", "two_tap_conv.hip",
           "lm_head.hip", "top_p.hip", "noalloc.hip", "checks.hip",
           "status.cpp"]
CHECKED_FLAGS = ["-DDFLASH_DEVICE_CHECKS=1"]

# Device code generation: no packed-fp32 instructions anywhere (the host pass
# of hipcc prints a harmless "not a recognized feature" warning for this flag),
# and MFMA results in ordinary VGPRs rather than AGPRs, which keeps the
# attention kernel's softmax (vector ALU work on the MFMA results) free of
# register-class copies.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", *DEVICE_FLAGS,
         "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def build(verbose: bool = False) -> str:
    """Compile both libraries (two hipcc processes at once); returns libdflash.so."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    jobs = []
    for out, extra in ((LIB, []), (LIB_CHECKED, CHECKED_FLAGS)):
        cmd = [hipcc, *FLAGS, *extra, *srcs, "-o", out + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    failed = []
    for out, proc in jobs:
        _, stderr = proc.communicate()
        errs = "\n".join(l for l in (stderr or "").splitlines() if "packed-fp32-ops" not in l)
        if proc.returncode != 0:
            failed.append(f"{os.path.basename(out)}: hipcc failed ({proc.returncode}):\n{errs}")
        elif verbose and errs.strip():
            print(errs, file=sys.stderr)
    if failed:
        raise RuntimeError("\n".join(failed))
    for out, _ in jobs:
        os.replace(out + ".tmp", out)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
