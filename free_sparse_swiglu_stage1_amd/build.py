"""Builds libprox.so (the HIP library behind include/prox.h) for gfx950.

    python -m free_sparse_swiglu_stage1_amd.build

Compiles every .hip source under csrc/ with hipcc into one shared library
next to this file.  Always recompiles (the build is a few seconds per file).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libprox.so")

ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # IEEE-correct fp32 division and square root (the quantizer's scale and
    # codes must round exactly like binary32 division)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-ffp-contract=fast",
    # no packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the Prox HIP library)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


LIB_SAN = os.path.join(HERE, "libprox_san.so")

# The host code (argument checks, workspace layout, launch sequence) under
# AddressSanitizer and UndefinedBehaviorSanitizer; the GPU code is built as
# usual.  Each sanitizer flag applies to the host pass only.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-g"]


def build(verbose: bool = False, extra_flags=None, sanitize: bool = False) -> str:
    out = LIB_SAN if sanitize else LIB
    tmp = out + ".tmp%d" % os.getpid()
    flags = HIPCC_FLAGS + (SANITIZE_FLAGS if sanitize else [])
    cmd = [hipcc()] + flags + list(extra_flags or []) + ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
                                                         "-o", tmp] + sources()
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + r.stdout)
    if verbose and r.stdout.strip():
        print(r.stdout)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
