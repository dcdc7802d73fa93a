"""Build ``libqknorm.so`` (the HIP library) in-tree for gfx950.

``python -m layerwise_qk_norm_amd.build`` compiles it; ``build_library()`` is
what ``__graft_entry__.build()`` calls. Compilation always runs (it is the
"does it build" check); a failed compile raises.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqknorm.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_cmd(out: str, extra=()) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 (v_pk_*_f32) instructions stay off in all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        *extra,
        "-o", out, os.path.join(CSRC, "qknorm.hip"),
    ]


def build_library(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = compile_cmd(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the device-only feature flag; drop that notice
    log = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{log}")
    if verbose and log.strip():
        print(log)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
