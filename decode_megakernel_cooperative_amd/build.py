"""Builds the decode library (libamk.so) in-tree with hipcc for gfx950.

    python -m decode_megakernel_cooperative_amd.build

The kernel is compiled with packed-fp32 instructions disabled; the host quantizer is
compiled without fast-math so its divisions and round-half-even stay IEEE.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libamk.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd[:3])} ...")
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    common = ["-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}"]
    kobjs = []
    for src in ("amk_decode.hip",):
        kobj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        _run([cc, f"--offload-arch={ARCH}", "-O3", *common,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-c", os.path.join(CSRC, src), "-o", kobj], verbose)
        kobjs.append(kobj)
    hobj = os.path.join(BUILD_DIR, "amk_host.o")
    _run([cc, "-x", "c++", "-O2", "-fno-fast-math", "-ffp-contract=off", "-D__HIP_PLATFORM_AMD__",
          "-I/opt/rocm/include", *common,
          "-c", os.path.join(CSRC, "amk_host.cpp"), "-o", hobj], verbose)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *kobjs, hobj, "-o", tmp, "-lpthread"], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
