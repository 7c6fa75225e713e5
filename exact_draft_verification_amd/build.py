"""Build libspecverify.so (HIP, gfx950) in the package directory.

Usage: ``python -m exact_draft_verification_amd.build``.  The library is built
in-tree so that it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspecverify.so")
SOURCES = ["api.hip", "chain.hip", "tree.hip", "outcome.hip", "treebuild.hip", "treestoch.hip"]
ARCH = os.environ.get("SPEC_VERIFY_ARCH", "gfx950")

# All device code is compiled without packed-fp32 instructions (the compiler
# would otherwise fuse float pairs into them).
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every HIP source into ``libspecverify.so`` (always rebuilds)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", tmp,
           *[os.path.join(CSRC, s) for s in SOURCES]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
