"""Build step for libfa.so: hipcc, gfx950 only, in-tree.

    python -m io_aware_exact_fa2_amd.build

compiles csrc/fa_fwd.hip and csrc/fa_bwd.hip into io_aware_exact_fa2_amd/libfa.so. Packed fp32 VALU
forms are disabled for all device code (-packed-fp32-ops), and MFMA builtins use
their VGPR-accumulator form.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f) for f in ("fa_fwd.hip", "fa_bwd.hip")]
OUT = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA builtins accumulate in VGPRs (the wide kernel keeps its output
    # accumulators in AGPRs through inline assembly, and its S^T tiles, which the
    # VALU reads, in VGPRs; by default the compiler would put both in AGPRs once a
    # kernel may use more than 256 registers)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library needs ROCm's hipcc to build")


def build_library(extra_flags=(), out: str = OUT, verbose: bool = False) -> str:
    """Compile the C-ABI library; returns its path. Always recompiles."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"),
           *SRCS, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature; that warning is harmless
    msgs = [l for l in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in l and l.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
