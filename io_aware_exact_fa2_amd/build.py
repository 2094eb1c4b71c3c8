"""Build step for libfa.so: hipcc, gfx950 only, in-tree.

    python -m io_aware_exact_fa2_amd.build

compiles the HIP sources in csrc/ (each with the common options plus its own, in
parallel) and links them into io_aware_exact_fa2_amd/libfa.so. Packed fp32 VALU forms are
disabled for all device code (-packed-fp32-ops), and MFMA builtins use their
VGPR-accumulator form.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
# source -> options of its own. The slot-scheduled kernels (the forward's wide kernel and
# the backward's dK/dV and dQ kernels) unroll a ring of iterations, each of dozens of
# MFMA slots, past the default limit of forced unrolling (the ring slots must be
# compile-time offsets; a loop left rolled indexes register arrays at run time, through
# scratch memory). The d = 128 backward uses LLVM's iterative ILP machine
# scheduler: its 32-key dK/dV kernel (taken at a zero scale; one wave per SIMD, more than
# 256 registers) then issues LDS operand reads further ahead of their products (measured
# +6 to +12% on that backward); the d = 64 backward measured 3% slower with it, and the
# forward sources and the slot-scheduled backward kernels order their loops explicitly.
SOURCES = {
    "fa_fwd.hip": ["-mllvm", "-pragma-unroll-threshold=200000"],
    "fa_bwd.hip": [],
    "fa_bwd_d64.hip": ["-mllvm", "-pragma-unroll-threshold=200000"],
    "fa_bwd_d128.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp",
                        "-mllvm", "-pragma-unroll-threshold=200000"],
}
SRCS = [os.path.join(PKG, "csrc", f) for f in SOURCES]
OUT = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
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


# The compiler's per-kernel resource remarks, so that a spill of a slot-scheduled kernel
# (one whose name holds "wide") fails the build instead of running through scratch memory
RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"


def _messages(res) -> list:
    # the host pass does not know the device-only feature; that warning is harmless
    return [l for l in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in l and l.strip() and "kernel-resource-usage" not in l
            and not l.startswith("In file included from")
            and not l.lstrip().startswith(("|", "^")) and not l.strip()[0].isdigit()]


def resource_usage(text: str) -> dict:
    """Kernel name -> {remark key: value} from the compiler's resource remarks."""
    usage, name = {}, None
    for line in text.splitlines():
        if "kernel-resource-usage" not in line or "remark:" not in line:
            continue
        body = line.split("remark:", 1)[1].split("[-Rpass", 1)[0].strip()
        key, _, val = body.partition(":")
        if key == "Function Name":
            name = val.strip()
            usage[name] = {}
        elif name is not None:
            usage[name][key.strip()] = val.strip()
    return usage


def check_no_spills(usage: dict) -> None:
    bad = [f"{n}: scratch {u.get('ScratchSize [bytes/lane]')} bytes/lane"
           for n, u in usage.items()
           if "wide" in n and u.get("ScratchSize [bytes/lane]", "0") != "0"]
    if bad:
        raise RuntimeError("slot-scheduled kernels spill to scratch memory:\n" + "\n".join(bad))


def build_library(extra_flags=(), out: str = OUT, verbose: bool = False) -> str:
    """Compile the C-ABI library; returns its path. Always recompiles."""
    tmp = out + ".tmp"
    msgs = []
    with tempfile.TemporaryDirectory(prefix="fa355_build_") as objdir:
        procs, objs = [], []
        for name, own in SOURCES.items():
            obj = os.path.join(objdir, name + ".o")
            cmd = [hipcc(), *HIPCC_FLAGS, *own, *extra_flags, RESOURCE_REMARKS,
                   "-I", os.path.join(ROOT, "include"), "-c", os.path.join(PKG, "csrc", name),
                   "-o", obj]
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
        failed = None
        usage = {}
        for cmd, proc in procs:
            out_s, err_s = proc.communicate()
            res = subprocess.CompletedProcess(cmd, proc.returncode, out_s, err_s)
            msgs += _messages(res)
            usage.update(resource_usage(out_s + err_s))
            if res.returncode != 0 and failed is None:
                failed = (cmd, _messages(res))
        if failed is not None:
            raise RuntimeError("hipcc failed:\n" + " ".join(failed[0]) + "\n" + "\n".join(failed[1]))
        check_no_spills(usage)
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        msgs += _messages(res)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + " ".join(cmd) + "\n" + "\n".join(_messages(res)))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
