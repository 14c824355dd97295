"""Build libmfa.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m masked_flash_attention_amd.build  [--jobs N] [--debug]

Every source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled, then linked into masked_flash_attention_amd/libmfa.so.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmfa.so")
SOURCES = ["api.cpp", "maskrep.hip", "attn_fwd.hip", "attn_bwd.hip"]

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}", "-fPIC", "-std=c++17", "-O3",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
]
# Extra flags per source. attn_bwd.hip: the dK/dV pass at D = 128 holds its
# dK and dV accumulators (128 registers) beside about 250 other live values,
# one wave per SIMD. With the backend's default AGPR form for every MFMA, the
# S and dP results also landed in AGPRs and were copied to VGPRs for the
# softmax, with dK/dV blocks shuttled back and forth: about 450 accumulator
# moves per 64-query step. The VGPR form leaves the choice to the register
# allocator, which keeps S and dP in VGPRs (about 100 moves left; dK/dV pass
# 5.72 -> 5.41 ms on causal N=8192, identical code otherwise).
EXTRA = {"attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def flags_for(src):
    """hipcc flags of one source (gfx950, no packed fp32, plus its extras)."""
    return COMMON + EXTRA.get(src, [])


def flag_signature(src):
    """The flags of one source without the include paths (which depend on
    where the tree lies): what code generation depends on."""
    out, skip = [], False
    for f in flags_for(src):
        if skip:
            skip = False
        elif f == "-I":
            skip = True
        else:
            out.append(f)
    return " ".join(out)


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmfa)")


def _backend_option_ok(opt):
    """Whether this compiler's backend accepts `-mllvm opt` (such options
    come and go between LLVM versions)."""
    probe = os.path.join(BUILD, "_probe.hip")
    with open(probe, "w") as fh:
        fh.write("__global__ void k() {}\n")
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "--offload-device-only", "-mllvm", opt, "-x", "hip", "-c",
                        probe, "-o", probe + ".o"], capture_output=True, text=True)
    return r.returncode == 0


def _usable_flags(src):
    """flags_for(src), less any backend option the compiler rejects (the
    build then proceeds without that tuning, and says so)."""
    flags, out, i = flags_for(src), [], 0
    while i < len(flags):
        if flags[i] == "-mllvm" and i + 1 < len(flags):
            if _backend_option_ok(flags[i + 1]):
                out += flags[i:i + 2]
            else:
                print(f"warning: hipcc rejects -mllvm {flags[i + 1]}; building {src} without it", file=sys.stderr)
            i += 2
        else:
            out.append(flags[i])
            i += 1
    return out


def _compile(src, debug):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + _usable_flags(src) + (["-g"] if debug else []) + ["-x", "hip", "-c", os.path.join(CSRC, src),
                                                                         "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs=None, debug=False, verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    jobs = jobs or min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, debug), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libmfa.so failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True).stdout
    missing = [ln.split()[-1] for ln in nm.splitlines() if "__device_stub__" in ln]
    if missing:
        raise RuntimeError(f"libmfa.so has undefined kernel stubs (kernel templates dropped by the host pass): "
                           f"{missing[:3]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--debug", action="store_true")
    a = ap.parse_args()
    try:
        build(a.jobs, a.debug)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
