"""Builds libfa.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: ``python -m exact_io_aware_55_amd.build`` or ``build_library()``.
Each ``csrc/*.hip`` is compiled with hipcc into ``_build/`` and linked into
``exact_io_aware_55_amd/libfa.so``.  Packed fp32 instructions are disabled
(``-packed-fp32-ops``) and fp32 atomics use the hardware instruction.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function", "-Wno-inline-asm",
]


# Per-source extra flags.  The kernels keep their score tiles in VGPRs:
# without this flag the compiler would put every MFMA result in AGPRs once
# any accumulator lives there, and copy the tiles back for the softmax.  The
# long-lived d = 128 dK/dV accumulators are placed in AGPRs explicitly.
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA = {"fa_bwd.hip": _VGPR_FORM, "fa_calib.hip": _VGPR_FORM}


# The synchronisation check build: the same sources with -DFA_DEBUG_SYNC,
# which makes every pipelined kernel wait for all memory operations and meet
# at a barrier at each block or step and before each LDS ring refill.  Its
# outputs must equal libfa.so's bit for bit (a GPU test compares them).
SYNC_LIB = os.path.join(PKG, "libfa_sync.so")
VARIANTS = {LIB: ("", []), SYNC_LIB: ("sync", ["-DFA_DEBUG_SYNC"])}


def _compile(job) -> str:
    src, sub, defines = job
    out_dir = os.path.join(BUILD, sub) if sub else BUILD
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    extra = EXTRA.get(os.path.basename(src), [])
    cmd = [HIPCC, *FLAGS, *extra, *defines, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)


def build_library(verbose: bool = False) -> str:
    """Compile every csrc/*.hip and link libfa.so and the synchronisation
    check build libfa_sync.so; returns the path of libfa.so."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = []
    for lib, (sub, defines) in VARIANTS.items():
        os.makedirs(os.path.join(BUILD, sub) if sub else BUILD, exist_ok=True)
        jobs += [(src, sub, defines) for src in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(_compile, jobs))
    for n, lib in enumerate(VARIANTS):
        _link(objs[n * len(srcs):(n + 1) * len(srcs)], lib)
        if verbose:
            print(f"built {lib} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
