"""Build the HIP library (gfx950) and the CPU check library, in-tree.

    python -m bit_gemm_amd.build

produces bit_gemm_amd/libmosaicq.so (the C ABI of include/mosaicq.h) and
bit_gemm_amd/libmq_hostcheck.so (the packer's integer arithmetic built for
the host, used by CPU tests). Every call recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmosaicq.so")
HOSTCHECK = os.path.join(HERE, "libmq_hostcheck.so")
SOURCES = ["api.cpp", "pack.hip", "pack_blocks.hip", "gemv.hip", "gemm.hip", "gemm_mid.hip", "gemm_rw.hip", "residual.hip", "migrate.hip", "w4a4.hip", "probe.hip"]
# per-source code generation options: the prefill GEMM's stage body is one
# long basic block; the ILP-oriented machine scheduler interleaves its
# widening arithmetic with the MFMAs instead of clustering it after them
EXTRA: dict = {"gemm.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}
ARCH = os.environ.get("MQ_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
            # packed fp32 VALU forms are kept out of the device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {cmd[-1]}")
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc, "-x", "hip", *_flags(), *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(4, len(cmds))) as ex:
        list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    tmp = HOSTCHECK + ".tmp"
    _run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-fvisibility=hidden", "-I", CSRC,
          os.path.join(CSRC, "hostcheck.cpp"), "-o", tmp])
    os.replace(tmp, HOSTCHECK)
    if verbose:
        print(f"built {LIB} and {HOSTCHECK}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
