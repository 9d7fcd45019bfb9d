"""Build libmoe_w8a8.so (HIP, gfx950) in-tree with hipcc.

    python -m w8a8_int8_expert_amd.build

Every source under csrc/ is compiled to an object under _build/ (in parallel)
and linked into w8a8_int8_expert_amd/libmoe_w8a8.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_w8a8.so")
ARCH = os.environ.get("MOE_W8A8_ARCH", "gfx950")


def _hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
              shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libmoe_w8a8.so)")


def compile_flags() -> list:
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            # quantisation decisions must round every product to fp32
            "-ffp-contract=off",
            # packed fp32 arithmetic stays off on this target
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose: bool = False, jobs: int = 8) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    flags = compile_flags()

    def one(src):
        obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
        cmd = [hipcc, "-c", src, "-o", obj] + flags
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(one, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, "-shared", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
