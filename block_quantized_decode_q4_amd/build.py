"""Ahead-of-time build of libq4k.so for gfx950 with hipcc (in-tree).

    python -m block_quantized_decode_q4_amd.build

The library is compiled for gfx950 only.  Packed-FP32 instructions are
disabled (-packed-fp32-ops): the kernels are written for one f32 result per
lane and instruction.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libq4k.so")
SOURCES = [os.path.join(CSRC, "q4k_kernels.hip"), os.path.join(CSRC, "q4k_dpp.hip"),
           os.path.join(CSRC, "q4k_mfma.hip"), os.path.join(CSRC, "q4k_q8.hip"),
           os.path.join(CSRC, "q4k_q6k.hip"), os.path.join(CSRC, "q4k_f16.hip"),
           os.path.join(CSRC, "q4k_api.hip")]
HEADERS = [os.path.join(CSRC, "q4k_kernels.h"), os.path.join(CSRC, "q4k_device.h"),
           os.path.join(CSRC, "q4k_lines.h"), os.path.join(CSRC, "q4k_xrep.h"),
           os.path.join(os.path.dirname(PKG), "include", "q4k.h")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libq4k.so)")


def compile_flags() -> list[str]:
    return [
        "--offload-arch=" + ARCH,
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]


def build(verbose: bool = False) -> str:
    """Compile every source into a fresh libq4k.so (always rebuilds)."""
    objs = []
    procs = []
    cc = hipcc()
    for src in SOURCES:     # the sources compile in parallel
        obj = os.path.join(CSRC, os.path.splitext(os.path.basename(src))[0] + ".o")
        cmd = [cc] + compile_flags() + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), cmd))
        objs.append(obj)
    failed = [cmd for proc, cmd in procs if proc.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    for obj in objs:
        os.remove(obj)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
