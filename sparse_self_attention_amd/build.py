"""Builds libtra.so (the C-ABI library of the Token Radius Attention hot path)
in-tree for gfx950 with hipcc.

usage: python -m sparse_self_attention_amd.build
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libtra.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("tra_api.cpp", "tra_kernels.hip", "tra_dense.hip", "tra_noalloc.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("TRA_OFFLOAD_ARCH", "gfx950")
ROCM_LIB = "/opt/rocm/lib"


def command(out=LIB):
    return [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # packed fp32 VALU forms are kept out of every kernel
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
            "-o", out] + SOURCES + [
            # profiler ranges around the plan stages and calls (rocprofv3 --marker-trace)
            "-L", ROCM_LIB, "-Wl,-rpath," + ROCM_LIB, "-lrocprofiler-sdk-roctx"]


SANITIZE_FLAGS = [
    # host code only: the device code is built as usual
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g",
]


def build_sanitized(out, verbose=True):
    """libtra with its host code built under AddressSanitizer and
    UndefinedBehaviorSanitizer (for host-only checks on a machine without a
    GPU; the executable that loads it must be linked with -fsanitize too)."""
    cmd = command(out)
    cmd = cmd[:1] + SANITIZE_FLAGS + cmd[1:]
    cmd = [c if c != "-O3" else "-O1" for c in cmd]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building the sanitized library")
    return out


def build(verbose=True):
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libtra.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
