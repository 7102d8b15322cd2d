"""Builds libmoe_mxfp4.so (HIP, gfx950) and the host-only synth library in-tree.

hipcc cross-compiles for gfx950 without a GPU, so this runs on any host with
ROCm.  Packed fp32 VALU instructions are switched off for all device code.
"""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libmoe_mxfp4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# host-only sanitizers for the checking build: each -fsanitize= applies to the host pass alone
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-shared-libsan", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LIB_PATH = os.path.join(LIB_DIR, "libmoe_mxfp4_san.so")


def build_library(verbose: bool = False, sanitize: bool = False) -> str:
    """hipcc build of every csrc/*.hip into lib/libmoe_mxfp4.so.  sanitize=True
    builds lib/libmoe_mxfp4_san.so with AddressSanitizer and UBSan on the
    host code (argument validation, launch set-up); device code is the same."""
    os.makedirs(LIB_DIR, exist_ok=True)
    path = SAN_LIB_PATH if sanitize else LIB_PATH
    tmp = path + ".tmp"
    cmd = [HIPCC] + HIP_FLAGS + (HOST_SANITIZE if sanitize else []) + ["-I", os.path.join(ROOT, "include")] + \
        sources() + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, path)
    return path


def build_all(verbose: bool = False) -> None:
    from . import synth

    synth.build(verbose)
    build_library(verbose)


if __name__ == "__main__":
    build_all(verbose=True)
