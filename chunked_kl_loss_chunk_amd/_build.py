"""Build the HIP library ``libkdkl.so`` in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libkdkl.so")
CLIENT_SRC = os.path.join(PKG, "examples", "abi_client.cpp")
CLIENT_PATH = os.path.join(PKG, "examples", "abi_client")
SOURCES = ["kd_fused_kl.hip", "kd_plan.cpp"]
HEADERS = ["kd_gemm.h", "kd_plan.h"]


def hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def compile_cmd(out: str, extra=()) -> list:
    return [
        hipcc(),
        "--offload-arch=gfx950",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        # packed fp32 VALU ops are kept out of the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
        *[os.path.join(CSRC, s) for s in SOURCES],
        *extra,
        "-o", out,
    ]


def build(verbose: bool = False) -> str:
    """Compile every source into libkdkl.so next to this file. Returns its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = compile_cmd(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    # A C++ caller of the ABI alone (no Python), built by the host compiler
    # and linked against the library and the HIP runtime.
    tmp = CLIENT_PATH + ".tmp"
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = [shutil.which("g++") or "g++", "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__",
           "-I", INCLUDE, "-I", os.path.join(rocm, "include"), CLIENT_SRC, "-o", tmp,
           "-L", PKG, "-lkdkl", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/..", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, CLIENT_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
