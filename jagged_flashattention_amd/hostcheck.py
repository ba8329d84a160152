"""Host-check build of the library: the planner and the C ABI's argument
validation (plan.cpp, api.cpp) compiled with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, the kernel launchers replaced by stubs that
report that no kernel is available (csrc/hostcheck_stubs.cpp). No device
code is built. Load it with JFA_LIBRARY=<path> and the ASan runtime preloaded.

Usage: python -m jagged_flashattention_amd.hostcheck
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(BUILD, "libjfa_hostcheck.so")
SOURCES = ["plan.cpp", "api.cpp", "hostcheck_stubs.cpp"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SANITIZE = ["-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer"]


def available() -> bool:
    return shutil.which("g++") is not None and os.path.exists(
        os.path.join(ROCM, "include", "hip", "hip_runtime_api.h"))


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", *SANITIZE,
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(os.path.dirname(PKG), "include"),
           *[os.path.join(CSRC, s) for s in SOURCES],
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("host-check build failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
