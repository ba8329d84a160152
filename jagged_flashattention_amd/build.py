"""Build libjfa.so (HIP kernels for gfx950 + host planner/API) in-tree with hipcc,
and libjfa_debug.so, the same sources with the executed-tile log compiled in
(JFA_TILE_LOG; see jfa_debug_tile_log in include/jfa.h).

Usage: python -m jagged_flashattention_amd.build   (or __graft_entry__.build()).
Objects go to jagged_flashattention_amd/_build/, the libraries next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libjfa.so")
DEBUG_LIB = os.path.join(PKG, "libjfa_debug.so")
SOURCES = ["plan.cpp", "api.cpp", "noalloc.hip", "fwd.hip", "bwd.hip", "bwd_mx.hip", "dq.hip", "dq_mx.hip", "mx.hip"]
ARCH = "gfx950"

# Packed fp32 VALU ops are disabled for all device code (ordinary float code is
# still vectorised by the compiler into plain VALU instructions).
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(os.path.dirname(PKG), "include")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(job) -> str:
    src, outdir, defines = job
    obj = os.path.join(outdir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *defines, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)


def build(verbose: bool = False, debug: bool = True) -> str:
    """Build libjfa.so (and, with debug, libjfa_debug.so); returns the former."""
    variants = [(LIB, BUILD, [])]
    if debug:
        variants.append((DEBUG_LIB, os.path.join(BUILD, "debug"), ["-DJFA_TILE_LOG"]))
    jobs = []
    for _, outdir, defines in variants:
        os.makedirs(outdir, exist_ok=True)
        jobs += [(src, outdir, defines) for src in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, jobs))
    for i, (lib, _, _) in enumerate(variants):
        _link(objs[i * len(SOURCES):(i + 1) * len(SOURCES)], lib)
        if verbose:
            print("built", lib)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
