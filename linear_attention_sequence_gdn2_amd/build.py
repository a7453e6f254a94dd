"""Build libgdn2.so (HIP, gfx950) in-tree with hipcc.

Each translation unit is compiled to an object in parallel, then linked into
``linear_attention_sequence_gdn2_amd/libgdn2.so``.  ``python -m
linear_attention_sequence_gdn2_amd.build`` rebuilds it.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgdn2.so")
STAMPS_LIB = os.path.join(HERE, "libgdn2_stamps.so")
POISON_LIB = os.path.join(HERE, "libgdn2_poison.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["gdn2_api.cpp", "gdn2_bwd.hip", "gdn2_reverse.hip", "gdn2_step.hip", "gdn2_output.hip",
           "gdn2_sweep.hip", "gdn2_noalloc.cpp", "gdn2_probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# packed fp32 VALU ops are kept out of the generated code on purpose
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC, "-Wno-unused-result"]


def _compile(src: str, extra=(), tag="") -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + tag + ".o")
    cmd = [HIPCC] + FLAGS + list(extra) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), p.stderr[-8000:]))
    return obj


def build(verbose: bool = False, stamps: bool = False, poison: bool = False) -> str:
    """Build libgdn2.so; with stamps=True the instrumented libgdn2_stamps.so instead (-DGDN2_STAMPS:
    the forward's kernels record s_memtime at their phase boundaries, for per-phase MFMA use);
    with poison=True the debug libgdn2_poison.so (-DGDN2_LDS_POISON: every kernel first fills
    its LDS with NaN words, so that a read of LDS before its write changes the results)."""
    if stamps and poison:
        raise ValueError("one variant at a time")
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    extra, tag = (["-DGDN2_STAMPS"], ".stamps") if stamps else (["-DGDN2_LDS_POISON"], ".poison") if poison else ((), "")
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, extra, tag), SOURCES))
    lib = STAMPS_LIB if stamps else POISON_LIB if poison else LIB
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), p.stderr[-8000:]))
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True, stamps="--stamps" in sys.argv[1:], poison="--poison" in sys.argv[1:])
    sys.exit(0)
