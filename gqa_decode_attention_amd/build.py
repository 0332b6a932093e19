"""Build the HIP library libgqa_decode.so in-tree for gfx950.

Usage: ``python -m gqa_decode_attention_amd.build`` (or ``build()`` from
Python).  Every call recompiles all sources; objects go to ``_build/`` at the
repository root and the library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libgqa_decode.so")

# Every C++ and HIP source of csrc/ goes into the one library.
SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith((".cpp", ".hip")))

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions are turned off for the device code; the host pass
# warns that it does not know the feature, which is harmless.
# Matrix-core results are kept in ordinary VGPRs (not accumulation registers):
# the online softmax rescales the V-sum accumulators on the vector ALU, which
# with accumulation registers costs a copy out and back in on every tile.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form=1", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall",
          "-Wno-unused-function"]
# Per-file flags.  The matrix-core kernels never have a NaN among their
# operands (stale rows are never loaded; masked scores are -inf), so their
# maxima need no NaN-quieting copies: without them the large-group kernel's
# score maxima take a third of the maximum instructions of each tile.
EXTRA = {"kernels_mfma.hip": ["-fno-honor-nans"], "kernels_mfma_qkv.hip": ["-fno-honor-nans"]}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in r.stderr.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([HIPCC, *COMMON, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(len(cmds), 8)) as ex:
        for err in ex.map(_run, cmds):
            if verbose and err.strip():
                print(err, file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
