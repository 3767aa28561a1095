"""Build the gfx950 attention library: libattn_mi355x.so next to this file.

Offline, in-tree, with hipcc only:  python -m exact_attention_attn_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libattn_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["attn_fwd.hip", "attn_bwd.hip", "attn_decode.hip", "attn_noalloc.hip", "attn_api.cpp"]
# Per-source code-generation options.  The forward kernel keeps its MFMA
# accumulators in architectural VGPRs: the softmax rescales them with VALU
# instructions, and accumulators in AGPRs would be copied back and forth
# around that (rarely taken) branch on every tile.
# The forward is also built without NaN semantics: its inputs are finite
# (infinities are still honoured: masked scores are -inf), and maxnum then
# needs no canonicalising copies of its operands in the per-tile row maximum.
SOURCE_FLAGS = {"attn_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
                "attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"

# Packed fp32 VALU instructions are kept out of the code object.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build the library")
    return path


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source for gfx950 and link the shared library; return its path."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = [cc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-c",
               "-I", INCLUDE, "-I", CSRC, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), *extra_flags,
               os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
