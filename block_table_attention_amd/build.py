"""Build libpba.so for gfx950 with hipcc (in-tree, next to this file).

    python block_table_attention_amd/build.py [--asm]

(run as a script: importing the package would load the library first).

Every HIP source under csrc/ is compiled for gfx950 only.  Packed-FP32 VALU
instructions are disabled.  ``--asm`` also writes the gfx950 assembly of each
source to ``_build/`` for inspection.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpba.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["pba_api.hip", "kv_append.hip", "block_copy.hip", "paged_decode.hip", "tables.hip",
           "bundle.hip", "vkv.hip", "noalloc.hip", "plan.cpp"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # MFMA accumulators in arch VGPRs: the online-softmax rescale is VALU
         # work on them, and AGPR homes cost two copies per chunk.
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         # The decode kernel's leading scalar arguments (10 of them, 14 dwords,
         # the hardware maximum) arrive preloaded in SGPRs.
         "-mllvm", "-amdgpu-kernarg-preload-count=10",
         "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature.
    lines = [l for l in proc.stdout.splitlines()
             if "packed-fp32-ops' is not a recognized feature" not in l]
    if lines:
        print("\n".join(lines), file=sys.stderr)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}")


def build(asm: bool = False, verbose: bool = True) -> str:
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        _run([HIPCC, *FLAGS, "-c", path, "-o", obj])
        objs.append(obj)
        if asm and src.endswith(".hip"):
            _run([HIPCC, *FLAGS, "--cuda-device-only", "-S", path,
                  "-o", os.path.join(objdir, src.replace(".hip", ".s"))])
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(asm="--asm" in sys.argv)
