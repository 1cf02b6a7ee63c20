"""Build libbsa.so for gfx950 with hipcc (in-tree, no JIT cache).

Usage: python -m block_sparse_attention_27_amd.build  (or call build()).
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbsa.so")
SOURCES = ["bsa_api.hip", "score.hip", "ibcs.hip", "select.hip", "permute.hip", "attend_bf16_d128.hip",
           "attend_bf16_d64.hip", "attend_fp32.hip", "measure.hip"]

# Packed-fp32 instructions stay off (hipcc may otherwise form v_pk_* from float code).
HIPFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# The attention kernels never produce NaN on purpose (masked logits are -inf);
# dropping NaN canonicalisation lets row maxima use v_max3 directly.
UNIT_FLAGS = {"attend_bf16_d128.hip": ["-fno-honor-nans"], "attend_bf16_d64.hip": ["-fno-honor-nans"]}


def _hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def build(verbose: bool = False, jobs: int = 6) -> str:
    """Compile every source and link libbsa.so; returns the library path."""
    obj_dir = os.path.join(PKG, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    hipcc = _hipcc()

    def compile_one(src):
        obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
        cmd = [hipcc, *HIPFLAGS, *UNIT_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
