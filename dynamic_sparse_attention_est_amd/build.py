"""Builds libmsattn.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Every .hip file under csrc/ is compiled by hipcc into _build/ and linked into
dynamic_sparse_attention_est_amd/libmsattn.so.  Run as a script or call
build_library().
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmsattn.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
    f"-I{CSRC}",
    # Packed fp32 VALU forms stay off (hipcc would otherwise emit them from plain float code).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: keeps the attention kernel's working set in
    # one register file (no AGPR round trips) at two waves per SIMD.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]
# Per-file additions.  The attention kernel never produces NaN (masked logits
# are -inf, exp2(-inf) = 0, and every -inf - -inf is guarded), so its max
# reductions may skip the NaN-quieting copies of their operands.
FILE_FLAGS = {
    "sparse_attn.hip": ["-fno-honor-nans"],
    "group_attn.hip": ["-fno-honor-nans"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
