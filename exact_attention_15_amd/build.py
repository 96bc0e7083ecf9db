"""Build libexattn.so (the HIP kernels and the C ABI) for gfx950, in-tree."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libexattn.so")
SOURCES = ["abi.hip", "mask.hip", "fwd.hip", "fwd8.hip", "bwd.hip", "decode.hip", "quant.hip"]
# The forward kernel relies on no NaN semantics (masked scores are -inf), so
# it drops IEEE NaN quieting: max/min then need no canonicalising moves.
# The backward kernels take every MFMA result in VGPRs: the score products
# are read by the VALU, and left to its heuristic the compiler put them in
# AGPRs and moved the dK/dV accumulators between the two register files
# every tile (hundreds of v_accvgpr copies per tile).
EXTRA = {"fwd.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"], "fwd8.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"],
         "bwd.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans", "-mllvm", "--amdgpu-mfma-vgpr-form=1"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I", os.path.join(ROOT, "include"),
    # Keep the compiler from forming packed fp32 VALU ops (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build() -> str:
    """Compile every source and link libexattn.so; always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
