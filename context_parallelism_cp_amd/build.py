"""Build libcpattn.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m context_parallelism_cp_amd.build [--resource-usage]

Objects go to ``context_parallelism_cp_amd/_build/``; the library lands next
to this file so that it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcpattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["cp_api.cpp", "attn_bf16.hip", "attn_f32.hip", "lse_merge.hip", "repack.hip",
           "bwd_f32.hip", "bwd_bf16.hip", "scratch.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per-source device-compiler options.  The attention kernel keeps its MFMA
# accumulators in VGPRs: with AGPR accumulators every VALU touch of the
# output (the rescale) and of the scores costs v_accvgpr copies.
# The backward kernels read every S and dP accumulator with VALU too; in the
# dk/dv kernel the compiler then uses the accumulation registers as spill
# room for the long-lived dK/dV values instead (measured +3.6%).
SOURCE_FLAGS = {
    "attn_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "bwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, resource_usage: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, "-x", "hip", *FLAGS, *SOURCE_FLAGS.get(src, []),
           "-I", os.path.join(HERE, "..", "include"),
           "-c", os.path.join(CSRC, src), "-o", obj]
    if resource_usage and src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if resource_usage:
        sys.stdout.write("".join(line + "\n" for line in r.stderr.splitlines()
                                 if "remark" in line and src.split(".")[0] in line))
    return obj


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, resource_usage), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(resource_usage="--resource-usage" in sys.argv, verbose=True))
