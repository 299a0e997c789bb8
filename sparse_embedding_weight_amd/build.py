"""Build libembedding_wgrad.so (HIP, gfx950) in place, next to this file.

    python sparse_embedding_weight_amd/build.py
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libembedding_wgrad.so")
SOURCES = ["api.hip", "sort_tokens.hip", "accumulate.hip", "many_tokens.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions (v_pk_add_f32 and friends)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32: keep denormals, no contraction, no reassociation
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off", "-fno-fast-math",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    tmp = LIBRARY + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
