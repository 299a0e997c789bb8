"""Build libembedding_wgrad.so (HIP, gfx950) in place, next to this file.

    python sparse_embedding_weight_amd/build.py
"""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

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
    # atomics stay as written: the optimizer's rewrite of a uniform-address
    # atomic reads its result back at once, which makes a wave wait for every
    # load it has in flight, and its per-wave reductions cost more than the
    # LDS atomics they replace here
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel (each holds its own kernels
    and their launchers), then link the shared library."""
    tmp = LIBRARY + ".tmp"
    compile_flags = [f for f in FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory() as objdir:
        cmds = [[HIPCC, *compile_flags, "-c", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                 os.path.join(CSRC, s), "-o", os.path.join(objdir, s + ".o")] for s in SOURCES]
        if verbose:
            for c in cmds:
                print(" ".join(c), file=sys.stderr)
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as pool:
            for r in pool.map(lambda c: subprocess.run(c), cmds):
                if r.returncode != 0:
                    raise subprocess.CalledProcessError(r.returncode, r.args)
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                *[os.path.join(objdir, s + ".o") for s in SOURCES], "-o", tmp]
        if verbose:
            print(" ".join(link), file=sys.stderr)
        subprocess.run(link, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
