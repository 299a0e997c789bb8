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


CHECKED_LIBRARY = os.path.join(HERE, "libembedding_wgrad_checked.so")


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel (each holds its own kernels
    and their launchers), then link the shared library; the same again with
    the device-side bounds checks compiled in (-DEWG_DEVICE_CHECKS=1), as
    libembedding_wgrad_checked.so, for the GPU test of those checks."""
    variants = [(LIBRARY, []), (CHECKED_LIBRARY, ["-DEWG_DEVICE_CHECKS=1"])]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory() as objdir:
        def obj(v, s):
            return os.path.join(objdir, f"{v}_{s}.o")
        cmds = [[HIPCC, *compile_flags, *extra, "-c", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                 os.path.join(CSRC, s), "-o", obj(v, s)]
                for v, (_, extra) in enumerate(variants) for s in SOURCES]
        if verbose:
            for c in cmds:
                print(" ".join(c), file=sys.stderr)
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as pool:
            for r in pool.map(lambda c: subprocess.run(c), cmds):
                if r.returncode != 0:
                    raise subprocess.CalledProcessError(r.returncode, r.args)
        for v, (path, _) in enumerate(variants):
            tmp = path + ".tmp"
            link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                    *[obj(v, s) for s in SOURCES], "-o", tmp]
            if verbose:
                print(" ".join(link), file=sys.stderr)
            subprocess.run(link, check=True)
            os.replace(tmp, path)
    return LIBRARY


HOST_ASAN_LIBRARY = os.path.join(HERE, "libembedding_wgrad_hostasan.so")


def build_host_asan(verbose: bool = False) -> str:
    """The same library with its host code under AddressSanitizer (device code
    as usual, at -O1), for a CPU test of the host entry points: argument
    checks, workspace sizes, predicates and status text. Load it with the
    sanitizer runtime preloaded (asan_runtime())."""
    tmp = HOST_ASAN_LIBRARY + ".tmp"
    flags = [f for f in FLAGS if f not in ("-O3", "-shared")]
    with tempfile.TemporaryDirectory() as objdir:
        cmds = [[HIPCC, *flags, "-O1", "-g", "-Xarch_host", "-fsanitize=address",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-c", "-I", os.path.join(ROOT, "include"),
                 "-I", CSRC, os.path.join(CSRC, s), "-o", os.path.join(objdir, s + ".o")]
                for s in SOURCES]
        if verbose:
            for c in cmds:
                print(" ".join(c), file=sys.stderr)
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as pool:
            for r in pool.map(lambda c: subprocess.run(c), cmds):
                if r.returncode != 0:
                    raise subprocess.CalledProcessError(r.returncode, r.args)
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                "-shared-libsan", *[os.path.join(objdir, s + ".o") for s in SOURCES], "-o", tmp]
        subprocess.run(link, check=True)
    os.replace(tmp, HOST_ASAN_LIBRARY)
    return HOST_ASAN_LIBRARY


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime ('' if absent)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang")
    try:
        out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                             capture_output=True, text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return ""
    return out if os.path.isabs(out) and os.path.exists(out) else ""


if __name__ == "__main__":
    print(build(verbose=True))
