"""Compile the CPU oracle (test infrastructure) into oracle/liboracle_embedding_wgrad.so.

Plain gcc, no fast-math and no FP contraction, so every fp32 operation in the
oracle is one IEEE binary32 operation in the order the source writes it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "embedding_wgrad_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle_embedding_wgrad.so")

CFLAGS = [
    "-O2", "-std=c11", "-fPIC", "-shared",
    "-fno-fast-math", "-ffp-contract=off", "-fexcess-precision=standard",
    "-Wall", "-Wextra",
]


def build() -> str:
    tmp = LIBRARY + ".tmp"
    subprocess.run(["gcc", *CFLAGS, SOURCE, "-o", tmp], check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build())
