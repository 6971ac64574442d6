"""Build the CPU oracle library (test infrastructure only).

gcc, C11, OpenMP, -ffp-contract=off so that no multiply-add is fused unless
the source calls fmaf() explicitly.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libcsk_oracle.so")


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB):
        return LIB
    src = os.path.join(HERE, "csk_oracle.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=gnu11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
