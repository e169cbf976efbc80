"""Compile the fp64 CPU oracle (test infrastructure) with gcc.

IEEE fp64 with no fast-math and no FMA contraction, so the summation order
written in ssd_oracle.c is the order executed.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ssd_oracle.c")
LIB = os.path.join(HERE, "libssd_oracle.so")


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
