"""Builds the CPU oracle (oracle/sagesla_oracle.c, oracle/w8a8_oracle.c) into
oracle/libsagesla_oracle.so with gcc.

Plain scalar C: -O2, no fast-math, no FMA contraction, no vector intrinsics.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "sagesla_oracle.c"), os.path.join(HERE, "w8a8_oracle.c")]
LIB = os.path.join(HERE, "libsagesla_oracle.so")


def build(force: bool = False) -> str:
    if not force and os.path.exists(LIB) and all(os.path.getmtime(LIB) >= os.path.getmtime(s) for s in SRCS):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-o", tmp, *SRCS, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--force" in sys.argv))
