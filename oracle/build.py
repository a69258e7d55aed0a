"""Build step for the CPU oracle (test infrastructure): one gcc call.

-O2 with -fno-fast-math and -ffp-contract=off keeps every float operation a
single IEEE binary32 operation (no FMA contraction, no flush-to-zero).
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "i8mp_oracle.c")
LIB_PATH = os.path.join(HERE, "libi8mp_oracle.so")


def build() -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
