"""Builds the oracle's C part (plain gcc, host only; test infrastructure)."""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kmeans.c")
LIB = os.path.join(HERE, "_kmeans_oracle.so")


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
                    SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
