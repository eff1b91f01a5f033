"""Build the CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain C, -O2, no fast-math, no intrinsics.  Usage: python oracle/build.py
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sq_oracle.c")
OUT = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, src: str = SRC, out: str = OUT) -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
           "-D_GNU_SOURCE", "-Wall", "-Wextra", "-o", out + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
