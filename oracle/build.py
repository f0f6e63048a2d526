"""Compile the CPU oracle (plain C, gcc) into oracle/liboracle.so.

The oracle is test infrastructure: only the tests, the package smoke check and
the benchmark's CPU-baseline leg load it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "spmm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off: no multiply-add fusion unless the code calls fmaf itself.
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared",
          "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB, extra=()) -> str:
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
