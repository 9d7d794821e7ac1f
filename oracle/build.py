"""Compile the CPU oracle (``oracle.c``) into ``libropequant_oracle.so``.

Test infrastructure: the oracle is a plain single-threaded C definition of the
hot path.  It is compiled with ``-ffp-contract=off`` and without any ``-march``
or fast-math flag, so every float operation is one IEEE-754 binary32 basic
operation (x86-64 SSE2) with no fused multiply-add.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "libropequant_oracle.so")

CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fno-math-errno", "-Wall", "-Wextra", "-Werror"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
