"""Compile libropequant (``csrc/ropequant.hip``) for gfx950 into this package.

    python -m rope_fp8_quant_amd.build

Flags: ``-ffp-contract=off`` keeps every multiply and add separately rounded
(no FMA contraction); ``-target-feature -packed-fp32-ops`` keeps the compiler
from emitting packed fp32 instructions; no fast-math flag is used, so fp32
divide and square root stay correctly rounded.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "ropequant.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libropequant.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def compile_hip(src: str, out: str, verbose: bool = False) -> str:
    """hipcc `src` for gfx950 into the shared library `out` with the flags above."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, f"-I{INCLUDE}", src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so;
    # that line is expected and harmless.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    return compile_hip(SRC, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
