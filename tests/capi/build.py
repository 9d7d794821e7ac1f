"""Build the plain-C parity program (``capi_parity``) of the C ABI.

    python -m tests.capi.build

A host-only C11 program: gcc against the HIP runtime headers, linked with
libropequant.so and the oracle's libropequant_oracle.so (both built first),
with run paths relative to the binary so the tree can move.  Test tool only.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "capi_parity.c")
BIN = os.path.join(HERE, "capi_parity")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build():
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{ROOT}/include", SRC, "-o", BIN,
           f"-L{ROOT}/rope_fp8_quant_amd", "-lropequant", f"-L{ROOT}/oracle", "-lropequant_oracle",
           f"-L{ROCM}/lib", "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../rope_fp8_quant_amd:$ORIGIN/../../oracle:" + f"{ROCM}/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("gcc failed:\n" + res.stdout + res.stderr)
    return BIN


if __name__ == "__main__":
    print(build())
