"""Build the exactness checkers of the kernels' division forms.

    python -m tests.exact.build

div448_host (gcc, hardware FMA when the CPU has it) and exact_div_gpu (hipcc
for gfx950, including the kernels' own exact_div.h) land next to their
sources.  Test tools only: the library never uses them.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_SRC = os.path.join(HERE, "div448_host.c")
HOST_BIN = os.path.join(HERE, "div448_host")
GPU_SRC = os.path.join(HERE, "exact_div_gpu.hip")
GPU_BIN = os.path.join(HERE, "exact_div_gpu")


def _cpu_has_fma():
    try:
        with open("/proc/cpuinfo") as f:
            return any(" fma " in (l + " ") for l in f if l.startswith("flags"))
    except OSError:
        return False


def build_host():
    flags = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Werror"]
    if _cpu_has_fma():
        flags.append("-mfma")
    subprocess.run(["gcc", *flags, HOST_SRC, "-o", HOST_BIN, "-lm"], check=True)
    return HOST_BIN


def build_gpu():
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", GPU_SRC, "-o", GPU_BIN]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    return GPU_BIN


def build():
    return build_host(), build_gpu()


if __name__ == "__main__":
    for p in build():
        print(p)
