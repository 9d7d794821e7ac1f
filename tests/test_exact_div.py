"""The kernels' division forms against IEEE division, on every input.

The kernels compute m / 448 and 1 / s with short FMA sequences instead of
the compiler's divide expansion (rope_fp8_quant_amd/csrc/exact_div.h); the
oracle divides.  Scales are compared bit for bit, so those forms must be
correctly rounded on every input the kernels can give them:
  * m / 448 for every positive normal m >= 2^-116 (the amax floor): checked
    on the host here, and on the GPU with the kernels' own header;
  * 1 / s for every positive normal s < 2^126 (scales stay below 2^119, and
    the RMSNorm's square roots below 2^64): checked on the GPU.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from tests.exact import build as exact_build


def test_div448_form_is_exact_on_the_host():
    if not os.path.exists(exact_build.HOST_BIN):
        exact_build.build_host()
    parts = max(1, min(8, os.cpu_count() or 1))

    def run(i):
        return subprocess.run([exact_build.HOST_BIN, str(parts), str(i)], capture_output=True,
                              text=True, timeout=600)

    with ThreadPoolExecutor(parts) as ex:
        res = list(ex.map(run, range(parts)))
    for r in res:
        assert r.returncode == 0, r.stdout + r.stderr
        assert "0 mismatches" in r.stdout


@pytest.mark.gpu
def test_division_forms_are_exact_on_the_gpu():
    assert os.path.exists(exact_build.GPU_BIN), "run python -m tests.exact.build first"
    print("[case] exact division forms, every positive normal fp32", flush=True)
    r = subprocess.run([exact_build.GPU_BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count(" 0 mismatches") == 2
