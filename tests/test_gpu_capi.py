"""The C ABI from plain C: tests/capi/capi_parity.c, built by build(), runs
the library on HIP-runtime buffers and its own stream (no Python, no torch)
and compares with the oracle's C functions to the parity bar."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "capi", "capi_parity")


def test_c_program_matches_the_oracle():
    assert os.path.exists(BIN), "tests/capi/capi_parity is not built (run build())"
    print("[case] capi_parity (plain C caller)", flush=True)
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().endswith("capi parity OK")
    # 2 per IRQ format, 2 QNR (index and pairwise RMSNorm order), 2 KVI, 1 rejected call
    assert res.stdout.count("[capi]") == 9
