"""Helpers for the GPU parity tests: device transfer and the parity bar.

Parity bar (GPU result vs the CPU oracle on identical inputs):
  * scales, slot placement, padding, untouched bytes: bit-exact;
  * e4m3 codes: equal, except at most 1e-4 of the elements may differ by one
    code step (same sign, adjacent magnitude) from fp32 rounding-order ties;
  * bf16 outputs: equal (same fixed operation order on both sides).
"""
import numpy as np
import torch

DEV = "cuda:0"


def dev(a):
    """numpy array -> GPU tensor with the same bits (uint16 arrays -> bf16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def host(t):
    """GPU tensor -> numpy array of its bits (bf16 -> uint16, f8 -> uint8)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32)
    return t.numpy()


def assert_codes_match(got, exp, what="codes", max_frac=1e-4):
    got = np.asarray(got, np.uint8).ravel()
    exp = np.asarray(exp, np.uint8).ravel()
    assert got.shape == exp.shape
    bad = np.flatnonzero(got != exp)
    n = bad.size
    print(f"[parity] {what}: {got.size - n}/{got.size} codes exact, {n} differ", flush=True)
    if n == 0:
        return
    g, e = got[bad].astype(np.int32), exp[bad].astype(np.int32)
    same_sign = (g >> 7) == (e >> 7)
    adjacent = np.abs((g & 0x7F) - (e & 0x7F)) == 1
    assert (same_sign & adjacent).all(), (
        f"{what}: non-adjacent code mismatch at flat index {bad[~(same_sign & adjacent)][:8]}")
    assert n <= max_frac * got.size, f"{what}: {n} one-code differences exceed {max_frac:g}"


def assert_bits_equal(got, exp, what):
    got = np.asarray(got)
    exp = np.asarray(exp)
    assert got.shape == exp.shape, (what, got.shape, exp.shape)
    gb = got.view(np.uint8).reshape(-1)
    eb = exp.view(np.uint8).reshape(-1)
    bad = np.flatnonzero(gb != eb)
    assert bad.size == 0, f"{what}: {bad.size} bytes differ, first at {bad[:8]}"
