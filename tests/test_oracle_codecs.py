"""Pins for the oracle's number-format codecs (CPU only).

Each codec is checked against something other than itself: torch's
bfloat16 / float8_e4m3fn casts (library routines), a brute-force nearest-code
search over the 256 e4m3 values, and closed-form values of the OCP E4M3
format (max 448 = 0x7E, smallest subnormal 2^-9 = 0x01, NaN 0x7F).
"""
import numpy as np
import pytest

import oracle
from tests.helpers import f32_bits, from_bits, torch_bf16, torch_e4m3, torch_e4m3_decode


def _positive_code_values():
    codes = np.arange(0x7F, dtype=np.uint8)  # 0x00..0x7E, all finite
    return codes, oracle.e4m3_to_f32(codes).astype(np.float64)


def _boundary_set():
    """fp32 values within 96 ulps of every e4m3 value and every midpoint."""
    _, vals = _positive_code_values()
    mids = (vals[:-1] + vals[1:]) / 2.0  # exact in fp32 (4 significant bits)
    anchors = np.concatenate([vals, mids]).astype(np.float32)
    anchors = anchors[anchors > 0]
    base = f32_bits(anchors).astype(np.int64)
    offs = np.arange(-96, 97, dtype=np.int64)
    bits = (base[:, None] + offs[None, :]).ravel()
    bits = bits[(bits > 0) & (bits <= f32_bits(np.float32(448.0)).item())]
    pos = from_bits(bits.astype(np.uint32))
    return np.concatenate([pos, -pos, np.array([0.0, -0.0], dtype=np.float32)])


def _random_in_range(n, seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, f32_bits(np.float32(448.0)).item() + 1, size=n, dtype=np.int64)
    sign = rng.integers(0, 2, size=n, dtype=np.int64) << 31
    return from_bits((bits | sign).astype(np.uint32))


def _brute_force_e4m3(x):
    """Nearest finite e4m3 value, ties to the even code (mantissa LSB 0)."""
    codes, vals = _positive_code_values()
    a = np.abs(x.astype(np.float64))
    idx = np.searchsorted(vals, a)  # vals[idx-1] < a <= vals[idx]
    hi = np.clip(idx, 0, len(vals) - 1)
    lo = np.clip(idx - 1, 0, len(vals) - 1)
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(codes[lo] % 2 == 0, lo, hi)))
    pick = np.where(a == vals[hi], hi, pick)
    sign = (f32_bits(x) >> 31).astype(np.uint8)
    return (codes[pick] | (sign << 7)).astype(np.uint8)


def test_e4m3_encode_nan_takes_the_nan_code_with_its_sign():
    # NaN (an infinite block maximum times a zero reciprocal) encodes as
    # S.1111.111, as torch's cast does
    x = from_bits(np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF], np.uint32))
    got = oracle.f32_to_e4m3(x)
    assert (got == np.array([0x7F, 0xFF, 0x7F, 0xFF], np.uint8)).all()
    assert (got == torch_e4m3(x)).all()


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_to_f32(codes)
    ref = torch_e4m3_decode(codes)
    nan = np.isnan(ref)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.isnan(mine[nan]).all()
    assert (f32_bits(mine[~nan]) == f32_bits(ref[~nan])).all()


def test_e4m3_format_closed_forms():
    dec = oracle.e4m3_to_f32(np.array([0x7E, 0x01, 0x08, 0x07, 0x80, 0xFE, 0x38], np.uint8))
    assert list(dec) == [448.0, 2.0 ** -9, 2.0 ** -6, 7 * 2.0 ** -9, -0.0, -448.0, 1.0]
    enc = oracle.f32_to_e4m3(np.array([448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10,
                                       -0.0, 0.0, 1.0, 232.0, 240.0, 248.0, 1.0625,
                                       1.1875, -1e-30], np.float32))
    # 2^-10 is the midpoint of 0 and 2^-9 -> even code 0; 3*2^-10 -> 0x02;
    # 232 is the midpoint of 224 (0x76) and 240 (0x77): even -> 0x76;
    # 248 is the midpoint of 240 (0x77) and 256 (0x78): even -> 0x78;
    # 1.0625 ties 1.0 (0x38) / 1.125 (0x39) -> 0x38; 1.1875 ties 0x39/0x3A -> 0x3A.
    assert list(enc) == [0x7E, 0x01, 0x00, 0x02, 0x80, 0x00, 0x38, 0x76, 0x77, 0x78,
                         0x38, 0x3A, 0x80]


@pytest.mark.parametrize("which", ["boundaries", "random", "bf16_grid"])
def test_e4m3_encode_matches_torch_and_brute_force(which):
    if which == "boundaries":
        x = _boundary_set()
    elif which == "random":
        x = _random_in_range(1 << 22, seed=7)
    else:
        allbf = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
        x = allbf[np.isfinite(allbf) & (np.abs(allbf) <= 448.0)]
    mine = oracle.f32_to_e4m3(x)
    assert (mine == torch_e4m3(x)).all()
    assert (mine == _brute_force_e4m3(x)).all()


def test_e4m3_encode_fp32_subnormal_inputs():
    rng = np.random.default_rng(3)
    bits = rng.integers(1, 1 << 23, size=4096, dtype=np.int64).astype(np.uint32)
    x = np.concatenate([from_bits(bits), -from_bits(bits)])
    mine = oracle.f32_to_e4m3(x)
    assert (mine == torch_e4m3(x)).all()
    assert set(np.unique(mine)) <= {0x00, 0x80}


def test_bf16_to_f32_all_patterns_match_torch():
    import torch
    bits = np.arange(1 << 16, dtype=np.uint16)
    mine = oracle.bf16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert (f32_bits(mine) == f32_bits(ref)).all()


def test_f32_to_bf16_rne_matches_torch():
    rng = np.random.default_rng(11)
    hi = rng.integers(0, 1 << 16, size=1 << 18, dtype=np.int64)
    hi = hi[((hi >> 7) & 0xFF) != 0xFF]  # finite high halves only
    ties = (hi << 16) | 0x8000
    near = np.concatenate([(hi << 16) | 0x7FFF, (hi << 16) | 0x8001])
    rnd = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.int64)
    rnd = rnd[((rnd >> 23) & 0xFF) != 0xFF]
    u = np.concatenate([ties, near, rnd, [0, 1 << 31, 1, 0x7F7FFFFF]]).astype(np.uint32)
    x = from_bits(u)
    x = x[np.isfinite(x)]
    mine = oracle.f32_to_bf16(x)
    assert (mine == torch_bf16(x)).all()


def test_pow2_ceil_exp_brackets():
    rng = np.random.default_rng(5)
    t = from_bits(rng.integers(0x00800000, 0x7F000000, size=1 << 16,
                               dtype=np.int64).astype(np.uint32))
    powers = np.ldexp(np.float32(1.0), np.arange(-126, 127)).astype(np.float32)
    above = from_bits(f32_bits(powers) + 1)
    t = np.concatenate([t, powers, above[np.isfinite(above)]])
    k = oracle.pow2_ceil_exp(t).astype(np.int64)
    tt = t.astype(np.float64)
    assert (np.ldexp(1.0, k) >= tt).all()
    assert (np.ldexp(1.0, k - 1) < tt).all()
    assert (k[len(t) - len(powers) - len(above):][:len(powers)] == np.arange(-126, 127)).all()
