"""Pins for the oracle's per-head steps: RoPE, block FP8 quant, RMSNorm.

Every check here is independent of the oracle's own formulas: fp64 complex
rotation with angles computed from the RoPE frequency definition, exact
special tables (cos 0 / sin 1), the inverse-after-forward round trip, the
dequantization error bound, the block-max-maps-to-448 property, torch's e4m3
cast on cases where the scale is an exact power of two, an fp64 RMSNorm, and
hand-derived sums that fix the summation order.
"""
import numpy as np
import pytest

import oracle
from rope_fp8_quant_amd import synth
from tests.helpers import bf16_value, e4m3_ulp, f32_bits, rope_angles, torch_e4m3


def _head(seed, std=1.0, nonzero=True):
    x = np.random.default_rng(seed).standard_normal(512).astype(np.float32) * std
    if nonzero:
        x[x == 0] = 1.0
    return x


# ------------------------------------------------------------------ RoPE

def test_rope_nope_dims_bit_identical():
    cache = synth.cos_sin_cache(100)
    for inverse in (True, False):
        x = _head(1)
        y = oracle.rope_head(x, cache[37], inverse)
        assert (f32_bits(y[:448]) == f32_bits(x[:448])).all()
        assert not (f32_bits(y[448:]) == f32_bits(x[448:])).all()


def test_rope_position_zero_is_identity():
    cache = synth.cos_sin_cache(4)
    x = _head(2)
    for inverse in (True, False):
        assert (f32_bits(oracle.rope_head(x, cache[0], inverse)) == f32_bits(x)).all()


def test_rope_quarter_turn_exact():
    # cos = 0, sin = 1: rotation by +90 degrees maps (e, o) -> (-o, e);
    # the inverse maps (e, o) -> (o, -e).  Every product is exact.
    row = np.concatenate([np.zeros(32), np.ones(32)]).astype(np.float32)
    x = _head(3)
    e, o = x[448::2], x[449::2]
    fwd = oracle.rope_head(x, row, inverse=False)
    inv = oracle.rope_head(x, row, inverse=True)
    assert (fwd[448::2] == -o).all() and (fwd[449::2] == e).all()
    assert (inv[448::2] == o).all() and (inv[449::2] == -e).all()


@pytest.mark.parametrize("inverse", [True, False])
def test_rope_matches_fp64_complex_rotation(inverse):
    max_pos = 65536
    positions = np.array([1, 2, 3, 17, 255, 4095, 16383, 40000, 65535])
    cache = synth.cos_sin_cache(max_pos)
    ang = rope_angles(positions)  # [P, 32], independent of the table
    for pi, p in enumerate(positions):
        x = _head(10 + pi)
        y = oracle.rope_head(x, cache[p], inverse)
        z = x[448::2].astype(np.float64) + 1j * x[449::2].astype(np.float64)
        rot = np.exp((-1j if inverse else 1j) * ang[pi])
        w = z * rot
        # Bound: table entries are cos/sin rounded to fp32 (<= 2^-25 each),
        # then two rounded products and one rounded sum (<= 2^-24 relative
        # each), so |error| <= 2^-22 * (|e| + |o|).
        tol = 2.0 ** -22 * (np.abs(x[448::2]) + np.abs(x[449::2])).astype(np.float64)
        assert (np.abs(y[448::2] - w.real) <= tol).all()
        assert (np.abs(y[449::2] - w.imag) <= tol).all()


def test_rope_inverse_after_forward_recovers_input():
    cache = synth.cos_sin_cache(65536)
    rng = np.random.default_rng(4)
    for p in rng.integers(0, 65536, size=64):
        x = _head(int(p), std=3.0)
        back = oracle.rope_head(oracle.rope_head(x, cache[p], False), cache[p], True)
        assert (np.abs(back - x) <= 1e-5 * np.maximum(1.0, np.abs(x))).all()


def test_rope_pair_columns_are_distinct():
    # Row with c_i = (i+1)/64 and s_i = (i+65)/128 (exact fp32 values): with
    # e = 1, o = 0 the inverse gives e' = c_i, o' = -s_i for pair 224+i, which
    # pins which column each pair reads.
    i = np.arange(32)
    row = np.concatenate([(i + 1) / 64.0, (i + 65) / 128.0]).astype(np.float32)
    x = np.zeros(512, np.float32)
    x[448::2] = 1.0
    y = oracle.rope_head(x, row, inverse=True)
    assert (y[448::2] == row[:32]).all() and (y[449::2] == -row[32:]).all()
    y = oracle.rope_head(x, row, inverse=False)
    assert (y[448::2] == row[:32]).all() and (y[449::2] == row[32:]).all()


# ----------------------------------------------------------------- quant

def _check_dequant_bound(x, codes, scales):
    for b in range(4):
        xb = x[128 * b:128 * (b + 1)].astype(np.float64)
        s = float(scales[b])
        deq = oracle.e4m3_to_f32(codes[128 * b:128 * (b + 1)]).astype(np.float64) * s
        # code rounding: half an e4m3 ulp of x/s (in units of s); plus the two
        # fp32 roundings of 1/s and x*(1/s): <= 2^-22 |x|
        bound = 0.5 * e4m3_ulp(xb / s) * s + 2.0 ** -22 * np.abs(xb) + 1e-45
        assert (np.abs(deq - xb) <= bound).all(), b


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_quant_fp32_scale_properties(seed):
    x = _head(seed, std=2.0)
    x[5] = 37.0  # an outlier in block 0
    codes, sc, _ = oracle.quant_head(x, oracle.SCALE_FP32, 1e-10)
    _check_dequant_bound(x, codes, sc)
    for b in range(4):
        blk = codes[128 * b:128 * (b + 1)]
        dec = oracle.e4m3_to_f32(blk)
        # the block's largest magnitude maps to exactly +-448 (code 0x7E/0xFE)
        assert np.abs(dec).max() == 448.0
        am = np.abs(x[128 * b:128 * (b + 1)]).max()
        # scale is amax/448 up to one fp32 rounding
        assert abs(float(sc[b]) - am / 448.0) <= 2.0 ** -24 * am / 448.0


def test_quant_scale_is_exact_quotient():
    x = _head(9)
    codes, sc, _ = oracle.quant_head(x, oracle.SCALE_FP32, 1e-10)
    am = np.abs(x.reshape(4, 128)).max(axis=1).astype(np.float32)
    assert (f32_bits(sc) == f32_bits(am / np.float32(448.0))).all()


def test_quant_blocks_are_independent():
    x = _head(8)
    for b in range(4):
        x[128 * b:128 * (b + 1)] *= np.float32(10.0 ** b)
    codes, sc, _ = oracle.quant_head(x, oracle.SCALE_FP32, 1e-10)
    assert np.all(sc[1:] / sc[:-1] > 5)  # each scale follows its own block
    _check_dequant_bound(x, codes, sc)


@pytest.mark.parametrize("k", [0, -3, 5])
def test_quant_power_of_two_scale_reduces_to_torch_cast(k):
    # If a block's amax is 448 * 2^k the scale is exactly 2^k, 1/s is exact,
    # and the codes are torch's e4m3 cast of x * 2^-k.
    rng = np.random.default_rng(100 + k)
    x = (rng.uniform(-1, 1, 512) * 448.0).astype(np.float32)
    for b in range(4):
        x[128 * b + 3] = 448.0
    x = (x * np.float32(2.0 ** k)).astype(np.float32)
    codes, sc, _ = oracle.quant_head(x, oracle.SCALE_FP32, 1e-10)
    assert (sc == np.float32(2.0 ** k)).all()
    assert (codes == torch_e4m3(x * np.float32(2.0 ** -k))).all()


def test_quant_zero_block_uses_eps():
    x = _head(12)
    x[128:256] = 0.0
    eps = 1e-10
    codes, sc, _ = oracle.quant_head(x, oracle.SCALE_FP32, eps)
    assert (codes[128:256] == 0).all()
    assert abs(float(sc[1]) - eps / 448.0) <= 2.0 ** -23 * eps / 448.0
    x[128:256] = -0.0
    codes, _, _ = oracle.quant_head(x, oracle.SCALE_FP32, eps)
    assert (codes[128:256] == 0x80).all()


@pytest.mark.parametrize("scale_fmt", [oracle.SCALE_FP32, oracle.SCALE_UE8M0])
def test_quant_overflowed_block(scale_fmt):
    # Block 3 holds +inf (a rotated pair that overflowed fp32); the other
    # blocks are unaffected.  IEEE arithmetic on the same formulas: FP32 gives
    # s = inf / 448 = inf and 1/s = 0, so finite values encode as signed
    # zeros and the infinity as NaN (inf * 0); UE8M0 gives k = 128, s = 2^128
    # = inf and exponent byte 0xFF, and the finite values are scaled by the
    # exact 2^-128 (the infinity clamps to 448).
    x = _head(31, std=1e30)
    x[500] = np.inf
    codes, sc, word = oracle.quant_head(x, scale_fmt)
    ref_c, ref_s, ref_w = oracle.quant_head(np.where(np.arange(512) < 384, x, 1.0)
                                            .astype(np.float32), scale_fmt)
    assert (codes[:384] == ref_c[:384]).all() and (sc[:3] == ref_s[:3]).all()
    assert sc[3] == np.inf
    blk = x[384:]
    if scale_fmt == oracle.SCALE_FP32:
        fin = np.isfinite(blk)
        assert (codes[384:][fin] == np.where(np.signbit(blk[fin]), 0x80, 0x00)).all()
        assert codes[500] & 0x7F == 0x7F  # NaN code
    else:
        assert (word >> 24) == 0xFF and (word & 0xFFFFFF) == (ref_w & 0xFFFFFF)
        scaled = blk.astype(np.float64) * 2.0 ** -128  # exact
        exp = torch_e4m3(np.clip(scaled, -448, 448).astype(np.float32))
        assert (codes[384:] == exp).all()
        assert codes[500] == 0x7E


@pytest.mark.parametrize("seed", [0, 1])
def test_quant_ue8m0_properties(seed):
    x = _head(seed, std=3.0)
    x[300] = -250.0
    codes, sc, word = oracle.quant_head(x, oracle.SCALE_UE8M0, 1e-10)
    for b in range(4):
        am = float(np.abs(x[128 * b:128 * (b + 1)]).max())
        t = np.float32(am) / np.float32(448.0)
        s = float(sc[b])
        m, e = np.frexp(s)
        assert m == 0.5  # a power of two
        assert s / 2 < t <= s
        assert ((word >> (8 * b)) & 0xFF) == int(e - 1) + 127
        dec = oracle.e4m3_to_f32(codes[128 * b:128 * (b + 1)]).astype(np.float64) * s
        xb = x[128 * b:128 * (b + 1)].astype(np.float64)
        # x * 2^-k is exact, so only the e4m3 rounding remains
        assert (np.abs(dec - xb) <= 0.5 * e4m3_ulp(xb / s) * s + 1e-45).all()
        # and the codes are torch's cast of the exactly scaled values
        assert (codes[128 * b:128 * (b + 1)] ==
                torch_e4m3(np.clip(x[128 * b:128 * (b + 1)] / np.float32(s), -448, 448))).all()


# --------------------------------------------------------------- RMSNorm

def _rms64(x, w, eps):
    x = x.astype(np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x) + eps)
    return x * r * (1.0 if w is None else bf16_value(w).astype(np.float64))


@pytest.mark.parametrize("sum_order", ["index", "pairwise"])
@pytest.mark.parametrize("eps", [1e-6, 0.5])
def test_rmsnorm_matches_fp64(eps, sum_order):
    w = synth.uniform_bf16((512,), 3, synth.T_W, 0.5, 1.5)
    for seed in range(8):
        x = _head(seed, std=2.0)
        y = oracle.rmsnorm_head(x, w, eps, sum_order=sum_order).astype(np.float64)
        ref = _rms64(x, w, eps)
        assert (np.abs(y - ref) <= 4e-6 * np.abs(ref) + 1e-30).all()


def test_rmsnorm_constant_row_closed_form():
    for c in (0.5, 3.0, -7.25):
        x = np.full(512, c, np.float32)
        y = oracle.rmsnorm_head(x, None, 1e-6).astype(np.float64)
        ref = c / np.sqrt(c * c + 1e-6)
        assert (np.abs(y - ref) <= 2.0 ** -21 * abs(ref)).all()


def test_rmsnorm_null_weight_equals_unit_weight():
    x = _head(21)
    ones = np.full(512, 0x3F80, np.uint16)  # bf16 1.0
    a = oracle.rmsnorm_head(x, None, 1e-6)
    b = oracle.rmsnorm_head(x, ones, 1e-6)
    assert (f32_bits(a) == f32_bits(b)).all()


def _r_of_ss(ss, eps=1e-6):
    """r for a given fp32 sum of squares, each step one fp32 rounding."""
    mean = np.float32(ss) / np.float32(512.0)
    return np.float32(1.0) / np.sqrt(mean + np.float32(eps), dtype=np.float32)


def test_rmsnorm_index_order_hand_derived():
    # x = [2^12, 1 x 511].  Left to right, 2^24 + 1 lies halfway between 2^24
    # and 2^24 + 2 and rounds to the even 2^24, so each of the 511 additions
    # leaves 2^24: ss = 2^24.  The exact sum is 2^24 + 511; summed right to
    # left it is 2^24 + 512 (511 + 2^24 ties to the even 2^24 + 512).
    x = np.ones(512, np.float32)
    x[0] = 2.0 ** 12
    assert f32_bits(oracle.sum_squares(x)) == f32_bits(np.float32(2.0 ** 24))
    y = oracle.rmsnorm_head(x, None, 1e-6)
    r = _r_of_ss(2.0 ** 24)
    assert f32_bits(y[1]) == f32_bits(r)
    assert f32_bits(y[0]) == f32_bits(np.float32(2.0 ** 12) * r)
    for other in (2.0 ** 24 + 511, 2.0 ** 24 + 512):
        assert _r_of_ss(other) != r  # the case tells the orders apart


# Pairwise summation by hand.  A range's sum is its two halves' sums added
# ([0, n/2) and [n/2, n)); a lone square is itself.  Near 2^24 fp32 holds the
# even integers, and an odd one rounds to the even neighbour whose last
# significand bit is 0: 2^24 + 1 -> 2^24, 2^24 + 3 -> 2^24 + 4.
PAIRWISE_CASES = [
    # x = [2^12, 1 x 511]: [0, 2) = 2^24 + 1 -> 2^24; every other range of 2^l
    # dims is 2^l exactly; [0, 2^l) = 2^24 + 2 + 4 + ... + 2^(l-1) =
    # 2^24 + 2^l - 2, exact, so [0, 512) = 2^24 + 510.  (Index order 2^24;
    # exact 2^24 + 511; right to left 2^24 + 512; left to right within 8-dim
    # chunks, then pairwise over the chunks, 2^24 + 504.)
    ("ones", [2.0 ** 12] + [1.0] * 511, 2.0 ** 24 + 510),
    # x = [2^12, 0, 1, 1, 0 x 508]: [0, 2) = 2^24, [2, 4) = 2, [0, 4) =
    # 2^24 + 2, the rest zeros.  Adding a lone 1 to 2^24 first (index order,
    # left to right within chunks, halving strides that pair dim i with
    # i + n/2) gives 2^24.
    ("pair", [2.0 ** 12, 0.0, 1.0, 1.0] + [0.0] * 508, 2.0 ** 24 + 2),
    # ragged lengths: n = 3 is x0^2 + (x1^2 + x2^2) = 2^24 + 2; n = 5 is
    # (x0^2 + x1^2) + (x2^2 + (x3^2 + x4^2)) = 2^24 + 3 -> 2^24 + 4
    ("n3", [2.0 ** 12, 1.0, 1.0], 2.0 ** 24 + 2),
    ("n5", [2.0 ** 12, 1.0, 1.0, 1.0, 1.0], 2.0 ** 24 + 4),
    ("n1", [-3.0], 9.0),
    # x = [2^12, 0 x 254, 1, 1, 0 x 255]: the ones at dims 255 and 256 lie in
    # different halves; [0, 256) = 2^24 + 1 -> 2^24, [256, 512) = 1, and
    # 2^24 + 1 -> 2^24.  (Right to left, or a split elsewhere than the middle,
    # adds the two ones first: 2^24 + 2.)
    ("split", [2.0 ** 12] + [0.0] * 254 + [1.0, 1.0] + [0.0] * 255, 2.0 ** 24),
]


@pytest.mark.parametrize("name,x,ss", PAIRWISE_CASES, ids=[c[0] for c in PAIRWISE_CASES])
def test_sum_squares_pairwise_hand_derived(name, x, ss):
    x = np.asarray(x, np.float32)
    assert f32_bits(oracle.sum_squares(x, "pairwise")) == f32_bits(np.float32(ss))
    if name not in ("n1", "split"):  # these tell pairwise from index order
        assert f32_bits(oracle.sum_squares(x)) == f32_bits(np.float32(2.0 ** 24))


@pytest.mark.parametrize("sum_order", ["index", "pairwise"])
def test_rmsnorm_applies_its_sum(sum_order):
    # the normalisation after the sum: mean = ss / 512, r = 1 / sqrt(mean +
    # eps), y = x * r, each one fp32 rounding
    rows = [np.asarray(PAIRWISE_CASES[0][1], np.float32),
            np.asarray(PAIRWISE_CASES[1][1], np.float32)]
    rows += [_head(seed, std=2.0) for seed in range(3)]
    for x in rows:
        r = _r_of_ss(oracle.sum_squares(x, sum_order))
        y = oracle.rmsnorm_head(x, None, 1e-6, sum_order=sum_order)
        assert (f32_bits(y) == f32_bits(x * r)).all()


def test_rmsnorm_pairwise_order_hand_derived():
    # x = [2^12, 0, 1, 1, 0 x 508] (the "pair" case): ss = 2^24 + 2 pairwise,
    # 2^24 in index order, and the two give different r.
    x = np.asarray(PAIRWISE_CASES[1][1], np.float32)
    r = _r_of_ss(2.0 ** 24 + 2)
    y = oracle.rmsnorm_head(x, None, 1e-6, sum_order="pairwise")
    assert f32_bits(y[2]) == f32_bits(np.float32(1.0) * r)
    assert f32_bits(y[0]) == f32_bits(np.float32(2.0 ** 12) * r)
    r_index = _r_of_ss(2.0 ** 24)
    assert r != r_index  # the test can tell the orders apart
    assert f32_bits(oracle.rmsnorm_head(x, None, 1e-6)[2]) == f32_bits(r_index)


@pytest.mark.parametrize("sum_order", ["index", "pairwise"])
def test_rmsnorm_orders_exact_on_exact_sums(sum_order):
    # Small integers: every square and every partial sum is an exact fp32
    # integer, so any order gives the exact sum, and both orders agree bit for
    # bit with each other and with the fp64 closed form rounded per step.
    rng = np.random.default_rng(5)
    for _ in range(4):
        x = rng.integers(-8, 9, 512).astype(np.float32)
        ss = float(np.sum(x.astype(np.float64) ** 2))
        y = oracle.rmsnorm_head(x, None, 1e-6, sum_order=sum_order)
        assert (f32_bits(y) == f32_bits(x * _r_of_ss(ss))).all()
