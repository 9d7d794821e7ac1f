"""Helpers for the GPU parity tests: device transfer, launch-table sizes and
the parity bar.

Parity bar (GPU result vs the CPU oracle on identical inputs):
  * scales, slot placement, padding, untouched bytes: bit-exact;
  * e4m3 codes: equal, except at most 1e-4 of the elements may differ by one
    code step (same sign, adjacent magnitude) from fp32 rounding-order ties;
  * bf16 outputs: equal (same fixed operation order on both sides);
  * the q paths, whose RMSNorm sums 512 squares in an order the pages do not
    fix: against the oracle's definition (index order), within bounds derived
    from the two orders' rounding (Q_RTOL below), with at most 1e-3 of the
    bf16 elements and 1e-4 of the codes differing; and bit for bit against
    the oracle summing by recursive pairwise summation, the kernel's order,
    which isolates the summation order from every other step.
"""
import numpy as np
import torch

import oracle
from tests.helpers import e4m3_ulp, torch_e4m3_decode

DEV = "cuda:0"

# The library's launch table: a launch of at least TABLE_ROWS work units
# (512-dim heads; for the indexer, four-head items: ceil(H/4) per token)
# takes its kernel's prefill workgroup size, a smaller one 64-thread
# workgroups.  Tests reach both entries by the size of their inputs.
TABLE_ROWS = 16384
SHAPES = ("decode_table", "prefill_table")


def table_tokens(shape, rows_per_token, base=37):
    """A token count whose launch lands in table entry `shape`: `base` for the
    64-thread entry, else past TABLE_ROWS units (`rows_per_token` per token).  Where the row count per token
    allows it, the total is kept off a multiple of 16 so that the last
    workgroup is ragged in either entry."""
    if shape == "decode_table":
        assert base * rows_per_token < TABLE_ROWS
        return base
    n = -(-TABLE_ROWS // rows_per_token) + base
    if rows_per_token % 16 and (n * rows_per_token) % 16 == 0:
        n += 1
    return n


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


# Derived bound on how far the q paths may move between two summation orders
# of RMSNorm's 512 squares.  Any order of n non-negative addends is within
# gamma_(n-1) = 511*2^-24/(1-511*2^-24) of the exact sum, so two orders differ
# by at most about 3.05e-5 relative; 1/sqrt halves that, and the few further
# roundings (sqrt, divide, the weight product, the rotation, amax/448) add
# under 2^-20: 1.7e-5 < 2^-15.  So the normalized values, and every block
# scale, move by at most Q_RTOL relative; a rotated value e*c - o*s moves by
# at most Q_RTOL * (|e| + |o|) <= Q_RTOL * sqrt(2) * |(e', o')| (the rotation
# keeps the pair's norm), which is many of its own ulps when the two products
# nearly cancel.
Q_RTOL = 2.0 ** -15

# On the forward workloads (8192 tokens x 64 heads with a norm weight, and
# slices of them) the q paths may also differ from the definition's rounding
# in at most 1e-3 of the bf16 values and 1e-4 of the e4m3 codes.  Without a
# weight, or with a large eps, r cancels out of the codes to first order and
# far more values sit on rounding midpoints, so these counts are asserted on
# those workloads only.
Q_DEF_FRAC_BF16 = 1e-3
Q_DEF_FRAC_CODES = 1e-4


def _q_slack(z):
    """Per element of fp32 q values z [..., 512]: the derived bound on how far
    another summation order can move it (Q_RTOL relative, plus the rotated
    pair's norm term in dims 448..511)."""
    z = np.asarray(z, np.float64)
    d = Q_RTOL * np.abs(z)
    pair = z[..., 448:].reshape(z.shape[:-1] + (32, 2))
    norm = np.sqrt((pair ** 2).sum(-1))
    d[..., 448:] += np.repeat(Q_RTOL * np.sqrt(2.0) * norm, 2, axis=-1)
    return d


def _rounding_interval(ordinal, values, lo_end=-np.inf, hi_end=np.inf):
    """[lo, hi] of the reals that round to the value of each ordinal (a
    monotonic integer index of the format's values), from the midpoints to
    its neighbours; the ends of the range are open towards lo_end / hi_end."""
    ordinal = np.asarray(ordinal, np.int64)
    lo_n = values(ordinal - 1)
    hi_n = values(ordinal + 1)
    v = values(ordinal)
    lo = np.where(np.isfinite(lo_n), (lo_n + v) / 2, lo_end)
    hi = np.where(np.isfinite(hi_n), (hi_n + v) / 2, hi_end)
    return lo, hi


def _bf16_ordinal(bits):
    b = np.asarray(bits, np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _bf16_of_ordinal(k):
    k = np.asarray(k, np.int64)
    bits = np.where(k < 0, 0x8000 | (-k), k)
    ok = np.abs(k) <= 0x7F7F  # finite bf16 magnitudes
    v = (np.where(ok, bits, 0).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.where(ok, v, np.where(k > 0, np.inf, -np.inf))


def _e4m3_ordinal(codes):
    c = np.asarray(codes, np.int64)
    return np.where(c & 0x80, -(c & 0x7F), c)


_E4M3_POS = None


def _e4m3_of_ordinal(k):
    global _E4M3_POS
    if _E4M3_POS is None:
        _E4M3_POS = torch_e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    k = np.asarray(k, np.int64)
    ok = np.abs(k) <= 0x7E  # 448 is the largest finite magnitude
    v = _E4M3_POS[np.minimum(np.abs(k), 0x7E)] * np.sign(k)
    return np.where(ok, v, np.where(k > 0, np.inf, -np.inf))


def _outside(z, lo, hi):
    return np.maximum(np.maximum(lo - z, z - hi), 0.0)


def assert_bf16_near_definition(got, z_def, exp, what, max_frac=None):
    """q-path bf16 rows of the live heads against the oracle's definition:
    where a value differs from the definition's rounding `exp`, the
    definition's fp32 value z_def must lie within the derived slack of the
    interval of reals that round to the value written.  With max_frac, at
    most that fraction of the values may differ at all."""
    got = np.asarray(got, np.uint16).reshape(-1, 512)
    exp = np.asarray(exp, np.uint16).reshape(-1, 512)
    z = np.asarray(z_def, np.float32).reshape(-1, 512)
    assert got.shape == exp.shape == z.shape, (what, got.shape, exp.shape, z.shape)
    rows = np.flatnonzero((got != exp).any(axis=1))
    g, e, zr = got[rows], exp[rows], z[rows].astype(np.float64)
    diff = g != e
    lo, hi = _rounding_interval(_bf16_ordinal(g[diff]), _bf16_of_ordinal)
    off = _outside(zr[diff], lo, hi)
    slack = _q_slack(zr)[diff]
    n = int(diff.sum())
    far = int((np.abs(g.astype(np.int32) - e.astype(np.int32))[diff] > 1).sum())
    print(f"[parity] {what}: {got.size - n}/{got.size} equal, {n} differ ({n / got.size:.2e}; "
          f"{far} by more than one ulp), each within the summation-order slack of its "
          f"rounding boundary", flush=True)
    assert (off <= slack).all(), f"{what}: {int((off > slack).sum())} differences unexplained"
    if max_frac is not None:
        assert n <= max_frac * got.size, f"{what}: {n / got.size:.2e} of the values differ"


def assert_q_out_parity(got, q, w, pos, cache, hpad, eps, what, max_frac=None):
    """QNR bf16 rows: pad heads exact, live heads within the derived slack of
    the RMSNorm definition (and, with max_frac, differing from it in at most
    that fraction of the values), and bit for bit the oracle with the
    kernel's summation order (pairwise)."""
    got = np.asarray(got, np.uint16)
    exp = oracle.qnorm_rope(q, w, pos, cache, hpad, eps)
    hq = q.shape[1]
    assert_bits_equal(got[:, hq:], exp[:, hq:], f"{what} pad heads")
    z = oracle.qnorm_rope_f32(q, w, pos, cache, eps)
    assert_bf16_near_definition(got[:, :hq], z, exp[:, :hq], f"{what} vs index-order RMSNorm",
                                max_frac)
    exp_pw = oracle.qnorm_rope(q, w, pos, cache, hpad, eps, sum_order="pairwise")
    assert_bits_equal(got, exp_pw, f"{what} vs pairwise-summed RMSNorm")


def _scales_f32(sc, fmt):
    """Block scales as float64 [n, 4] (UE8M0 words unpacked to 2^(e-127))."""
    sc = np.asarray(sc)
    if fmt == "ue8m0":
        w = sc.view(np.uint32).reshape(-1)
        e = np.stack([(w >> (8 * b)) & 0xFF for b in range(4)], axis=1).astype(np.int64)
        return e, np.ldexp(1.0, e - 127)
    return None, sc.view(np.float32).reshape(-1, 4).astype(np.float64)


def assert_fp8_near_definition(codes, sc, z_def, ec, es, fmt, what, max_frac=None):
    """FP8 q path of the live heads against the oracle's definition: block
    scales within Q_RTOL (UE8M0: exponent bytes within one), and where a code
    differs from the definition's, the definition's fp32 value scaled by the
    written block's own multiplier must lie within the derived slack (plus
    two fp32 roundings) of the interval of values that encode to the written
    code.  With max_frac, at most that fraction of the codes may differ at
    all."""
    ge, gs = _scales_f32(sc, fmt)
    ee, xs = _scales_f32(es, fmt)
    assert gs.shape == xs.shape
    if fmt == "ue8m0":
        assert (np.abs(ge - ee) <= 1).all(), f"{what}: UE8M0 exponents more than one apart"
        mult = np.ldexp(1.0, -(ge - 127))
    else:
        rel = np.abs(gs - xs) / xs
        assert (rel <= Q_RTOL).all(), f"{what}: scale off by {rel.max():.3g}"
        mult = (np.float32(1.0) / gs.astype(np.float32)).astype(np.float64)
    gc = np.asarray(codes, np.uint8).reshape(-1, 4, 128)
    xc = np.asarray(ec, np.uint8).reshape(-1, 4, 128)
    z = np.asarray(z_def, np.float32).reshape(-1, 4, 128)
    diff = gc != xc
    n = int(diff.sum())
    heads = np.flatnonzero(diff.reshape(diff.shape[0], -1).any(axis=1))
    v = (z[heads].astype(np.float64) * mult[heads][:, :, None]).reshape(-1, 512)
    slack = _q_slack(v).reshape(-1, 4, 128) + 2.0 ** -22 * np.abs(v).reshape(-1, 4, 128)
    d = diff[heads]
    lo, hi = _rounding_interval(_e4m3_ordinal(gc[heads][d]), _e4m3_of_ordinal)
    off = _outside(v.reshape(-1, 4, 128)[d], lo, hi)
    print(f"[parity] {what}: {int((gs != xs).sum())}/{gs.size} block scales and {n}/{gc.size} "
          f"codes ({n / gc.size:.2e}) differ from the definition, each within the "
          f"summation-order slack of its rounding boundary", flush=True)
    assert (off <= slack[d]).all(), f"{what}: {int((off > slack[d]).sum())} codes unexplained"
    if max_frac is not None:
        assert n <= max_frac * gc.size, f"{what}: {n / gc.size:.2e} of the codes differ"


def assert_q_fp8_parity(codes, sc, q, w, pos, cache, hpad, eps, fmt, what, quant_eps=1e-10,
                        max_frac=None):
    """FP8 q path: pad heads exact, live heads within the derived slack of the
    definition (and, with max_frac, differing from it in at most that
    fraction of the codes), and bit for bit (codes to the code bar) the
    oracle with the kernel's summation order (pairwise)."""
    f = oracle.SCALE_UE8M0 if fmt == "ue8m0" else oracle.SCALE_FP32
    codes = np.asarray(codes, np.uint8)
    sc = np.asarray(sc)
    ec, es = oracle.qnorm_rope_fp8(q, w, pos, cache, hpad, eps, f, quant_eps)
    hq = q.shape[1]
    assert_bits_equal(codes[:, hq:], ec[:, hq:], f"{what} pad-head codes")
    assert_bits_equal(sc[:, hq:], es[:, hq:], f"{what} pad-head scales")
    z = oracle.qnorm_rope_f32(q, w, pos, cache, eps)
    assert_fp8_near_definition(codes[:, :hq], sc[:, :hq], z, ec[:, :hq], es[:, :hq], fmt,
                               f"{what} vs index-order RMSNorm", max_frac)
    ec, es = oracle.qnorm_rope_fp8(q, w, pos, cache, hpad, eps, f, quant_eps,
                                   sum_order="pairwise")
    assert_bits_equal(sc, es, f"{what} scales vs pairwise-summed RMSNorm")
    assert_codes_match(codes, ec, f"{what} codes vs pairwise-summed RMSNorm")
