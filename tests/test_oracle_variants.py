"""Pins for the oracle's output variants: inverse RoPE without quantization
(bf16 out), the q path into FP8, and the kv path into a token-strided bf16
cache.

Each variant is checked against things other than its own composition:
fp64 rotations with angles from the frequency definition, exact closed forms
(identity tables, constant-magnitude heads, zero heads), layouts rebuilt with
numpy reshapes, and agreement with the already pinned quantized ops through
dequantization.
"""
import math

import numpy as np
import pytest

import oracle
from rope_fp8_quant_amd import synth
from tests.helpers import bf16_value, e4m3_ulp, f32_bits, rope_angles


def _identity_cache(max_pos):
    c = np.zeros((max_pos, 64), np.float32)
    c[:, :32] = 1.0
    return c


def _bf16_ulp(y):
    a = np.maximum(np.abs(y), 1e-30)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _rotate64(x, ang, sign):
    """fp64 GPT-J rotation of dims 448..511 by sign*angle (x is fp64 [512])."""
    y = x.copy()
    z = (x[448::2] + 1j * x[449::2]) * np.exp(sign * 1j * ang)
    y[448::2], y[449::2] = z.real, z.imag
    return y


def _rounding_bound(x, y):
    """One bf16 rounding of y, plus fp32 product/sum errors on the rotated pairs
    (relative to the pair's magnitude, which covers cancellation)."""
    mag = np.zeros_like(x)
    pair = np.abs(x[448::2]) + np.abs(x[449::2])
    mag[448::2] = pair
    mag[449::2] = pair
    return 0.5 * _bf16_ulp(y) + 2.0 ** -20 * mag + 1e-30


# ------------------------------------------------------ inverse RoPE, bf16

@pytest.mark.parametrize("H,hpg", [(8, 8), (32, 8), (48, 6), (6, 3)])
def test_irb_identity_table_is_the_input_in_group_layout(H, hpg):
    # cos = 1, sin = 0: every output element is its input's bits, placed at
    # [g, t, j*512 + d] (rebuilt with numpy reshapes only)
    N = 5
    o = synth.normal_bf16((N, H, 512), 31, synth.T_O)
    out = oracle.inv_rope_bf16(o, np.arange(N, dtype=np.int64), _identity_cache(8), hpg)
    expect = o.reshape(N, H // hpg, hpg * 512).transpose(1, 0, 2)
    assert (out == expect).all()


def test_irb_pass_through_dims_are_bit_copies():
    o, pos, cache = synth.irq_inputs(synth.IRQ_TINY)
    out = oracle.inv_rope_bf16(o, pos, cache, 8)
    got = out.reshape(16, 8, 512)  # G == 1: [1, N, 8*512] is [N, 8, 512]
    assert (got[:, :, :448] == o[:, :, :448]).all()
    assert not (got[:, :, 448:] == o[:, :, 448:]).all()


def test_irb_fp64_inverse_rotation_within_one_rounding():
    o, pos, cache = synth.irq_inputs(synth.IRQ_TINY)
    out = oracle.inv_rope_bf16(o, pos, cache, 8).reshape(16, 8, 512)
    ang = rope_angles(pos)
    for t in range(16):
        for h in range(8):
            x = bf16_value(o[t, h]).astype(np.float64)
            ref = _rotate64(x, ang[t], -1)
            got = bf16_value(out[t, h]).astype(np.float64)
            assert (np.abs(got - ref) <= _rounding_bound(x, ref)).all()


def test_irb_agrees_with_the_quantized_op():
    # dequantized IRQ codes (a pinned op) sit within the e4m3 step of the bf16
    # output, head by head, in the same group-major places
    cfg = dict(synth.IRQ_TINY, N=6, H=12, hpg=6)
    o, pos, cache = synth.irq_inputs(cfg)
    codes, sc = oracle.inv_rope_fp8_quant(o, pos, cache, 6)
    out = oracle.inv_rope_bf16(o, pos, cache, 6)
    y = bf16_value(out).astype(np.float64)
    s = np.repeat(sc.astype(np.float64), 128, axis=2)
    deq = oracle.e4m3_to_f32(codes).astype(np.float64) * s
    bound = 0.5 * e4m3_ulp(y / s) * s + 0.5 * _bf16_ulp(y) + 1e-30
    assert (np.abs(deq - y) <= bound).all()


def test_irb_token_major_is_group_major_permuted():
    cfg = dict(synth.IRQ_TINY, N=7, H=12, hpg=4)
    o, pos, cache = synth.irq_inputs(cfg)
    g = oracle.inv_rope_bf16(o, pos, cache, 4, layout="group")
    t = oracle.inv_rope_bf16(o, pos, cache, 4, layout="token")
    assert (t.reshape(7, 3, 4 * 512).transpose(1, 0, 2) == g).all()


def test_irb_rejects_bad_arguments():
    o, pos, cache = synth.irq_inputs(synth.IRQ_TINY)
    with pytest.raises(oracle.OracleError):
        oracle.inv_rope_bf16(o, pos, cache, 3)
    bad = pos.copy()
    bad[0] = -1
    with pytest.raises(oracle.OracleError):
        oracle.inv_rope_bf16(o, bad, cache, 8)


# ---------------------------------------------------------- q path, FP8

def _pow2_ceil_exp_f64(t):
    """Smallest k with 2^k >= t, from frexp (t = m * 2^e, 0.5 <= m < 1)."""
    m, e = math.frexp(float(t))
    return e - 1 if m == 0.5 else e


def test_qf8_constant_magnitude_heads_hit_full_scale():
    # heads of +-a with no weight and an identity table: RMSNorm makes every
    # element +-1 (to rounding), the block amax is that magnitude, and every
    # code is +-448 (0x7E / 0xFE)
    N, Hq, Hpad = 3, 4, 4
    rng = np.random.default_rng(5)
    sgn = rng.choice([-1.0, 1.0], size=(N, Hq, 512))
    a = np.array([0.5, 3.0, 40.0, 1e-3])[None, :, None]
    q = synth.f32_to_bf16_bits((sgn * a).astype(np.float32))
    codes, sc = oracle.qnorm_rope_fp8(q, None, np.zeros(N, np.int64), _identity_cache(1), Hpad,
                                      1e-6)
    assert (codes == np.where(sgn > 0, 0x7E, 0xFE)).all()
    a_eff = np.broadcast_to(np.abs(bf16_value(q)[:, :, :1]).astype(np.float64), (N, Hq, 4))
    r = 1.0 / np.sqrt(a_eff ** 2 + 1e-6)
    assert np.allclose(sc.astype(np.float64), a_eff * r / 448.0, rtol=2.0 ** -18, atol=0)


@pytest.mark.parametrize("fmt", [oracle.SCALE_FP32, oracle.SCALE_UE8M0])
def test_qf8_pad_heads_are_quantized_zero_heads(fmt):
    cfg = dict(synth.QNR_FORWARD, N=3, Hq=2, Hpad=5)
    q, w, pos, cache = synth.qnr_inputs(cfg)
    eps = 1e-10
    codes, sc = oracle.qnorm_rope_fp8(q, w, pos, cache, 5, 1e-6, fmt, eps)
    assert (codes[:, 2:] == 0).all()
    t = np.float32(eps) / np.float32(448.0)
    if fmt == oracle.SCALE_FP32:
        assert (f32_bits(sc[:, 2:]) == f32_bits(np.full((3, 3, 4), t, np.float32))).all()
    else:
        k = _pow2_ceil_exp_f64(t)
        b = k + 127
        assert (sc[:, 2:] == np.uint32(b | b << 8 | b << 16 | b << 24)).all()


@pytest.mark.parametrize("fmt", [oracle.SCALE_FP32, oracle.SCALE_UE8M0])
def test_qf8_dequant_matches_the_bf16_q_path(fmt):
    # the bf16 QNR oracle (pinned) and this one quantize the same fp32 head:
    # the two differ by at most half an e4m3 step plus half a bf16 step
    cfg = dict(synth.QNR_FORWARD, N=4, Hq=6, Hpad=8)
    q, w, pos, cache = synth.qnr_inputs(cfg)
    codes, sc = oracle.qnorm_rope_fp8(q, w, pos, cache, 8, 1e-6, fmt)
    ref = bf16_value(oracle.qnorm_rope(q, w, pos, cache, 8, 1e-6)).astype(np.float64)
    if fmt == oracle.SCALE_FP32:
        s = np.repeat(sc.astype(np.float64), 128, axis=2)
    else:
        e = np.stack([(sc >> (8 * b)) & 0xFF for b in range(4)], axis=-1).astype(np.float64)
        s = np.repeat(2.0 ** (e - 127), 128, axis=2)
    deq = oracle.e4m3_to_f32(codes).astype(np.float64) * s
    bound = 0.5 * e4m3_ulp(ref / s) * s + 0.5 * _bf16_ulp(ref) + 1e-30
    assert (np.abs(deq - ref) <= bound).all()


def test_qf8_scales_are_block_amax_over_448_in_fp64():
    cfg = dict(synth.QNR_FORWARD, N=3, Hq=5, Hpad=5)
    q, w, pos, cache = synth.qnr_inputs(cfg)
    codes, sc = oracle.qnorm_rope_fp8(q, w, pos, cache, 5, 1e-6)
    ang = rope_angles(pos)
    wf = bf16_value(w).astype(np.float64)
    for t in range(3):
        for h in range(5):
            x = bf16_value(q[t, h]).astype(np.float64)
            y = _rotate64(x / np.sqrt(np.mean(x * x) + 1e-6) * wf, ang[t], 1)
            amax = np.abs(y).reshape(4, 128).max(axis=1)
            assert np.allclose(sc[t, h].astype(np.float64) * 448.0, amax, rtol=2.0 ** -16)


def test_qf8_ue8m0_scales_are_the_smallest_covering_powers_of_two():
    cfg = dict(synth.QNR_FORWARD, N=2, Hq=7, Hpad=7)
    q, w, pos, cache = synth.qnr_inputs(cfg)
    _, s32 = oracle.qnorm_rope_fp8(q, w, pos, cache, 7, 1e-6, oracle.SCALE_FP32)
    _, word = oracle.qnorm_rope_fp8(q, w, pos, cache, 7, 1e-6, oracle.SCALE_UE8M0)
    for t in range(2):
        for h in range(7):
            for b in range(4):
                k = int((word[t, h] >> (8 * b)) & 0xFF) - 127
                assert k == _pow2_ceil_exp_f64(s32[t, h, b])


def test_qf8_rejects_bad_arguments():
    cfg = dict(synth.QNR_FORWARD, N=2, Hq=3, Hpad=3)
    q, w, pos, cache = synth.qnr_inputs(cfg)
    with pytest.raises(oracle.OracleError):
        oracle.qnorm_rope_fp8(q, w, pos, cache, 2, 1e-6)
    with pytest.raises(oracle.OracleError):
        oracle.qnorm_rope_fp8(q, w, pos, cache, 3, 1e-6, quant_eps=0.0)
    with pytest.raises(oracle.OracleError):
        oracle.qnorm_rope_fp8(q, w, pos, cache, 3, 1e-6, scale_fmt=2)


# ------------------------------------------------ kv path, bf16 full cache

def _small_full(N=10, ns=23, row=520, seed=4, holes=()):
    kv = synth.normal_bf16((N, 512), seed, synth.T_KV)
    pos = synth.uniform_positions(N, 512, seed)
    slots = synth.slot_permutation(N, ns, seed)
    for i in holes:
        slots[i] = -1
    cache = synth.cos_sin_cache(512)
    full = np.full((ns, row), 0xAAAA, np.uint16)
    oracle.kv_rope_insert_full(kv, pos, cache, slots, full)
    return kv, pos, slots, cache, full


def test_kvf_rows_land_on_their_slots_only():
    kv, pos, slots, cache, full = _small_full(holes=(1, 6))
    live = slots[slots >= 0]
    untouched = np.setdiff1d(np.arange(full.shape[0]), live)
    assert (full[untouched] == 0xAAAA).all()
    assert (full[:, 512:] == 0xAAAA).all()  # the row gap is never written
    for t, s in enumerate(slots):
        if s >= 0:
            assert (full[s, :448] == kv[t, :448]).all()


def test_kvf_fp64_forward_rotation_within_one_rounding():
    kv, pos, slots, cache, full = _small_full()
    ang = rope_angles(pos)
    for t, s in enumerate(slots):
        x = bf16_value(kv[t]).astype(np.float64)
        ref = _rotate64(x, ang[t], 1)
        got = bf16_value(full[s, :512]).astype(np.float64)
        assert (np.abs(got - ref) <= _rounding_bound(x, ref)).all()


def test_kvf_agrees_with_the_quantized_cache():
    kv, pos, slots, cache, full = _small_full(N=8, ns=8)
    bs = 4
    k_cache = np.zeros((2, bs * 528), np.uint8)
    oracle.kv_rope_quant_insert(kv, pos, cache, slots, k_cache, bs)
    flat = k_cache.reshape(-1)
    for t, s in enumerate(slots):
        off = (s // bs) * bs * 528 + (s % bs) * 528
        sc = np.repeat(flat[off + 512:off + 528].view(np.float32).astype(np.float64), 128)
        deq = oracle.e4m3_to_f32(flat[off:off + 512]).astype(np.float64) * sc
        y = bf16_value(full[s, :512]).astype(np.float64)
        bound = 0.5 * e4m3_ulp(y / sc) * sc + 0.5 * _bf16_ulp(y) + 1e-30
        assert (np.abs(deq - y) <= bound).all()


def test_kvf_rejects_duplicate_and_out_of_range_slots():
    kv = synth.normal_bf16((3, 512), 1, synth.T_KV)
    pos = np.zeros(3, np.int64)
    cache = synth.cos_sin_cache(4)
    full = np.zeros((4, 512), np.uint16)
    with pytest.raises(oracle.OracleError):
        oracle.kv_rope_insert_full(kv, pos, cache, np.array([1, 3, 1], np.int64), full)
    with pytest.raises(oracle.OracleError):
        oracle.kv_rope_insert_full(kv, pos, cache, np.array([0, 1, 4], np.int64), full)
    with pytest.raises(oracle.OracleError):
        oracle.kv_rope_insert_full(kv, pos, cache, np.array([0, 1, 2], np.int64),
                                   np.zeros((4, 500), np.uint16))
    oracle.kv_rope_insert_full(kv, pos, cache, np.array([-1, 3, -1], np.int64), full)
