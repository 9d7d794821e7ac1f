"""Pins for the oracle's indexer query path (CPU only): rotate-half RoPE with
the bf16 round trip, the per-head power-of-two e4m3 scale, and the weight fold.
"""
import numpy as np
import pytest

import oracle
from rope_fp8_quant_amd import synth
from tests.helpers import bf16_value, f32_bits, rope_angles, torch_bf16, torch_e4m3


def _bf16_head(seed, std=1.0):
    x = np.random.default_rng(seed).standard_normal(128).astype(np.float32) * std
    return bf16_value(torch_bf16(x))  # indexer inputs are bf16


def test_indexer_rope_nope_half_untouched_and_rotated_half_is_bf16():
    x = _bf16_head(1)
    y = oracle.indexer_rope(x, synth.cos_sin_cache(100)[41])
    assert (f32_bits(y[64:]) == f32_bits(x[64:])).all()
    assert (f32_bits(y[:64]) & 0xFFFF == 0).all()  # bf16 round trip
    assert not (f32_bits(y[:64]) == f32_bits(x[:64])).all()


def test_indexer_rope_position_zero_identity():
    x = _bf16_head(2)
    y = oracle.indexer_rope(x, synth.cos_sin_cache(2)[0])
    assert (f32_bits(y) == f32_bits(x)).all()


def test_indexer_rope_rotate_half_pairs_and_signs():
    # quarter turn: (x_i, x_{i+32}) -> (-x_{i+32}, x_i), exact
    row = np.concatenate([np.zeros(32), np.ones(32)]).astype(np.float32)
    x = _bf16_head(3)
    y = oracle.indexer_rope(x, row)
    assert (y[:32] == -x[32:64]).all() and (y[32:64] == x[:32]).all()
    # unit vectors pick out the columns: x = e_i gives y_i = c_i, y_{i+32} = s_i
    i = np.arange(32)
    row = np.concatenate([(i + 1) / 64.0, (i + 65) / 128.0]).astype(np.float32)
    for k in (0, 7, 31):
        x = np.zeros(128, np.float32)
        x[k] = 1.0
        y = oracle.indexer_rope(x, row)
        assert y[k] == row[k] and y[k + 32] == row[32 + k]
        assert np.count_nonzero(y) == 2


def test_indexer_rope_matches_fp64_within_bf16_rounding():
    positions = np.array([1, 5, 77, 1000, 4095])
    cache = synth.cos_sin_cache(4096)
    ang = rope_angles(positions)
    for n, p in enumerate(positions):
        x = _bf16_head(10 + n, std=2.0)
        y = oracle.indexer_rope(x, cache[p]).astype(np.float64)
        z = (x[:32].astype(np.float64) + 1j * x[32:64]) * np.exp(1j * ang[n])
        exact = np.concatenate([z.real, z.imag])
        # half a bf16 ulp of the result, plus the fp32 table and evaluation
        # error (below 2^-21 (|x_i| + |x_{i+32}|))
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - 7)
        pair = (np.abs(x[:32]) + np.abs(x[32:64])).astype(np.float64)
        tol = 0.5 * ulp + 2.0 ** -21 * np.concatenate([pair, pair])
        assert (np.abs(y[:64] - exact) <= tol).all()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_indexer_scale_is_pow2_ceiling_and_codes_are_exact_scaling(seed):
    x = _bf16_head(seed, std=3.0)
    row = synth.cos_sin_cache(64)[seed + 5]
    codes, w_out, qs = oracle.indexer_head(x, row, 1.0, 1.0)
    y = oracle.indexer_rope(x, row)
    t = np.float32(np.abs(y).max()) / np.float32(448.0)
    m, e = np.frexp(float(qs))
    assert m == 0.5 and qs / 2 < t <= qs
    assert (codes == torch_e4m3(y / qs)).all()  # division by a power of two is exact
    assert np.abs(oracle.e4m3_to_f32(codes)).max() <= 448.0


def test_indexer_weight_fold_order():
    x = _bf16_head(5)
    row = synth.cos_sin_cache(8)[3]
    # powers of two: every product exact, so the fold is w * q_scale * 2^-3 * 2
    codes, w_out, qs = oracle.indexer_head(x, row, 1.0, 2.0 ** -3, 2.0)
    assert w_out == np.float32(qs * 2.0 ** -2)
    # general values: left-to-right fp32 products, within 3 roundings of fp64
    for w, ss, hs in [(0.37, 128 ** -0.5, 1.0), (0.9, 0.1, 1.7)]:
        _, w_out, qs = oracle.indexer_head(x, row, w, ss, hs)
        exact = float(np.float32(w)) * float(qs) * float(np.float32(ss)) * float(np.float32(hs))
        assert abs(float(w_out) - exact) <= 3 * 2.0 ** -24 * abs(exact)
        # and the order is the printed one: ((w * q) * ss) * hs
        ref = ((np.float32(w) * np.float32(qs)) * np.float32(ss)) * np.float32(hs)
        assert f32_bits(np.float32(w_out)) == f32_bits(ref)
    # q_scale is a power of two, so only (w * ss) * hs against w * (ss * hs)
    # can round differently; at w = 0.9, ss = 128^-0.5, hs = 1.7 they do (each
    # product of two fp32 values is exact in fp64, so every step below is one
    # fp32 rounding)
    w, ss, hs = np.float32(0.9), np.float32(128 ** -0.5), np.float32(1.7)
    _, w_out, qs = oracle.indexer_head(x, row, w, ss, hs)
    printed = np.float32(np.float32(np.float32(w * qs) * ss) * hs)
    other = np.float32(w * np.float32(qs * np.float32(ss * hs)))
    assert printed != other
    assert f32_bits(np.float32(w_out)) == f32_bits(printed)


def test_indexer_zero_head_uses_eps_floor():
    codes, w_out, qs = oracle.indexer_head(np.zeros(128, np.float32),
                                           synth.cos_sin_cache(4)[1], 0.5, 1.0, eps=1e-4)
    assert (codes == 0).all()
    t = np.float32(1e-4) / np.float32(448.0)
    assert qs / 2 < t <= qs


def test_indexer_op_is_per_head_composition_and_batch_invariant():
    N, H = 5, 6
    q = synth.normal_bf16((N, H, 128), 7, synth.T_Q)
    w = np.random.default_rng(7).uniform(0, 1, (N, H)).astype(np.float32)
    pos = synth.uniform_positions(N, 4096, 7)
    cache = synth.cos_sin_cache(4096)
    out, wo = oracle.indexer_q_rope_quant(q, pos, cache, w, 128 ** -0.5)
    for t in range(N):
        for h in range(H):
            c, wv, _ = oracle.indexer_head(bf16_value(q[t, h]), cache[pos[t]], w[t, h],
                                           128 ** -0.5)
            assert (out[t, h] == c).all() and f32_bits(np.float32(wv)) == f32_bits(wo[t, h])
    one, wone = oracle.indexer_q_rope_quant(q[2:3].copy(), pos[2:3].copy(), cache, w[2:3].copy(),
                                            128 ** -0.5)
    assert (one[0] == out[2]).all() and (wone[0] == wo[2]).all()
    bad = pos.copy()
    bad[0] = 4096
    with pytest.raises(oracle.OracleError):
        oracle.indexer_q_rope_quant(q, bad, cache, w, 128 ** -0.5)
