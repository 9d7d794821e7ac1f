"""GPU parity of indexer_q_rope_quant (HIP path through the C ABI) vs the oracle."""
import numpy as np
import pytest
import torch

import oracle
import rope_fp8_quant_amd as rq
from rope_fp8_quant_amd import synth
from tests.gpu_util import (DEV, SHAPES, TABLE_ROWS, assert_bits_equal, assert_codes_match, dev,
                            host, table_tokens)

pytestmark = pytest.mark.gpu

SOFTMAX_SCALE = 128 ** -0.5


def idx_inputs(N, H, seed, max_pos=4096, pos=None):
    q = synth.normal_bf16((N, H, 128), seed, synth.T_Q)
    w = np.random.default_rng([seed, 9]).uniform(0, 1, (N, H)).astype(np.float32)
    if pos is None:
        pos = synth.uniform_positions(N, max_pos, seed)
    return q, w, pos, synth.cos_sin_cache(max_pos)


def idx_gpu(q, w, pos, cache, head_scale=1.0, eps=1e-10, q_dev=None, inplace=False):
    N, H, _ = q.shape
    q_fp8 = torch.full((N, H, 128), 0xCD, dtype=torch.uint8, device=DEV)
    wd = dev(w)
    wo = wd if inplace else torch.full((N, H), -3.0, dtype=torch.float32, device=DEV)
    rq.indexer_q_rope_quant(dev(q) if q_dev is None else q_dev, dev(pos), dev(cache), wd, q_fp8,
                            wo, SOFTMAX_SCALE, head_scale, eps)
    torch.cuda.synchronize()
    return host(q_fp8), host(wo)


def idx_check(q, w, pos, cache, what, head_scale=1.0, eps=1e-10, **kw):
    print(f"[case] indexer {what} N={q.shape[0]} H={q.shape[1]}", flush=True)
    got, gw = idx_gpu(q, w, pos, cache, head_scale, eps, **kw)
    exp, ew = oracle.indexer_q_rope_quant(q, pos, cache, w, SOFTMAX_SCALE, head_scale, eps)
    assert_bits_equal(gw, ew, f"indexer {what} weights")
    assert_codes_match(got, exp, f"indexer {what} codes")


def test_indexer_full_size():
    # 4096 tokens x 64 heads x 128 dims, weights ~U(0,1), softmax scale 128^-0.5
    idx_check(*idx_inputs(4096, 64, 55, max_pos=4096, pos=np.arange(4096, dtype=np.int64)),
              "4096x64x128")


# A wave takes two 4-head items, so a token of H heads is 2 * ceil(H / 4)
# rows of the launch table.
@pytest.mark.parametrize("shape", SHAPES)
def test_indexer_ragged(shape):
    idx_check(*idx_inputs(table_tokens(shape, 2), 5, 56, max_pos=65536), f"ragged {shape}")


@pytest.mark.parametrize("N", synth.DECODE_NS)
def test_indexer_decode_sizes(N):
    idx_check(*idx_inputs(N, 64, 60 + N, max_pos=65536), "decode", head_scale=0.75)


def test_indexer_strided_input_and_in_place_weights():
    q, w, pos, cache = idx_inputs(19, 12, 57)
    big = torch.zeros((19, 12, 384), dtype=torch.bfloat16, device=DEV)
    big[:, :, 128:256] = dev(q)
    print("[case] indexer strided + in-place", flush=True)
    got, gw = idx_gpu(q, w, pos, cache, q_dev=big[:, :, 128:256], inplace=True)
    exp, ew = oracle.indexer_q_rope_quant(q, pos, cache, w, SOFTMAX_SCALE)
    assert_bits_equal(gw, ew, "in-place weights")
    assert_codes_match(got, exp, "strided codes")


@pytest.mark.parametrize("shape", SHAPES)
def test_indexer_strided_outputs_partial_item(shape):
    # 7 heads: every token's second 4-head item holds 3 heads.  Codes rows
    # padded to 192 bytes, weight rows to 10 and 12 floats; the padding must
    # come back untouched.
    N, H = table_tokens(shape, 2, base=41), 7
    q, w, pos, cache = idx_inputs(N, H, 62, max_pos=65536)
    q8_big = torch.full((N, H, 192), 0xCD, dtype=torch.uint8, device=DEV)
    w_big = torch.full((N, 10), -7.0, dtype=torch.float32, device=DEV)
    w_big[:, :H] = dev(w)
    wo_big = torch.full((N, 12), -3.0, dtype=torch.float32, device=DEV)
    print(f"[case] indexer strided outputs {shape}", flush=True)
    rq.indexer_q_rope_quant(dev(q), dev(pos), dev(cache), w_big[:, :H], q8_big[:, :, :128],
                            wo_big[:, :H], SOFTMAX_SCALE, 0.5)
    torch.cuda.synchronize()
    exp, ew = oracle.indexer_q_rope_quant(q, pos, cache, w, SOFTMAX_SCALE, 0.5)
    g8, gw = host(q8_big), host(wo_big)
    assert_bits_equal(gw[:, :H], ew, "strided weights")
    assert_codes_match(g8[:, :, :128], exp, "strided codes")
    assert (g8[:, :, 128:] == 0xCD).all() and (gw[:, H:] == -3.0).all()
    assert (host(w_big)[:, H:] == -7.0).all()


def test_indexer_degenerate_heads():
    rng = np.random.default_rng(58)
    q = np.zeros((4, 8, 128), np.uint16)
    q[0, 1] = 0x8000
    q[1, 0] = synth.f32_to_bf16_bits(np.full(128, -2.5, np.float32))
    q[1, 2] = synth.f32_to_bf16_bits(rng.standard_normal(128).astype(np.float32) * 1e20)
    q[2, 3] = synth.f32_to_bf16_bits(rng.standard_normal(128).astype(np.float32) * 1e-20)
    q[2, 4] = rng.integers(1, 0x80, size=128).astype(np.uint16)  # bf16 subnormals
    q[3] = synth.f32_to_bf16_bits(rng.standard_normal((8, 128)).astype(np.float32))
    q[3, 5, :64] = 0
    w = rng.uniform(0, 1, (4, 8)).astype(np.float32)
    pos = np.array([0, 3, 1000, 4095], np.int64)
    for eps in (1e-10, 1e-4):
        idx_check(q, w, pos, synth.cos_sin_cache(4096), f"degenerate eps={eps}", eps=eps)


def test_indexer_rotated_pair_near_and_past_overflow():
    # Rotate-half pair (i, i+32) = (v, -v) at 45 degrees: r0 = (v + v) * 0.7071.
    # v = 1.5 * 2^126 stays finite; v = the bf16 maximum overflows, so the
    # head's maximum is +inf: q_scale 2^128 = inf, folded weight +inf, finite
    # values scaled by 2^-128.  Weights and every code but the infinite
    # value's (unspecified) must match the oracle.
    N, H = 4, 8
    q, w, _, _ = idx_inputs(N, H, 63)
    pos = np.array([1, 0, 1, 1], np.int64)
    cache = np.zeros((2, 64), np.float32)
    cache[0, :32] = 1.0
    cache[1, :] = np.float32(np.sqrt(0.5))
    q[0, 2, 5], q[0, 2, 37] = 0x7EC0, 0xFEC0   # 1.5 * 2^126, negated
    q[2, 6, 9], q[2, 6, 41] = 0x7F7F, 0xFF7F   # the bf16 maximum, negated
    q[3, 1, 0], q[3, 1, 32] = 0x7F7F, 0xFF7F
    print("[case] indexer rotated overflow", flush=True)
    got, gw = idx_gpu(q, w, pos, cache)
    exp, ew = oracle.indexer_q_rope_quant(q, pos, cache, w, SOFTMAX_SCALE)
    assert_bits_equal(gw, ew, "overflow weights")
    assert np.isinf(ew[2, 6]) and np.isinf(ew[3, 1]) and np.isfinite(ew[0, 2])
    keep = np.ones(exp.shape, bool)
    keep[2, 6, 9] = keep[3, 1, 0] = False  # the infinite values
    assert_codes_match(got[keep], exp[keep], "overflow codes")


def test_indexer_bad_position_gives_nan_weight():
    q, w, pos, cache = idx_inputs(6, 4, 59)
    bad = pos.copy()
    bad[3] = cache.shape[0]
    got, gw = idx_gpu(q, w, bad, cache)
    good = [0, 1, 2, 4, 5]
    exp, ew = oracle.indexer_q_rope_quant(q[good].copy(), pos[good].copy(), cache,
                                          w[good].copy(), SOFTMAX_SCALE)
    assert (got[good] == exp).all() and (gw[good] == ew).all()
    assert np.isnan(gw[3]).all()


def test_indexer_launch_table_entries_bit_identical():
    # 1031 tokens x 64 heads (16 four-head items each, 16496 in all) take the
    # prefill entry of the launch table; the same tokens in two calls of
    # under 1024 tokens take the 64-thread entry
    q, w, pos, cache = idx_inputs(1031, 64, 61, max_pos=65536)
    assert 1031 * 16 >= TABLE_ROWS > 516 * 16
    print("[case] indexer launch-table entries", flush=True)
    full, fw = idx_gpu(q, w, pos, cache)
    for t0, t1 in ((0, 515), (515, 1031)):
        part, pw = idx_gpu(q[t0:t1].copy(), w[t0:t1].copy(), pos[t0:t1].copy(), cache)
        assert (part == full[t0:t1]).all()
        assert (pw.view(np.uint32) == fw[t0:t1].view(np.uint32)).all()
