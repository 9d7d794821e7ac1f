"""GPU parity of inv_rope_fp8_quant (HIP path through the C ABI) vs the oracle."""
import numpy as np
import pytest
import torch

import oracle
import rope_fp8_quant_amd as rq
from rope_fp8_quant_amd import synth
from tests.gpu_util import (DEV, SHAPES, assert_bits_equal, assert_codes_match, dev, host,
                            table_tokens)

pytestmark = pytest.mark.gpu

FMT = {"fp32": oracle.SCALE_FP32, "ue8m0": oracle.SCALE_UE8M0}


def run_gpu(o_bits, pos, cache, hpg, scale_fmt="fp32", eps=1e-10):
    N, H, _ = o_bits.shape
    out, sc = rq.empty_inv_rope_fp8_quant_outputs(N, H, hpg, DEV, scale_fmt)
    out.fill_(0xCD)
    sc.fill_(-7)
    rq.inv_rope_fp8_quant(dev(o_bits), dev(pos), dev(cache), hpg, out, sc, scale_fmt, eps)
    torch.cuda.synchronize()
    return host(out), host(sc)


def check(o_bits, pos, cache, hpg, scale_fmt="fp32", eps=1e-10, what=""):
    print(f"[case] irq {what} N={o_bits.shape[0]} H={o_bits.shape[1]} hpg={hpg} "
          f"fmt={scale_fmt}", flush=True)
    out, sc = run_gpu(o_bits, pos, cache, hpg, scale_fmt, eps)
    eo, es = oracle.inv_rope_fp8_quant(o_bits, pos, cache, hpg, FMT[scale_fmt], eps)
    assert_bits_equal(sc, es, f"{what} scales")
    assert_codes_match(out, eo, f"{what} codes")
    return out, sc


@pytest.mark.parametrize("scale_fmt", ["fp32", "ue8m0"])
def test_irq_tiny(scale_fmt):
    o, pos, cache = synth.irq_inputs(synth.IRQ_TINY)
    check(o, pos, cache, 8, scale_fmt, what="tiny")


# The pages' (heads, groups) grid, plus 48 heads in groups of 6, at a size in
# each entry of the launch table.
@pytest.mark.parametrize("H,G", [(64, 8), (32, 4), (128, 8), (24, 4), (48, 8)])
@pytest.mark.parametrize("shape", SHAPES)
def test_irq_head_group_grid(H, G, shape):
    N = table_tokens(shape, H)
    cfg = dict(synth.IRQ_TINY, N=N, H=H, hpg=H // G, max_pos=65536, seed=H * 10 + G)
    o, pos, cache = synth.irq_inputs(cfg)
    check(o, pos, cache, H // G, what=f"grid {shape}")


def test_irq_prefill_full_size():
    o, pos, cache = synth.irq_inputs(synth.IRQ_PREFILL)
    check(o, pos, cache, 8, what="prefill 16384x32")


def test_irq_prefill_ue8m0_token_slice():
    o, pos, cache = synth.irq_inputs(synth.IRQ_PREFILL, 8192, 9216)
    check(o, pos, cache, 8, "ue8m0", what="prefill slice")


def test_irq_irregular_full_size():
    o, pos, cache = synth.irq_inputs(synth.IRQ_IRREGULAR)
    check(o, pos, cache, 6, what="irregular 4096x48")


@pytest.mark.parametrize("N", synth.DECODE_NS)
def test_irq_decode_sizes(N):
    cfg = dict(synth.IRQ_TINY, N=N, H=32, hpg=8, max_pos=65536, seed=40 + N)
    o, pos, cache = synth.irq_inputs(cfg)
    check(o, pos, cache, 8, what="decode")


@pytest.mark.parametrize("scale_fmt", ["fp32", "ue8m0"])
def test_irq_launch_table_entries_bit_identical(scale_fmt):
    # 613 tokens x 32 heads take the prefill entry of the launch table; the
    # same tokens in two calls of under 512 tokens take the one-head-per-wave
    # entry (256-thread workgroups; decode sizes use its 64-thread ones)
    cfg = dict(synth.IRQ_TINY, N=613, H=32, hpg=8, max_pos=65536, seed=77)
    o, pos, cache = synth.irq_inputs(cfg)
    print(f"[case] irq launch-table entries {scale_fmt}", flush=True)
    full, fsc = run_gpu(o, pos, cache, 8, scale_fmt)
    for t0, t1 in ((0, 307), (307, 613)):
        part, psc = run_gpu(o[t0:t1].copy(), pos[t0:t1].copy(), cache, 8, scale_fmt)
        assert (part == full[:, t0:t1]).all()
        assert (psc.view(np.uint32) == fsc[:, t0:t1].view(np.uint32)).all()


def test_irq_batch_invariance():
    cfg = dict(synth.IRQ_TINY, N=40, H=32, hpg=8, max_pos=65536, seed=78)
    o, pos, cache = synth.irq_inputs(cfg)
    full, fsc = run_gpu(o, pos, cache, 8)
    for t in (0, 17, 39):
        one, osc = run_gpu(o[t:t + 1].copy(), pos[t:t + 1].copy(), cache, 8)
        assert (one[:, 0] == full[:, t]).all()
        assert (osc[:, 0].view(np.uint32) == fsc[:, t].view(np.uint32)).all()


@pytest.mark.parametrize("scale_fmt", ["fp32", "ue8m0"])
def test_irq_strided_input_token_major_output(scale_fmt):
    N, H, hpg = 19, 16, 4
    G = H // hpg
    cfg = dict(synth.IRQ_TINY, N=N, H=H, hpg=hpg, seed=79)
    o, pos, cache = synth.irq_inputs(cfg)
    print(f"[case] irq strided/token-major fmt={scale_fmt}", flush=True)
    big = torch.zeros((N, H, 1024), dtype=torch.bfloat16, device=DEV)
    big[:, :, 256:768] = dev(o)
    o_view = big[:, :, 256:768]  # strides (H*1024, 1024, 1)
    out_tok = torch.full((N, H, 512), 0xCD, dtype=torch.uint8, device=DEV)
    out_view = out_tok.view(N, G, hpg * 512).transpose(0, 1)
    if scale_fmt == "fp32":
        sc_tok = torch.full((N, H * 4), -7.0, dtype=torch.float32, device=DEV)
        sc_view = sc_tok.view(N, G, hpg * 4).transpose(0, 1)
    else:
        sc_tok = torch.full((N, H), -7, dtype=torch.int32, device=DEV)
        sc_view = sc_tok.view(N, G, hpg).transpose(0, 1)
    rq.inv_rope_fp8_quant(o_view, dev(pos), dev(cache), hpg, out_view, sc_view, scale_fmt)
    torch.cuda.synchronize()
    eo, es = oracle.inv_rope_fp8_quant(o, pos, cache, hpg, FMT[scale_fmt], layout="token")
    assert_bits_equal(host(sc_tok), es, "token-major scales")
    assert_codes_match(host(out_tok), eo, "token-major codes")


def test_irq_writes_nothing_outside_outputs():
    N, H, hpg = 33, 24, 6
    G = H // hpg
    cfg = dict(synth.IRQ_TINY, N=N, H=H, hpg=hpg, seed=80)
    o, pos, cache = synth.irq_inputs(cfg)
    print("[case] irq guard bytes", flush=True)
    pad = 4096
    ob = torch.full((2 * pad + G * N * hpg * 512,), 0xA5, dtype=torch.uint8, device=DEV)
    sb = torch.full((2 * pad + G * N * hpg * 4,), 1234.5, dtype=torch.float32, device=DEV)
    out = ob[pad:pad + G * N * hpg * 512].view(G, N, hpg * 512)
    sc = sb[pad:pad + G * N * hpg * 4].view(G, N, hpg * 4)
    rq.inv_rope_fp8_quant(dev(o), dev(pos), dev(cache), hpg, out, sc)
    torch.cuda.synchronize()
    obh, sbh = host(ob), host(sb)
    assert (obh[:pad] == 0xA5).all() and (obh[-pad:] == 0xA5).all()
    assert (sbh[:pad] == 1234.5).all() and (sbh[-pad:] == 1234.5).all()
    eo, es = oracle.inv_rope_fp8_quant(o, pos, cache, hpg)
    assert_bits_equal(sbh[pad:-pad].reshape(es.shape), es, "guarded scales")
    assert_codes_match(obh[pad:-pad], eo, "guarded codes")


@pytest.mark.parametrize("scale_fmt", ["fp32", "ue8m0"])
def test_irq_degenerate_values(scale_fmt):
    # zeros of both signs, all-zero heads (amax floor eps), huge and tiny
    # magnitudes, bf16 subnormals, and every finite bf16 value in [-448, 448]
    # quantized with scale exactly 1 (a 448 in each block).
    rng = np.random.default_rng(81)
    allbf = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = (allbf.astype(np.uint32) << 16).view(np.float32)
    probe = allbf[np.isfinite(vals) & (np.abs(vals) <= 448)]
    per_block = 127
    nblk = -(-probe.size // per_block)
    blocks = np.zeros((nblk, 128), np.uint16)
    flat = np.concatenate([probe, np.zeros(nblk * per_block - probe.size, np.uint16)])
    blocks[:, :per_block] = flat.reshape(nblk, per_block)
    blocks[:, 127] = 0x43E0  # 448.0
    heads = blocks.reshape(-1, 512) if nblk % 4 == 0 else np.concatenate(
        [blocks, np.tile(blocks[:1], (4 - nblk % 4, 1))]).reshape(-1, 512)
    special = np.zeros((8, 512), np.uint16)
    special[1] = 0x8000  # all -0
    special[2] = synth.f32_to_bf16_bits(rng.standard_normal(512).astype(np.float32) * 1e30)
    special[3] = synth.f32_to_bf16_bits(rng.standard_normal(512).astype(np.float32) * 1e-30)
    special[4] = rng.integers(1, 0x80, size=512).astype(np.uint16)  # bf16 subnormals
    special[5] = synth.f32_to_bf16_bits(np.full(512, -3.0, np.float32))
    special[6, ::7] = 0x4000  # sparse 2.0
    special[7] = synth.f32_to_bf16_bits(rng.standard_normal(512).astype(np.float32))
    special[7, :256] = 0
    allh = np.concatenate([heads, special])
    H = 8
    n = -(-allh.shape[0] // H)
    allh = np.concatenate([allh, np.zeros((n * H - allh.shape[0], 512), np.uint16)])
    o = allh.reshape(n, H, 512)
    pos = np.zeros(n, np.int64)  # position 0: cos 1, sin 0
    pos[n // 2:] = np.arange(n - n // 2) * 37 % 4096
    cache = synth.cos_sin_cache(4096)
    check(o, pos, cache, 4, scale_fmt, what="degenerate")


@pytest.mark.parametrize("scale_fmt", ["fp32", "ue8m0"])
def test_irq_bad_position_poisons_only_its_token(scale_fmt):
    cfg = dict(synth.IRQ_TINY, N=12, H=8, hpg=4, seed=82)
    o, pos, cache = synth.irq_inputs(cfg)
    bad = pos.copy()
    bad[5] = cache.shape[0]
    bad[9] = -1
    print(f"[case] irq bad positions fmt={scale_fmt}", flush=True)
    out, sc = run_gpu(o, bad, cache, 4, scale_fmt)
    good = [t for t in range(12) if t not in (5, 9)]
    eo, es = oracle.inv_rope_fp8_quant(o[good].copy(), pos[good].copy(), cache, 4,
                                       FMT[scale_fmt])
    assert (out[:, good] == eo).all()
    assert_bits_equal(sc[:, good], es, "good tokens")
    for t in (5, 9):  # NaN scales make every dequantized value NaN
        if scale_fmt == "fp32":
            assert np.isnan(sc[:, t]).all()
        else:
            assert (sc[:, t] == 0xFFFFFFFF).all()


def _half_turn_cache():
    """Row 0: cos 1, sin 0.  Row 1: cos = sin = fp32(sqrt(1/2)) in every column."""
    cache = np.zeros((2, 64), np.float32)
    cache[0, :32] = 1.0
    cache[1, :] = np.float32(np.sqrt(0.5))
    return cache


@pytest.mark.parametrize("scale_fmt", ["fp32", "ue8m0"])
def test_irq_rotated_pair_near_and_past_overflow(scale_fmt):
    # The last GPT-J pair (dims 510, 511) of some heads is set to (v, v) and
    # rotated by 45 degrees: e' = (e + o) * 0.7071.  v = 1.5 * 2^126 stays
    # finite (1.06 * 2^127); v = the bf16 maximum overflows to +inf, giving
    # block 3 an infinite maximum (scale +inf, or UE8M0 byte 0xFF).  Scales
    # must match the oracle bit for bit, and every code but the infinite
    # value's (unspecified) to the code bar.
    N, H, hpg = 8, 8, 4
    G = H // hpg
    o = synth.normal_bf16((N, H, 512), 83, synth.T_O)
    pos = np.array([0, 1, 1, 0, 1, 1, 1, 0], np.int64)
    near = [(1, 0), (2, 5), (4, 7)]
    past = [(1, 3), (5, 0), (6, 6)]
    for t, h in near:
        o[t, h, 510:512] = 0x7EC0  # 1.5 * 2^126
    for t, h in past:
        o[t, h, 510:512] = 0x7F7F  # the largest finite bf16
    cache = _half_turn_cache()
    print(f"[case] irq rotated overflow fmt={scale_fmt}", flush=True)
    out, sc = run_gpu(o, pos, cache, hpg, scale_fmt)
    eo, es = oracle.inv_rope_fp8_quant(o, pos, cache, hpg, FMT[scale_fmt])
    assert_bits_equal(sc, es, "overflow scales")
    if scale_fmt == "fp32":
        assert all(np.isinf(es[h // hpg, t, (h % hpg) * 4 + 3]) for t, h in past)
    else:
        assert all(es[h // hpg, t, h % hpg] >> 24 == 0xFF for t, h in past)
    keep = np.ones(eo.shape, bool)
    for t, h in past:
        keep[h // hpg, t, (h % hpg) * 512 + 510] = False  # the infinite value
    assert_codes_match(out[keep], eo[keep], "overflow codes")


def test_irq_zero_tokens_is_a_no_op():
    out, sc = rq.empty_inv_rope_fp8_quant_outputs(0, 8, 8, DEV)
    o = torch.empty((0, 8, 512), dtype=torch.bfloat16, device=DEV)
    pos = torch.empty((0,), dtype=torch.int64, device=DEV)
    cache = dev(synth.cos_sin_cache(4))
    rq.inv_rope_fp8_quant(o, pos, cache, 8, out, sc)
    torch.cuda.synchronize()
