"""GPU parity of qnorm_rope_kv_rope_quant_insert (one launch for the q and kv
paths) vs the oracle, and bit-identity with the two separate entry points."""
import numpy as np
import pytest
import torch

import oracle
import rope_fp8_quant_amd as rq
from rope_fp8_quant_amd import synth
from tests.gpu_util import (DEV, Q_DEF_FRAC_BF16, SHAPES, assert_bits_equal, assert_codes_match,
                            assert_q_out_parity, dev, host, table_tokens)

pytestmark = pytest.mark.gpu

FMT = {"fp32": oracle.SCALE_FP32, "ue8m0": oracle.SCALE_UE8M0}


def fused_inputs(N, Hq, nb, bs, seed, max_pos=65536, holes=()):
    q = synth.normal_bf16((N, Hq, 512), seed, synth.T_Q, std=2.0)
    w = synth.uniform_bf16((512,), seed, synth.T_W, 0.5, 1.5)
    kv = synth.normal_bf16((N, 512), seed, synth.T_KV)
    pos = synth.uniform_positions(N, max_pos, seed)
    slots = synth.slot_permutation(N, nb * bs, seed)
    for i in holes:
        slots[i] = -1
    return q, w, kv, pos, slots, synth.cos_sin_cache(max_pos)


def run_fused(q, w, kv, pos, slots, cache, hpad, nb, bs, scale_fmt="fp32", stride=None):
    N = q.shape[0]
    stride = bs * 528 if stride is None else stride
    q_out = torch.empty((N, hpad, 512), dtype=torch.bfloat16, device=DEV)
    q_out.view(torch.int16).fill_(-1)
    k_cache = torch.full((nb, stride), 0xAA, dtype=torch.uint8, device=DEV)
    pd, cd = dev(pos), dev(cache)
    rq.qnorm_rope_kv_rope_quant_insert(dev(q), None if w is None else dev(w), dev(kv), pd, cd,
                                       dev(slots), q_out, k_cache, bs, 1e-6, scale_fmt)
    torch.cuda.synchronize()
    return host(q_out), host(k_cache)


def run_separate(q, w, kv, pos, slots, cache, hpad, nb, bs, scale_fmt="fp32", stride=None):
    N = q.shape[0]
    stride = bs * 528 if stride is None else stride
    q_out = torch.empty((N, hpad, 512), dtype=torch.bfloat16, device=DEV)
    k_cache = torch.full((nb, stride), 0xAA, dtype=torch.uint8, device=DEV)
    pd, cd = dev(pos), dev(cache)
    rq.qnorm_rope(dev(q), None if w is None else dev(w), pd, cd, q_out, 1e-6)
    rq.kv_rope_quant_insert(dev(kv), pd, cd, dev(slots), k_cache, bs, scale_fmt)
    torch.cuda.synchronize()
    return host(q_out), host(k_cache)


def check_fused(q, w, kv, pos, slots, cache, hpad, nb, bs, scale_fmt="fp32", stride=None,
                what="", max_frac=None):
    print(f"[case] fused {what} N={q.shape[0]} Hq={q.shape[1]} Hpad={hpad} fmt={scale_fmt}",
          flush=True)
    gq, gk = run_fused(q, w, kv, pos, slots, cache, hpad, nb, bs, scale_fmt, stride)
    stride_b = bs * 528 if stride is None else stride
    # the fused op is, by definition, both ops on the same positions
    assert_q_out_parity(gq, q, w, pos, cache, hpad, 1e-6, f"fused {what} q_out", max_frac)
    ek = oracle.kv_rope_quant_insert(kv, pos, cache, slots,
                                     np.full((nb, stride_b), 0xAA, np.uint8), bs, stride_b,
                                     FMT[scale_fmt])
    diff = gk != ek
    rec = np.zeros(ek.size, bool)
    for s in slots[slots >= 0]:
        off = (s // bs) * stride_b + (s % bs) * 528
        rec[off:off + 512] = True
    rec = rec.reshape(ek.shape)
    assert not (diff & ~rec).any(), "cache bytes outside the code fields differ"
    assert_codes_match(gk[rec], ek[rec], f"fused {what} cache codes")
    sq, sk = run_separate(q, w, kv, pos, slots, cache, hpad, nb, bs, scale_fmt, stride)
    assert (sq == gq).all() and (sk == gk).all(), "fused differs from the separate ops"


def test_fused_forward_full_size():
    # the forward workload: q [8192, 64, 512] -> 128 padded heads, kv [8192, 512]
    # into 256 blocks x 64 slots, positions 0..8191 shared by both paths
    cq = synth.QNR_FORWARD
    q, w, pos, cache = synth.qnr_inputs(cq)
    kv, kpos, slots, _ = synth.kvi_inputs(synth.KVI_FORWARD)
    assert (kpos == pos).all()
    check_fused(q, w, kv, pos, slots, cache, 128, 256, 64, what="forward",
                max_frac=Q_DEF_FRAC_BF16)


@pytest.mark.parametrize("scale_fmt", ["fp32", "ue8m0"])
@pytest.mark.parametrize("shape", SHAPES)
def test_fused_ragged_holes_no_weight(scale_fmt, shape):
    # one grid of 7 q rows and 1 kv row per token (Hpad 7)
    N = table_tokens(shape, 8)
    nb = -(-N // 16) + 2
    q, w, kv, pos, slots, cache = fused_inputs(N, 5, nb, 16, 70, holes=(0, 13, 36))
    check_fused(q, None, kv, pos, slots, cache, 7, nb, 16, scale_fmt, stride=16 * 528 + 48,
                what=f"ragged {shape}")


@pytest.mark.parametrize("N", synth.DECODE_NS)
def test_fused_decode_sizes(N):
    q, w, kv, pos, slots, cache = fused_inputs(N, 32, 4, 64, 80 + N)
    check_fused(q, w, kv, pos, slots, cache, 128, 4, 64, what="decode")


def test_qnorm_rope_in_place():
    # q_head_padded == Hq and contiguous: q_out may be q_in itself
    cfg = dict(synth.QNR_FORWARD, N=33, Hq=12, Hpad=12, seed=71)
    q, w, pos, cache = synth.qnr_inputs(cfg)
    qd = dev(q)
    rq.qnorm_rope(qd, dev(w), dev(pos), dev(cache), qd, 1e-6)
    torch.cuda.synchronize()
    assert_q_out_parity(host(qd), q, w, pos, cache, 12, 1e-6, "in-place q")
