"""No kernel writes outside its outputs.

Every output here is a prefix view of a larger buffer filled with a sentinel;
the guard band after the view must come back untouched.  Each case runs at a
size in each entry of the launch table, ragged so that the grid holds rows
and waves past the last unit (they must store nothing), and the results
inside the views are checked against the oracle as well.
"""
import numpy as np
import pytest
import torch

import oracle
import rope_fp8_quant_amd as rq
from rope_fp8_quant_amd import synth
from tests.gpu_util import (DEV, SHAPES, assert_bits_equal, assert_codes_match,
                            assert_q_fp8_parity, assert_q_out_parity, dev, host, table_tokens)

pytestmark = pytest.mark.gpu

GUARD = 64 * 1024  # bytes after each output


class Guarded:
    """A tensor of `shape` / `dtype` at the front of a sentinel-filled buffer."""

    def __init__(self, shape, dtype, fill_byte=0x5A):
        elem = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape))
        self.nbytes = n * elem
        self.raw = torch.full((self.nbytes + GUARD,), fill_byte, dtype=torch.uint8, device=DEV)
        self.fill = fill_byte
        self.t = self.raw[:self.nbytes].view(dtype).view(shape)

    def guard_intact(self):
        tail = host(self.raw[self.nbytes:])
        return bool((tail == self.fill).all())


# 18 heads in 3 groups of 6: with an odd token count the unit count is 2 mod 4,
# so the last wave and workgroup are part-filled in either table entry
H_IRQ, HPG_IRQ = 18, 6


def ragged_irq(shape, seed):
    N = table_tokens(shape, H_IRQ)
    N += 1 - N % 2  # odd
    cfg = dict(synth.IRQ_TINY, N=N, H=H_IRQ, hpg=HPG_IRQ, max_pos=65536, seed=seed)
    return synth.irq_inputs(cfg)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("scale_fmt", ["fp32", "ue8m0"])
def test_irq_tail_waves_write_nothing(shape, scale_fmt):
    o, pos, cache = ragged_irq(shape, 150)
    N, H, hpg = o.shape[0], H_IRQ, HPG_IRQ
    G = H // hpg
    print(f"[case] irq guard {shape} N={N} {scale_fmt}", flush=True)
    out = Guarded((G, N, hpg * 512), torch.uint8)
    per = 4 * hpg if scale_fmt == "fp32" else hpg
    sc = Guarded((G, N, per), torch.float32 if scale_fmt == "fp32" else torch.int32)
    rq.inv_rope_fp8_quant(dev(o), dev(pos), dev(cache), hpg, out.t, sc.t, scale_fmt)
    torch.cuda.synchronize()
    assert out.guard_intact() and sc.guard_intact()
    eo, es = oracle.inv_rope_fp8_quant(o, pos, cache, hpg,
                                       {"fp32": 0, "ue8m0": 1}[scale_fmt])
    assert_bits_equal(host(sc.t), es, "guarded scales")
    assert_codes_match(host(out.t), eo, "guarded codes")


@pytest.mark.parametrize("shape", SHAPES)
def test_irb_tail_waves_write_nothing(shape):
    o, pos, cache = ragged_irq(shape, 151)
    N = o.shape[0]
    print(f"[case] inv_rope_bf16 guard {shape} N={N}", flush=True)
    out = Guarded((H_IRQ // HPG_IRQ, N, HPG_IRQ * 512), torch.bfloat16)
    rq.inv_rope_bf16(dev(o), dev(pos), dev(cache), HPG_IRQ, out.t)
    torch.cuda.synchronize()
    assert out.guard_intact()
    assert_bits_equal(host(out.t), oracle.inv_rope_bf16(o, pos, cache, HPG_IRQ), "guarded bf16")


def ragged_q(shape, seed):
    # Hpad 7: the unit count is not a multiple of 4 in either entry
    cfg = dict(synth.QNR_FORWARD, N=table_tokens(shape, 7), Hq=5, Hpad=7, seed=seed)
    return synth.qnr_inputs(cfg)


@pytest.mark.parametrize("shape", SHAPES)
def test_qnr_tail_waves_write_nothing(shape):
    q, w, pos, cache = ragged_q(shape, 152)
    N = q.shape[0]
    print(f"[case] qnorm_rope guard {shape} N={N}", flush=True)
    out = Guarded((N, 7, 512), torch.bfloat16)
    rq.qnorm_rope(dev(q), dev(w), dev(pos), dev(cache), out.t, 1e-6)
    torch.cuda.synchronize()
    assert out.guard_intact()
    assert_q_out_parity(host(out.t), q, w, pos, cache, 7, 1e-6, "guarded q")


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("scale_fmt", ["fp32", "ue8m0"])
def test_qf8_tail_waves_write_nothing(shape, scale_fmt):
    q, w, pos, cache = ragged_q(shape, 153)
    N = q.shape[0]
    print(f"[case] qnorm_rope_fp8 guard {shape} N={N} {scale_fmt}", flush=True)
    codes = Guarded((N, 7, 512), torch.uint8)
    sc = Guarded((N, 7, 4) if scale_fmt == "fp32" else (N, 7),
                 torch.float32 if scale_fmt == "fp32" else torch.int32)
    rq.qnorm_rope_fp8(dev(q), dev(w), dev(pos), dev(cache), codes.t, sc.t, 1e-6, scale_fmt)
    torch.cuda.synchronize()
    assert codes.guard_intact() and sc.guard_intact()
    assert_q_fp8_parity(host(codes.t), host(sc.t), q, w, pos, cache, 7, 1e-6, scale_fmt,
                        "guarded q")


@pytest.mark.parametrize("shape", SHAPES)
def test_kv_paths_tail_waves_write_nothing(shape):
    N, bs = table_tokens(shape, 1), 16
    nb = -(-N // bs)
    kv = synth.normal_bf16((N, 512), 154, synth.T_KV)
    pos = synth.uniform_positions(N, 4096, 154)
    slots = synth.slot_permutation(N, nb * bs, 154)
    cache = synth.cos_sin_cache(4096)
    print(f"[case] kv paths guard {shape} N={N}", flush=True)
    k_cache = Guarded((nb, bs * 528), torch.uint8, fill_byte=0xAA)
    rq.kv_rope_quant_insert(dev(kv), dev(pos), dev(cache), dev(slots), k_cache.t, bs)
    full = Guarded((nb * bs, 512), torch.bfloat16, fill_byte=0xAA)
    rq.kv_rope_insert_full(dev(kv), dev(pos), dev(cache), dev(slots), full.t)
    torch.cuda.synchronize()
    assert k_cache.guard_intact() and full.guard_intact()
    exp = oracle.kv_rope_insert_full(kv, pos, cache, slots,
                                     np.full((nb * bs, 512), 0xAAAA, np.uint16))
    assert_bits_equal(host(full.t), exp, "guarded kv rows")


@pytest.mark.parametrize("shape", SHAPES)
def test_indexer_tail_waves_write_nothing(shape):
    # 5 heads: two 4-head items per token, the second holding one head; four
    # rows per wave of two items, so 4 rows per token
    N, H = table_tokens(shape, 2), 5  # ceil(5/4) four-head items per token
    q = synth.normal_bf16((N, H, 128), 155, synth.T_Q)
    w = np.random.default_rng([155, 9]).uniform(0, 1, (N, H)).astype(np.float32)
    pos = synth.uniform_positions(N, 4096, 155)
    cache = synth.cos_sin_cache(4096)
    print(f"[case] indexer guard {shape} N={N}", flush=True)
    q8 = Guarded((N, H, 128), torch.uint8)
    wo = Guarded((N, H), torch.float32)
    rq.indexer_q_rope_quant(dev(q), dev(pos), dev(cache), dev(w), q8.t, wo.t, 128 ** -0.5)
    torch.cuda.synchronize()
    assert q8.guard_intact() and wo.guard_intact()
    ec, ew = oracle.indexer_q_rope_quant(q, pos, cache, w, 128 ** -0.5)
    assert_bits_equal(host(wo.t), ew, "guarded weights")
    assert_codes_match(host(q8.t), ec, "guarded indexer codes")
