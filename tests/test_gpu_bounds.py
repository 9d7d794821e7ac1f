"""No kernel writes outside its outputs.

Every output here is a prefix view of a larger buffer filled with a sentinel;
the guard band after the view must come back untouched.  The sizes are ragged
so that, in every launch shape, the grid holds waves past the last unit (the
tail waves must store nothing), and the results inside the views are checked
against the oracle as well.
"""
import numpy as np
import pytest
import torch

import oracle
import rope_fp8_quant_amd as rq
from rope_fp8_quant_amd import synth
from tests.gpu_util import DEV, assert_bits_equal, assert_codes_match, dev, host

pytestmark = pytest.mark.gpu

GUARD = 64 * 1024  # bytes after each output
THREADS = [64, 128, 256]


@pytest.fixture(autouse=True)
def _table_launch():
    rq.set_block_threads(0)
    yield
    rq.set_block_threads(0)


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


def ragged_irq(N=37, H=24, hpg=6, seed=150):
    cfg = dict(synth.IRQ_TINY, N=N, H=H, hpg=hpg, max_pos=65536, seed=seed)
    return synth.irq_inputs(cfg)


@pytest.mark.parametrize("threads", THREADS)
@pytest.mark.parametrize("scale_fmt", ["fp32", "ue8m0"])
def test_irq_tail_waves_write_nothing(threads, scale_fmt):
    rq.set_block_threads(threads)
    o, pos, cache = ragged_irq()
    N, H, hpg = 37, 24, 6
    G = H // hpg
    print(f"[case] irq guard threads={threads} {scale_fmt}", flush=True)
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


@pytest.mark.parametrize("threads", THREADS)
def test_irb_tail_waves_write_nothing(threads):
    rq.set_block_threads(threads)
    o, pos, cache = ragged_irq(seed=151)
    print(f"[case] inv_rope_bf16 guard threads={threads}", flush=True)
    out = Guarded((4, 37, 6 * 512), torch.bfloat16)
    rq.inv_rope_bf16(dev(o), dev(pos), dev(cache), 6, out.t)
    torch.cuda.synchronize()
    assert out.guard_intact()
    assert_bits_equal(host(out.t), oracle.inv_rope_bf16(o, pos, cache, 6), "guarded bf16")


def ragged_q(seed):
    cfg = dict(synth.QNR_FORWARD, N=37, Hq=5, Hpad=7, seed=seed)
    return synth.qnr_inputs(cfg)


@pytest.mark.parametrize("threads", THREADS)
def test_qnr_tail_waves_write_nothing(threads):
    rq.set_block_threads(threads)
    q, w, pos, cache = ragged_q(152)
    print(f"[case] qnorm_rope guard threads={threads}", flush=True)
    out = Guarded((37, 7, 512), torch.bfloat16)
    rq.qnorm_rope(dev(q), dev(w), dev(pos), dev(cache), out.t, 1e-6)
    torch.cuda.synchronize()
    assert out.guard_intact()
    assert_bits_equal(host(out.t), oracle.qnorm_rope(q, w, pos, cache, 7, 1e-6), "guarded q")


@pytest.mark.parametrize("threads", THREADS)
@pytest.mark.parametrize("scale_fmt", ["fp32", "ue8m0"])
def test_qf8_tail_waves_write_nothing(threads, scale_fmt):
    rq.set_block_threads(threads)
    q, w, pos, cache = ragged_q(153)
    print(f"[case] qnorm_rope_fp8 guard threads={threads} {scale_fmt}", flush=True)
    codes = Guarded((37, 7, 512), torch.uint8)
    sc = Guarded((37, 7, 4) if scale_fmt == "fp32" else (37, 7),
                 torch.float32 if scale_fmt == "fp32" else torch.int32)
    rq.qnorm_rope_fp8(dev(q), dev(w), dev(pos), dev(cache), codes.t, sc.t, 1e-6, scale_fmt)
    torch.cuda.synchronize()
    assert codes.guard_intact() and sc.guard_intact()
    ec, es = oracle.qnorm_rope_fp8(q, w, pos, cache, 7, 1e-6, {"fp32": 0, "ue8m0": 1}[scale_fmt])
    assert_bits_equal(host(sc.t), es, "guarded q scales")
    assert_codes_match(host(codes.t), ec, "guarded q codes")


@pytest.mark.parametrize("threads", THREADS)
def test_kv_paths_tail_waves_write_nothing(threads):
    rq.set_block_threads(threads)
    N, nb, bs = 37, 3, 16
    kv = synth.normal_bf16((N, 512), 154, synth.T_KV)
    pos = synth.uniform_positions(N, 4096, 154)
    slots = synth.slot_permutation(N, nb * bs, 154)
    cache = synth.cos_sin_cache(4096)
    print(f"[case] kv paths guard threads={threads}", flush=True)
    k_cache = Guarded((nb, bs * 528), torch.uint8, fill_byte=0xAA)
    rq.kv_rope_quant_insert(dev(kv), dev(pos), dev(cache), dev(slots), k_cache.t, bs)
    full = Guarded((nb * bs, 512), torch.bfloat16, fill_byte=0xAA)
    rq.kv_rope_insert_full(dev(kv), dev(pos), dev(cache), dev(slots), full.t)
    torch.cuda.synchronize()
    assert k_cache.guard_intact() and full.guard_intact()
    exp = oracle.kv_rope_insert_full(kv, pos, cache, slots,
                                     np.full((nb * bs, 512), 0xAAAA, np.uint16))
    assert_bits_equal(host(full.t), exp, "guarded kv rows")


@pytest.mark.parametrize("threads", THREADS)
def test_indexer_tail_waves_write_nothing(threads):
    rq.set_block_threads(threads)
    N, H = 37, 5
    q = synth.normal_bf16((N, H, 128), 155, synth.T_Q)
    w = np.random.default_rng([155, 9]).uniform(0, 1, (N, H)).astype(np.float32)
    pos = synth.uniform_positions(N, 4096, 155)
    cache = synth.cos_sin_cache(4096)
    print(f"[case] indexer guard threads={threads}", flush=True)
    q8 = Guarded((N, H, 128), torch.uint8)
    wo = Guarded((N, H), torch.float32)
    rq.indexer_q_rope_quant(dev(q), dev(pos), dev(cache), dev(w), q8.t, wo.t, 128 ** -0.5)
    torch.cuda.synchronize()
    assert q8.guard_intact() and wo.guard_intact()
    ec, ew = oracle.indexer_q_rope_quant(q, pos, cache, w, 128 ** -0.5)
    assert_bits_equal(host(wo.t), ew, "guarded weights")
    assert_codes_match(host(q8.t), ec, "guarded indexer codes")
