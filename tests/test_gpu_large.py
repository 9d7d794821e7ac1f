"""Tensors past 4 GiB: every offset the kernels form must stay exact there.

Each input is a small seeded block repeated along the tokens, so the result
for any token is the oracle's result on its block row at its own position;
the oracle computes a sample of tokens (the first, the last, both sides of
every 2^32-byte boundary the tensors cross, and random ones) one by one.
Sizes: IRQ reads 10 GiB and writes 5 GiB of codes; QNR writes 5 GiB; the
paged cache is 5.4 GB; the indexer reads 5 GiB.
"""
import numpy as np
import pytest
import torch

import oracle
import rope_fp8_quant_amd as rq
from rope_fp8_quant_amd import synth
from tests.gpu_util import (DEV, assert_bits_equal, assert_codes_match, assert_q_out_parity,
                            dev, host)

pytestmark = pytest.mark.gpu

BLOCK = 1024  # tokens in the repeated block


@pytest.fixture(autouse=True)
def _release_memory():
    yield
    torch.cuda.empty_cache()


def sample_tokens(N, bytes_per_token, seed, groups=1):
    """First and last tokens, the tokens on both sides of each 4 GiB line of a
    tensor of `groups` consecutive [N, bytes_per_token] blocks, and 16 random
    ones."""
    t = {0, 1, BLOCK - 1, BLOCK, N - 2, N - 1}
    group_bytes = N * bytes_per_token
    k = 1
    while k * (1 << 32) < groups * group_bytes:
        line = k * (1 << 32)
        edge = (line - (line // group_bytes) * group_bytes) // bytes_per_token
        t.update({edge - 1, edge, edge + 1})
        k += 1
    t.update(np.random.default_rng(seed).integers(0, N, 16).tolist())
    return np.array(sorted(x for x in t if 0 <= x < N), np.int64)


def test_irq_past_4_gib():
    N, H, hpg = 327680, 32, 8
    G = H // hpg
    small, _, cache = synth.irq_inputs(dict(synth.IRQ_TINY, N=BLOCK, H=H, hpg=hpg,
                                            max_pos=65536, seed=70))
    pos = (np.arange(N, dtype=np.int64) * 7) % 65536
    print(f"[case] irq large N={N} H={H}: o 10 GiB, codes 5 GiB", flush=True)
    o = dev(small).repeat(N // BLOCK, 1, 1)
    out, sc = rq.empty_inv_rope_fp8_quant_outputs(N, H, hpg, DEV)
    rq.inv_rope_fp8_quant(o, dev(pos), dev(cache), hpg, out, sc)
    torch.cuda.synchronize()
    del o
    ts = sample_tokens(N, H * 1024, 71)
    # the codes tensor [G, N, hpg*512] crosses a 4 GiB line inside group 3
    ts = np.union1d(ts, sample_tokens(N, hpg * 512, 72, groups=G))
    idx = torch.from_numpy(ts).to(DEV)
    got_o = host(out.index_select(1, idx))
    got_s = host(sc.index_select(1, idx))
    eo, es = oracle.inv_rope_fp8_quant(small[ts % BLOCK], pos[ts], cache, hpg)
    assert got_o.shape == (G, ts.size, hpg * 512)
    assert_bits_equal(got_s, es, "large irq scales")
    assert_codes_match(got_o, eo, "large irq codes")


def test_qnr_past_4_gib():
    N, Hq, Hpad = 40960, 64, 128
    cfg = dict(synth.QNR_FORWARD, N=BLOCK, seed=73)
    small, w, _, _ = synth.qnr_inputs(cfg)
    cache = synth.cos_sin_cache(65536)
    pos = (np.arange(N, dtype=np.int64) * 13) % 65536
    print(f"[case] qnorm_rope large N={N} Hq={Hq} Hpad={Hpad}: q_out 5 GiB", flush=True)
    q = dev(small).repeat(N // BLOCK, 1, 1)
    q_out = torch.empty((N, Hpad, 512), dtype=torch.bfloat16, device=DEV)
    rq.qnorm_rope(q, dev(w), dev(pos), dev(cache), q_out, cfg["eps"])
    torch.cuda.synchronize()
    del q
    ts = sample_tokens(N, Hpad * 1024, 74)
    got = host(q_out.index_select(0, torch.from_numpy(ts).to(DEV)))
    assert_q_out_parity(got, small[ts % BLOCK], w, pos[ts], cache, Hpad, cfg["eps"],
                        "large qnorm_rope")


def test_kvi_past_4_gib():
    N, bs, nb = 4096, 64, 160000
    ns = nb * bs  # 10,240,000 slots of 528 bytes
    kv = synth.normal_bf16((N, 512), 75, synth.T_KV)
    pos = synth.uniform_positions(N, 65536, 75)
    cache = synth.cos_sin_cache(65536)
    # the last two slots, the record that straddles 4 GiB, then seeded random ones
    special = np.array([ns - 1, ns - 2, (1 << 32) // 528], np.int64)
    rest = synth.slot_permutation(N + 3, ns, 75)
    slots = np.concatenate([special, rest[~np.isin(rest, special)][:N - 3]])
    assert slots.size == N and np.unique(slots).size == N
    print(f"[case] kv_rope_quant_insert large: cache {nb}x{bs} slots (5.4 GB)", flush=True)
    k_cache = rq.empty_kv_cache(nb, bs, DEV, fill=0xAA)
    rq.kv_rope_quant_insert(dev(kv), dev(pos), dev(cache), dev(slots), k_cache, bs)
    torch.cuda.synchronize()
    recs = k_cache.view(ns, 528)
    got = host(recs.index_select(0, torch.from_numpy(slots).to(DEV)))
    exp = oracle.kv_rope_quant_insert(kv, pos, cache, np.arange(N, dtype=np.int64),
                                      np.full((N, 528), 0xAA, np.uint8), 1)
    assert_bits_equal(got[:, 512:], exp[:, 512:], "large kvi scales")
    assert_codes_match(got[:, :512], exp[:, :512], "large kvi codes")
    # slots nobody wrote stay 0xAA, also past 4 GiB
    free = np.setdiff1d(np.random.default_rng(76).integers(0, ns, 4096), slots)
    free = np.union1d(free, np.setdiff1d([ns - 3, (1 << 32) // 528 + 1], slots))
    untouched = host(recs.index_select(0, torch.from_numpy(free.astype(np.int64)).to(DEV)))
    assert (untouched == 0xAA).all()


def test_indexer_past_4_gib():
    N, H = 327680, 64
    small = synth.normal_bf16((BLOCK, H, 128), 77, synth.T_Q)
    w_small = np.random.default_rng([77, 9]).uniform(0, 1, (BLOCK, H)).astype(np.float32)
    cache = synth.cos_sin_cache(65536)
    pos = (np.arange(N, dtype=np.int64) * 5) % 65536
    print(f"[case] indexer large N={N} H={H}: q 5 GiB", flush=True)
    q = dev(small).repeat(N // BLOCK, 1, 1)
    w = dev(w_small).repeat(N // BLOCK, 1)
    q8 = torch.empty((N, H, 128), dtype=torch.uint8, device=DEV)
    wo = torch.empty((N, H), dtype=torch.float32, device=DEV)
    rq.indexer_q_rope_quant(q, dev(pos), dev(cache), w, q8, wo, 128 ** -0.5)
    torch.cuda.synchronize()
    del q
    ts = sample_tokens(N, H * 256, 78)
    idx = torch.from_numpy(ts).to(DEV)
    got8, gotw = host(q8.index_select(0, idx)), host(wo.index_select(0, idx))
    e8, ew = oracle.indexer_q_rope_quant(small[ts % BLOCK], pos[ts], cache, w_small[ts % BLOCK],
                                         128 ** -0.5)
    assert_bits_equal(gotw, ew, "large indexer weights")
    assert_codes_match(got8, e8, "large indexer codes")
