"""GPU parity of qnorm_rope and kv_rope_quant_insert (HIP path through the C
ABI) vs the oracle."""
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


# ------------------------------------------------------------- qnorm_rope

def qnr_gpu(q, w, pos, cache, hpad, eps, q_dev=None):
    N = q.shape[0]
    q_out = torch.empty((N, hpad, 512), dtype=torch.bfloat16, device=DEV)
    q_out.view(torch.int16).fill_(-1)  # 0xFFFF everywhere: pads must be rewritten
    rq.qnorm_rope(dev(q) if q_dev is None else q_dev, None if w is None else dev(w), dev(pos),
                  dev(cache), q_out, eps)
    torch.cuda.synchronize()
    return host(q_out)


def qnr_check(q, w, pos, cache, hpad, eps, what, q_dev=None, max_frac=None):
    print(f"[case] qnr {what} N={q.shape[0]} Hq={q.shape[1]} Hpad={hpad}", flush=True)
    got = qnr_gpu(q, w, pos, cache, hpad, eps, q_dev)
    assert (got[:, q.shape[1]:] == 0).all(), "pad heads not zero"
    assert_q_out_parity(got, q, w, pos, cache, hpad, eps, f"qnr {what}", max_frac)
    return got


def test_qnr_forward_full_size():
    cfg = synth.QNR_FORWARD
    q, w, pos, cache = synth.qnr_inputs(cfg)
    qnr_check(q, w, pos, cache, cfg["Hpad"], cfg["eps"], "forward 8192x64->128",
              max_frac=Q_DEF_FRAC_BF16)


@pytest.mark.parametrize("shape", SHAPES)
def test_qnr_ragged_no_weight(shape):
    cfg = dict(synth.QNR_FORWARD, N=table_tokens(shape, 7), Hq=5, Hpad=7, max_pos=65536,
               seed=31)
    q, _, pos, cache = synth.qnr_inputs(cfg)
    qnr_check(q, None, pos, cache, 7, 1e-6, f"ragged no-weight {shape}")


@pytest.mark.parametrize("N", synth.DECODE_NS)
def test_qnr_decode_sizes(N):
    cfg = dict(synth.QNR_FORWARD, N=N, Hq=32, Hpad=128, std=1.0, seed=50 + N)
    q, w, _, cache = synth.qnr_inputs(cfg)
    pos = synth.uniform_positions(N, 65536, 50 + N)
    qnr_check(q, w, pos, synth.cos_sin_cache(65536), 128, 1e-6, "decode")


@pytest.mark.parametrize("weighted", [True, False])
def test_qnr_launch_table_entries_bit_identical(weighted):
    # 613 tokens x 24 heads padded to 32 (19616 heads) take qnorm_rope's
    # prefill entry.  The same tokens in calls of 1280 and 320 heads take the
    # one-head-per-wave entry (256- and 64-thread workgroups), and calls of
    # 4800 and 13216 heads the four-head entry in 64-thread workgroups.
    cfg = dict(synth.QNR_FORWARD, N=613, Hq=24, Hpad=32, max_pos=65536, seed=34)
    q, w, _, cache = synth.qnr_inputs(cfg)
    w = w if weighted else None
    pos = synth.uniform_positions(613, 65536, 34)
    print(f"[case] qnr launch-table entries weighted={weighted}", flush=True)
    full = qnr_gpu(q, w, pos, cache, 32, 1e-6)
    assert_q_out_parity(full, q, w, pos, cache, 32, 1e-6, "qnr prefill entry")
    for t0, t1 in ((0, 40), (40, 50), (50, 200), (200, 613)):
        part = qnr_gpu(q[t0:t1].copy(), w, pos[t0:t1].copy(), cache, 32, 1e-6)
        assert (part == full[t0:t1]).all(), f"tokens {t0}..{t1} differ from the prefill entry"


def test_qnr_strided_input():
    cfg = dict(synth.QNR_FORWARD, N=21, Hq=12, Hpad=16, seed=32)
    q, w, pos, cache = synth.qnr_inputs(cfg)
    big = torch.zeros((21, 12, 1536), dtype=torch.bfloat16, device=DEV)
    big[:, :, 1024:] = dev(q)
    qnr_check(q, w, pos, cache, 16, 1e-6, "strided", q_dev=big[:, :, 1024:])


def test_qnr_degenerate_heads():
    rng = np.random.default_rng(33)
    q = np.zeros((6, 4, 512), np.uint16)
    q[0, 1] = 0x8000
    q[1, 0] = synth.f32_to_bf16_bits(np.full(512, 3.0, np.float32))
    q[2, 2] = synth.f32_to_bf16_bits(rng.standard_normal(512).astype(np.float32) * 1e15)
    q[3, 3] = synth.f32_to_bf16_bits(rng.standard_normal(512).astype(np.float32) * 1e-20)
    q[4] = synth.f32_to_bf16_bits(rng.standard_normal((4, 512)).astype(np.float32))
    q[5, :, ::5] = 0x3F80
    w = synth.uniform_bf16((512,), 33, synth.T_W, 0.5, 1.5)
    pos = np.array([0, 1, 2, 100, 4095, 7], np.int64)
    qnr_check(q, w, pos, synth.cos_sin_cache(4096), 6, 1e-6, "degenerate")


def test_qnr_bad_position_poisons_only_its_token():
    cfg = dict(synth.QNR_FORWARD, N=6, Hq=3, Hpad=4, seed=34)
    q, w, pos, cache = synth.qnr_inputs(cfg)
    bad = pos.copy()
    bad[2] = -5
    got = qnr_gpu(q, w, bad, cache, 4, 1e-6)
    good = [0, 1, 3, 4, 5]
    assert_q_out_parity(got[good], q[good].copy(), w, pos[good].copy(), cache, 4, 1e-6,
                        "good tokens")
    assert (got[2, :3] == 0x7FC0).all() and (got[2, 3] == 0).all()


# --------------------------------------------------- kv_rope_quant_insert

def kvi_gpu(kv, pos, cache, slots, nb, bs, stride, scale_fmt="fp32", fill=0xAA):
    k_big = torch.full((nb, stride), fill, dtype=torch.uint8, device=DEV)
    rq.kv_rope_quant_insert(dev(kv), dev(pos), dev(cache), dev(slots), k_big, bs, scale_fmt)
    torch.cuda.synchronize()
    return host(k_big)


def kvi_check(kv, pos, cache, slots, nb, bs, stride=None, scale_fmt="fp32", what="",
              oracle_slots=None):
    stride = bs * 528 if stride is None else stride
    print(f"[case] kvi {what} N={kv.shape[0]} blocks={nb}x{bs} stride={stride} "
          f"fmt={scale_fmt}", flush=True)
    got = kvi_gpu(kv, pos, cache, slots, nb, bs, stride, scale_fmt)
    exp = np.full((nb, stride), 0xAA, np.uint8)
    oracle.kv_rope_quant_insert(kv, pos, cache, slots if oracle_slots is None else oracle_slots,
                                exp, bs, stride, FMT[scale_fmt])
    # placement, untouched bytes and scale bytes must be exact; codes to the bar
    diff = got != exp
    rec = np.zeros_like(diff)
    flat_slots = slots if oracle_slots is None else oracle_slots
    for s in flat_slots[flat_slots >= 0]:
        off = (s // bs) * stride + (s % bs) * 528
        rec.reshape(-1)[off:off + 512] = True
    assert not (diff & ~rec).any(), "bytes outside the code fields differ"
    assert_codes_match(got[rec], exp[rec], f"kvi {what} codes")
    return got


@pytest.mark.parametrize("scale_fmt", ["fp32", "ue8m0"])
def test_kvi_forward_full_size(scale_fmt):
    cfg = synth.KVI_FORWARD
    kv, pos, slots, cache = synth.kvi_inputs(cfg)
    kvi_check(kv, pos, cache, slots, cfg["num_blocks"], cfg["block_size"], None, scale_fmt,
              "forward 8192 -> 256x64")


@pytest.mark.parametrize("shape", SHAPES)
def test_kvi_holes_gaps_and_out_of_range(shape):
    N, bs = table_tokens(shape, 1, base=45), 16
    nb = -(-N // bs) + 2
    kv = synth.normal_bf16((N, 512), 35, synth.T_KV)
    pos = synth.uniform_positions(N, 65536, 35)
    slots = synth.slot_permutation(N, nb * bs, 35)
    slots[[3, 10, 44]] = -1
    slots[[7, 20]] = [nb * bs, 10 ** 12]  # no such slot: skipped by the kernel
    o_slots = slots.copy()
    o_slots[[7, 20]] = -1
    kvi_check(kv, pos, synth.cos_sin_cache(65536), slots, nb, bs, bs * 528 + 64, "fp32",
              f"holes {shape}", oracle_slots=o_slots)


@pytest.mark.parametrize("scale_fmt", ["fp32", "ue8m0"])
def test_kvi_launch_table_entries_bit_identical(scale_fmt):
    # 4500 tokens take the two-token kernel with nontemporal record stores;
    # the same tokens in calls of 2048 and 300 take the one-token kernel
    # (256- and 64-thread workgroups), and a call of 2152 the two-token
    # kernel with plain stores.  Every call writes the same cache bytes.
    N, bs = 4500, 64
    nb = -(-N // bs) + 3
    kv = synth.normal_bf16((N, 512), 36, synth.T_KV)
    pos = synth.uniform_positions(N, 65536, 36)
    slots = synth.slot_permutation(N, nb * bs, 36)
    slots[[5, 2100, 4400]] = -1
    cache = synth.cos_sin_cache(65536)
    print(f"[case] kvi launch-table entries fmt={scale_fmt}", flush=True)
    full = kvi_check(kv, pos, cache, slots, nb, bs, None, scale_fmt, "one call")
    parts = np.full_like(full, 0xAA)
    for t0, t1 in ((0, 2048), (2048, 2348), (2348, 4500)):
        part = kvi_gpu(kv[t0:t1].copy(), pos[t0:t1].copy(), cache, slots[t0:t1].copy(), nb, bs,
                       bs * 528, scale_fmt)
        touched = part != 0xAA
        parts[touched] = part[touched]
    # a record byte that happens to equal 0xAA stays as the fill in `parts`
    assert (parts == full).all(), "the split calls wrote different cache bytes"


@pytest.mark.parametrize("N", [4095, 4096])
@pytest.mark.parametrize("scale_fmt", ["fp32", "ue8m0"])
def test_kvi_store_policy_threshold(N, scale_fmt):
    # The library writes records with plain stores below 4096 tokens and
    # nontemporal ones from 4096 on; both sides of the switch, with holes,
    # must match the oracle and leave every other byte alone.
    bs = 64
    nb = -(-2 * N // bs)
    kv = synth.normal_bf16((N, 512), 37, synth.T_KV)
    pos = synth.uniform_positions(N, 65536, 37)
    slots = synth.slot_permutation(N, nb * bs, 37)
    slots[[0, N // 2, N - 1]] = -1
    kvi_check(kv, pos, synth.cos_sin_cache(65536), slots, nb, bs, None, scale_fmt,
              f"store-policy switch N={N}")


def test_kvi_bad_position_poisons_its_record():
    N, nb, bs = 8, 2, 8
    kv = synth.normal_bf16((N, 512), 36, synth.T_KV)
    pos = np.arange(N, dtype=np.int64)
    slots = synth.slot_permutation(N, nb * bs, 36)
    cache = synth.cos_sin_cache(64)
    bad = pos.copy()
    bad[4] = 64
    got = kvi_gpu(kv, bad, cache, slots, nb, bs, bs * 528)
    o_slots = slots.copy()
    o_slots[4] = -1
    exp = np.full((nb, bs * 528), 0xAA, np.uint8)
    oracle.kv_rope_quant_insert(kv, pos, cache, o_slots, exp, bs)
    s = slots[4]
    off = (s // bs) * bs * 528 + (s % bs) * 528
    g = got.reshape(-1)
    assert np.isnan(g[off + 512:off + 528].view(np.float32)).all()  # NaN scales
    g[off:off + 528] = 0xAA
    assert (got == exp).all()


# ------------------------------------------------------------- HIP graphs

def test_graph_replays_match_eager_results():
    # All three ops captured in one HIP graph, replayed several times with the
    # program's own eager work and synchronizations in between; every replay
    # must reproduce the eager outputs bit for bit.
    o, pos, cache = synth.irq_inputs(dict(synth.IRQ_TINY, N=24, H=32, hpg=8, seed=90))
    qc = dict(synth.QNR_FORWARD, N=24, Hq=8, Hpad=12, seed=91)
    q, w, qpos, qcache = synth.qnr_inputs(qc)
    kv = synth.normal_bf16((24, 512), 92, synth.T_KV)
    slots = synth.slot_permutation(24, 64, 92)
    od, pd, cd = dev(o), dev(pos), dev(cache)
    qd, wd, qpd, qcd = dev(q), dev(w), dev(qpos), dev(qcache)
    kd, sd = dev(kv), dev(slots)
    out, sc = rq.empty_inv_rope_fp8_quant_outputs(24, 32, 8, DEV)
    q_out = torch.empty((24, 12, 512), dtype=torch.bfloat16, device=DEV)
    k_cache = rq.empty_kv_cache(4, 16, DEV, fill=0xAA)

    def step():
        rq.inv_rope_fp8_quant(od, pd, cd, 8, out, sc)
        rq.qnorm_rope(qd, wd, qpd, qcd, q_out, 1e-6)
        rq.kv_rope_quant_insert(kd, qpd, qcd, sd, k_cache, 16)

    step()
    torch.cuda.synchronize()
    eager = [host(t).copy() for t in (out, sc, q_out, k_cache)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (out, q_out, k_cache):  # eager work between replays
            t.view(torch.uint8).fill_(0x5A) if t.dtype != torch.uint8 else t.fill_(0x5A)
        sc.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, exp, name in zip((out, sc, q_out, k_cache), eager, ("codes", "scales", "q_out",
                                                                    "k_cache")):
            g_bits = host(got)
            if name == "k_cache":  # bytes outside the records were refilled with 0x5A
                rec = np.zeros(exp.size, bool)
                for sl in slots:
                    off = (sl // 16) * 16 * 528 + (sl % 16) * 528
                    rec[off:off + 528] = True
                rec = rec.reshape(exp.shape)
                assert (g_bits[~rec] == 0x5A).all()
                g_bits = np.where(rec, g_bits, 0xAA).astype(np.uint8)
            assert_bits_equal(g_bits, exp, f"replay {rep} {name}")
