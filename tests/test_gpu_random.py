"""Seeded random sweeps of every op against the oracle, and stream ordering.

Each case draws its shape, grouping, strides (padded rows), scale format,
positions and slot holes from a seeded generator, at a size in one of the
two entries of the launch table, runs the HIP path through the C ABI and
compares with the oracle to the parity bar.  The case parameters are printed
before each GPU step.
"""
import numpy as np
import pytest
import torch

import oracle
import rope_fp8_quant_amd as rq
from rope_fp8_quant_amd import synth
from tests.gpu_util import (DEV, SHAPES, TABLE_ROWS, assert_bits_equal, assert_codes_match,
                            assert_q_fp8_parity, assert_q_out_parity, dev, host)

pytestmark = pytest.mark.gpu

FMTS = ("fp32", "ue8m0")
FMT = {"fp32": oracle.SCALE_FP32, "ue8m0": oracle.SCALE_UE8M0}


def draw_tokens(rng, shape, rows_per_token, spread):
    """A token count whose launch of rows_per_token 16-lane rows per token
    lands in table entry `shape`."""
    if shape == SHAPES[0]:
        return int(rng.integers(1, min(spread, (TABLE_ROWS - 1) // rows_per_token) + 1))
    return -(-TABLE_ROWS // rows_per_token) + int(rng.integers(0, spread))


def padded(a, pad_elems, seed):
    """A device copy of a [N, H, D] or [N, D] array inside a wider buffer
    (rows padded by pad_elems), returned as the strided view."""
    t = dev(a)
    if pad_elems == 0:
        return t
    shape = list(t.shape)
    shape[-1] += pad_elems
    big = torch.zeros(shape, dtype=t.dtype, device=DEV)
    big[..., :t.shape[-1]] = t
    return big[..., :t.shape[-1]]


@pytest.mark.parametrize("case", range(12))
def test_irq_random(case):
    rng = np.random.default_rng([200, case])
    hpg = int(rng.choice([1, 2, 3, 4, 6, 8, 12]))
    G = int(rng.integers(1, 6))
    shape = SHAPES[(case // 2) % 2]
    N = draw_tokens(rng, shape, G * hpg, 300)
    fmt = FMTS[case % 2]
    pad = int(rng.choice([0, 8, 64]))
    max_pos = int(rng.choice([64, 4096, 65536]))
    print(f"[case] irq random #{case}: N={N} H={G * hpg} hpg={hpg} fmt={fmt} {shape} "
          f"pad={pad} max_pos={max_pos}", flush=True)
    o = synth.normal_bf16((N, G * hpg, 512), 210 + case, synth.T_O, outlier_frac=0.01)
    pos = rng.integers(0, max_pos, N).astype(np.int64)
    cache = synth.cos_sin_cache(max_pos)
    out, sc = rq.empty_inv_rope_fp8_quant_outputs(N, G * hpg, hpg, DEV, fmt)
    rq.inv_rope_fp8_quant(padded(o, pad, case), dev(pos), dev(cache), hpg, out, sc, fmt)
    torch.cuda.synchronize()
    eo, es = oracle.inv_rope_fp8_quant(o, pos, cache, hpg, FMT[fmt])
    assert_bits_equal(host(sc), es, "random irq scales")
    assert_codes_match(host(out), eo, "random irq codes")
    # the bf16 form on the same inputs
    ob = torch.empty((G, N, hpg * 512), dtype=torch.bfloat16, device=DEV)
    rq.inv_rope_bf16(padded(o, pad, case), dev(pos), dev(cache), hpg, ob)
    torch.cuda.synchronize()
    assert_bits_equal(host(ob), oracle.inv_rope_bf16(o, pos, cache, hpg), "random irb")


@pytest.mark.parametrize("case", range(10))
def test_q_paths_random(case):
    rng = np.random.default_rng([300, case])
    Hq = int(rng.integers(1, 20))
    Hpad = Hq + int(rng.choice([0, 1, 3, 8, 20]))
    shape = SHAPES[(case // 2) % 2]
    N = draw_tokens(rng, shape, Hpad, 200)
    fmt = FMTS[case % 2]
    pad = int(rng.choice([0, 8, 136]))
    weighted = bool(case % 3)
    eps = float(rng.choice([1e-6, 1e-3, 0.5]))
    print(f"[case] q paths random #{case}: N={N} Hq={Hq} Hpad={Hpad} fmt={fmt} {shape} "
          f"pad={pad} weight={weighted} eps={eps}", flush=True)
    q = synth.normal_bf16((N, Hq, 512), 310 + case, synth.T_Q, std=float(rng.uniform(0.1, 4)))
    w = synth.uniform_bf16((512,), 310 + case, synth.T_W, 0.5, 1.5) if weighted else None
    pos = rng.integers(0, 65536, N).astype(np.int64)
    cache = synth.cos_sin_cache(65536)
    qd = padded(q, pad, case)
    wd = None if w is None else dev(w)
    q_out = torch.full((N, Hpad, 512), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    rq.qnorm_rope(qd, wd, dev(pos), dev(cache), q_out, eps)
    codes, sc = rq.empty_qnorm_rope_fp8_outputs(N, Hpad, DEV, fmt)
    rq.qnorm_rope_fp8(qd, wd, dev(pos), dev(cache), codes, sc, eps, fmt)
    torch.cuda.synchronize()
    assert_q_out_parity(host(q_out), q, w, pos, cache, Hpad, eps, "random qnr")
    assert_q_fp8_parity(host(codes), host(sc), q, w, pos, cache, Hpad, eps, fmt, "random qf8")


@pytest.mark.parametrize("case", range(10))
def test_kv_paths_random(case):
    rng = np.random.default_rng([400, case])
    shape = SHAPES[(case // 2) % 2]
    N = draw_tokens(rng, shape, 1, 400)
    bs = int(rng.choice([1, 4, 16, 64]))
    nb = -(-(N + int(rng.integers(0, 50))) // bs)
    fmt = FMTS[case % 2]
    gap = int(rng.choice([0, 16, 528]))
    pad = int(rng.choice([0, 8]))
    print(f"[case] kv paths random #{case}: N={N} blocks={nb}x{bs} fmt={fmt} {shape} "
          f"gap={gap} pad={pad}", flush=True)
    kv = synth.normal_bf16((N, 512), 410 + case, synth.T_KV)
    pos = rng.integers(0, 4096, N).astype(np.int64)
    slots = synth.slot_permutation(N, nb * bs, 410 + case)
    slots[rng.random(N) < 0.1] = -1
    cache = synth.cos_sin_cache(4096)
    stride = bs * 528 + gap
    k_cache = torch.full((nb, stride), 0xAA, dtype=torch.uint8, device=DEV)
    rq.kv_rope_quant_insert(padded(kv, pad, case), dev(pos), dev(cache), dev(slots), k_cache, bs,
                            fmt)
    row = 512 + int(rng.choice([0, 8, 64]))
    full = torch.full((nb * bs, row), -21846, dtype=torch.int16, device=DEV)
    full = full.view(torch.bfloat16)
    rq.kv_rope_insert_full(padded(kv, pad, case), dev(pos), dev(cache), dev(slots), full)
    torch.cuda.synchronize()
    exp = oracle.kv_rope_quant_insert(kv, pos, cache, slots, np.full((nb, stride), 0xAA, np.uint8),
                                      bs, stride, FMT[fmt])
    got = host(k_cache)
    rec = np.zeros(exp.size, bool)
    for s in slots[slots >= 0]:
        off = (s // bs) * stride + (s % bs) * 528
        rec[off:off + 512] = True
    rec = rec.reshape(exp.shape)
    assert (got[~rec] == exp[~rec]).all(), "random kvi: bytes outside the codes differ"
    assert_codes_match(got[rec], exp[rec], "random kvi codes")
    ef = oracle.kv_rope_insert_full(kv, pos, cache, slots,
                                    np.full((nb * bs, row), 0xAAAA, np.uint16))
    assert_bits_equal(host(full), ef, "random kvf")


@pytest.mark.parametrize("case", range(8))
def test_indexer_random(case):
    rng = np.random.default_rng([500, case])
    H = int(rng.integers(1, 70))
    shape = SHAPES[case % 2]
    # four rows per wave of two 4-head items: 2 * ceil(H / 4) rows per token
    N = draw_tokens(rng, shape, 2 * (-(-H // 4)), 300)
    hs = float(rng.uniform(0.25, 2.0))
    print(f"[case] indexer random #{case}: N={N} H={H} {shape} head_scale={hs:.3f}",
          flush=True)
    q = synth.normal_bf16((N, H, 128), 510 + case, synth.T_Q, std=float(rng.uniform(0.01, 30)))
    w = rng.uniform(0, 1, (N, H)).astype(np.float32)
    pos = rng.integers(0, 65536, N).astype(np.int64)
    cache = synth.cos_sin_cache(65536)
    q8 = torch.empty((N, H, 128), dtype=torch.uint8, device=DEV)
    wo = torch.empty((N, H), dtype=torch.float32, device=DEV)
    rq.indexer_q_rope_quant(dev(q), dev(pos), dev(cache), dev(w), q8, wo, 128 ** -0.5, hs)
    torch.cuda.synchronize()
    ec, ew = oracle.indexer_q_rope_quant(q, pos, cache, w, 128 ** -0.5, hs)
    assert_bits_equal(host(wo), ew, "random indexer weights")
    assert_codes_match(host(q8), ec, "random indexer codes")


@pytest.mark.parametrize("case", range(9))
def test_fused_forms_random(case):
    # The fused kernels split one grid at q_waves; ragged q-unit counts put q
    # and kv work in neighbouring waves.  Each fused form must equal its two
    # separate calls bit for bit, and the oracle.
    rng = np.random.default_rng([700, case])
    Hq = int(rng.integers(1, 11))
    Hpad = Hq + int(rng.choice([0, 1, 2, 5]))
    form = ("quant", "full_fp8", "full_bf16")[case % 3]
    fmt = FMTS[(case // 3) % 2]
    shape = SHAPES[case % 2]
    # one grid: a q row per head (Hq in place, else Hpad) and one kv row per token
    N = draw_tokens(rng, shape, (Hq if form == "full_bf16" else Hpad) + 1, 150)
    weighted = case % 2 == 0
    print(f"[case] fused random #{case}: form={form} N={N} Hq={Hq} Hpad={Hpad} fmt={fmt} "
          f"{shape} weight={weighted}", flush=True)
    q = synth.normal_bf16((N, Hq, 512), 710 + case, synth.T_Q, std=2.0)
    w = synth.uniform_bf16((512,), 710 + case, synth.T_W, 0.5, 1.5) if weighted else None
    kv = synth.normal_bf16((N, 512), 710 + case, synth.T_KV)
    pos = rng.integers(0, 4096, N).astype(np.int64)
    cache = synth.cos_sin_cache(4096)
    bs, nb = 16, -(-N // 16) + 2
    slots = synth.slot_permutation(N, nb * bs, 710 + case)
    slots[rng.random(N) < 0.1] = -1
    qd, wd, kd, pd, cd, sd = dev(q), None if w is None else dev(w), dev(kv), dev(pos), dev(cache), dev(slots)
    if form == "quant":
        outs = []
        for fused in (True, False):
            q_out = torch.full((N, Hpad, 512), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
            k_cache = rq.empty_kv_cache(nb, bs, DEV, fill=0xAA)
            if fused:
                rq.qnorm_rope_kv_rope_quant_insert(qd, wd, kd, pd, cd, sd, q_out, k_cache, bs,
                                                   1e-6, fmt)
            else:
                rq.qnorm_rope(qd, wd, pd, cd, q_out, 1e-6)
                rq.kv_rope_quant_insert(kd, pd, cd, sd, k_cache, bs, fmt)
            torch.cuda.synchronize()
            outs.append((host(q_out), host(k_cache)))
        assert_bits_equal(outs[0][0], outs[1][0], "fused vs separate q_out")
        assert_bits_equal(outs[0][1], outs[1][1], "fused vs separate k_cache")
        assert_q_out_parity(outs[0][0], q, w, pos, cache, Hpad, 1e-6, "fused q_out vs oracle")
        ek = oracle.kv_rope_quant_insert(kv, pos, cache, slots,
                                         np.full((nb, bs * 528), 0xAA, np.uint8), bs,
                                         scale_fmt=FMT[fmt])
        rec = np.zeros(ek.size, bool)
        for s_ in slots[slots >= 0]:
            rec[(s_ // bs) * bs * 528 + (s_ % bs) * 528:][:512] = True
        rec = rec.reshape(ek.shape)
        got = outs[0][1]
        assert (got[~rec] == ek[~rec]).all(), "fused cache bytes outside the codes differ"
        assert_codes_match(got[rec], ek[rec], "fused cache codes vs oracle")
        return
    ns = nb * bs
    full = []
    for fused in (True, False):
        cache_full = torch.full((ns, 512), -21846, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        if form == "full_fp8":
            codes, sc = rq.empty_qnorm_rope_fp8_outputs(N, Hpad, DEV, fmt)
            if fused:
                rq.qnorm_rope_fp8_kv_rope_insert_full(qd, wd, kd, pd, cd, sd, codes, sc,
                                                      cache_full, 1e-6, fmt)
            else:
                rq.qnorm_rope_fp8(qd, wd, pd, cd, codes, sc, 1e-6, fmt)
                rq.kv_rope_insert_full(kd, pd, cd, sd, cache_full)
            torch.cuda.synchronize()
            full.append((host(codes), host(sc), host(cache_full)))
        else:
            # q in place: needs Hpad == Hq and a contiguous q
            qi = dev(q)
            hp = Hq
            if fused:
                rq.qnorm_rope_kv_rope_insert_full(qi, wd, kd, pd, cd, sd, qi, cache_full, 1e-6)
            else:
                rq.qnorm_rope(qi, wd, pd, cd, qi, 1e-6)
                rq.kv_rope_insert_full(kd, pd, cd, sd, cache_full)
            torch.cuda.synchronize()
            full.append((host(qi), None, host(cache_full)))
    for a, b, what in zip(full[0], full[1], ("q", "q scales", "kv cache")):
        if a is not None:
            assert_bits_equal(a, b, f"fused vs separate {what}")
    ef = oracle.kv_rope_insert_full(kv, pos, cache, slots, np.full((ns, 512), 0xAAAA, np.uint16))
    assert_bits_equal(full[0][2], ef, "fused kv cache vs oracle")
    if form == "full_fp8":
        assert_q_fp8_parity(full[0][0], full[0][1], q, w, pos, cache, Hpad, 1e-6, fmt,
                            "fused q vs oracle")
    else:
        assert_q_out_parity(full[0][0], q, w, pos, cache, hp, 1e-6, "fused in-place q vs oracle")


def test_calls_run_in_order_on_the_callers_stream():
    # Work is enqueued on the stream passed in: a long fill queued first on a
    # side stream must finish before the op reads its input there, and the
    # op's output must be complete when that stream is synchronized.
    o, pos, cache = synth.irq_inputs(dict(synth.IRQ_TINY, N=64, H=16, hpg=8, seed=600))
    od = dev(o)
    scratch = torch.empty(1 << 28, dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    src = torch.zeros_like(od)
    out, sc = rq.empty_inv_rope_fp8_quant_outputs(64, 16, 8, DEV)
    print("[case] stream ordering", flush=True)
    with torch.cuda.stream(side):
        for _ in range(4):
            scratch.fill_(3)  # slow work ahead of the copy
        src.copy_(od)
        rq.inv_rope_fp8_quant(src, dev(pos), dev(cache), 8, out, sc, stream=side)
    side.synchronize()
    eo, es = oracle.inv_rope_fp8_quant(o, pos, cache, 8)
    assert_bits_equal(host(sc), es, "side-stream scales")
    assert_codes_match(host(out), eo, "side-stream codes")


def test_concurrent_callers_on_their_own_streams():
    # The library keeps no per-call state: host threads calling it at once
    # (ctypes drops the GIL for the call), each on its own stream and buffers,
    # all get their own results.
    import threading
    cases = []
    for i in range(4):
        cfg = dict(synth.IRQ_TINY, N=64 + 16 * i, H=16, hpg=8, max_pos=65536, seed=610 + i)
        o, pos, cache = synth.irq_inputs(cfg)
        out, sc = rq.empty_inv_rope_fp8_quant_outputs(cfg["N"], 16, 8, DEV)
        cases.append((o, pos, cache, dev(o), dev(pos), dev(cache), out, sc, torch.cuda.Stream()))
    errors = []

    def worker(case):
        o, pos, cache, od, pd, cd, out, sc, stream = case
        try:
            for _ in range(20):
                rq.inv_rope_fp8_quant(od, pd, cd, 8, out, sc, stream=stream)
        except Exception as e:  # reported below
            errors.append(e)

    print("[case] 4 threads x 20 calls, one stream each", flush=True)
    threads = [threading.Thread(target=worker, args=(c,)) for c in cases]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for o, pos, cache, _, _, _, out, sc, _ in cases:
        eo, es = oracle.inv_rope_fp8_quant(o, pos, cache, 8)
        assert_bits_equal(host(sc), es, "concurrent scales")
        assert_codes_match(host(out), eo, "concurrent codes")
