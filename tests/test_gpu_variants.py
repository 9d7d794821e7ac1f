"""GPU parity of the output variants (HIP path through the C ABI) vs the oracle:
inverse RoPE without quantization, MN-major scale strides, the q path into
FP8, the kv path into the token-strided bf16 cache, and the fused full-cache
forms (also bit-identical to their separate calls)."""
import numpy as np
import pytest
import torch

import oracle
import rope_fp8_quant_amd as rq
from rope_fp8_quant_amd import synth
from tests.gpu_util import (DEV, Q_DEF_FRAC_CODES, SHAPES, assert_bits_equal, assert_codes_match,
                            assert_q_fp8_parity, assert_q_out_parity, dev, host, table_tokens)

pytestmark = pytest.mark.gpu

FMT = {"fp32": oracle.SCALE_FP32, "ue8m0": oracle.SCALE_UE8M0}


# ------------------------------------------------------------ inv_rope_bf16

def irb_gpu(o, pos, cache, hpg, layout="group"):
    N, H, _ = o.shape
    G = H // hpg
    if layout == "group":
        out = torch.full((G, N, hpg * 512), -1, dtype=torch.int16, device=DEV)
        out = out.view(torch.bfloat16)
    else:
        base = torch.full((N, H, 512), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        out = base.view(N, G, hpg * 512).transpose(0, 1)
    rq.inv_rope_bf16(dev(o), dev(pos), dev(cache), hpg, out)
    torch.cuda.synchronize()
    return host(out if layout == "group" else base)


def irb_check(o, pos, cache, hpg, what, layout="group"):
    print(f"[case] inv_rope_bf16 {what} N={o.shape[0]} H={o.shape[1]} hpg={hpg} {layout}",
          flush=True)
    got = irb_gpu(o, pos, cache, hpg, layout)
    assert_bits_equal(got, oracle.inv_rope_bf16(o, pos, cache, hpg, layout), f"irb {what}")


def test_irb_prefill_full_size():
    o, pos, cache = synth.irq_inputs(synth.IRQ_PREFILL)
    irb_check(o, pos, cache, 8, "prefill 16384x32")


def test_irb_irregular_full_size_token_major():
    o, pos, cache = synth.irq_inputs(synth.IRQ_IRREGULAR)
    irb_check(o, pos, cache, 6, "irregular 4096x48", layout="token")


@pytest.mark.parametrize("H,G", [(64, 8), (24, 4), (48, 8), (18, 3)])
@pytest.mark.parametrize("shape", SHAPES)
def test_irb_ragged(H, G, shape):
    cfg = dict(synth.IRQ_TINY, N=table_tokens(shape, H), H=H, hpg=H // G, max_pos=65536,
               seed=H * 7 + G)
    o, pos, cache = synth.irq_inputs(cfg)
    irb_check(o, pos, cache, H // G, f"ragged {shape}")


@pytest.mark.parametrize("N", synth.DECODE_NS)
def test_irb_decode_sizes(N):
    cfg = dict(synth.IRQ_TINY, N=N, H=32, hpg=8, max_pos=65536, seed=90 + N)
    irb_check(*synth.irq_inputs(cfg), 8, "decode")


def test_irb_in_place_token_major():
    cfg = dict(synth.IRQ_TINY, N=29, H=16, hpg=4, max_pos=65536, seed=95)
    o, pos, cache = synth.irq_inputs(cfg)
    print("[case] inv_rope_bf16 in place", flush=True)
    od = dev(o)
    rq.inv_rope_bf16(od, dev(pos), dev(cache), 4, od.view(29, 4, 4 * 512).transpose(0, 1))
    torch.cuda.synchronize()
    assert_bits_equal(host(od), oracle.inv_rope_bf16(o, pos, cache, 4, "token"), "in place")


def test_irb_bad_position_gives_nan_heads():
    cfg = dict(synth.IRQ_TINY, N=6, H=8, hpg=4, seed=96)
    o, pos, cache = synth.irq_inputs(cfg)
    bad = pos.copy()
    bad[2] = cache.shape[0]
    got = irb_gpu(o, bad, cache, 4, "token")
    exp = oracle.inv_rope_bf16(o, pos, cache, 4, "token")
    good = [0, 1, 3, 4, 5]
    assert (got[good] == exp[good]).all()
    assert (got[2] == 0x7FC0).all()


# ------------------------------------------------- MN-major scale layouts

@pytest.mark.parametrize("scale_fmt", ["fp32", "ue8m0"])
def test_irq_mn_major_scales(scale_fmt):
    # scales laid out [G, per-token columns, N] (token fastest), codes
    # group-major: the same values as the default layout, transposed
    cfg = dict(synth.IRQ_TINY, N=41, H=32, hpg=8, max_pos=65536, seed=97)
    o, pos, cache = synth.irq_inputs(cfg)
    N, G, hpg = 41, 4, 8
    per = 4 * hpg if scale_fmt == "fp32" else hpg
    print(f"[case] irq MN-major scales {scale_fmt}", flush=True)
    out = torch.full((G, N, hpg * 512), 0xCD, dtype=torch.uint8, device=DEV)
    dt = torch.float32 if scale_fmt == "fp32" else torch.int32
    mn = torch.full((G, per, N), -7, dtype=dt, device=DEV)
    rq.inv_rope_fp8_quant(dev(o), dev(pos), dev(cache), hpg, out, mn.transpose(1, 2),
                          scale_fmt)
    torch.cuda.synchronize()
    eo, es = oracle.inv_rope_fp8_quant(o, pos, cache, hpg, FMT[scale_fmt])
    assert_bits_equal(host(mn), np.ascontiguousarray(es.transpose(0, 2, 1)), "MN-major scales")
    assert_codes_match(host(out), eo, "MN-major codes")


# ---------------------------------------------------------- qnorm_rope_fp8

def qf8_gpu(q, w, pos, cache, hpad, scale_fmt="fp32", q_dev=None):
    N = q.shape[0]
    codes, sc = rq.empty_qnorm_rope_fp8_outputs(N, hpad, DEV, scale_fmt)
    codes.fill_(0xCD)
    sc.fill_(-7)
    rq.qnorm_rope_fp8(dev(q) if q_dev is None else q_dev, None if w is None else dev(w),
                      dev(pos), dev(cache), codes, sc, 1e-6, scale_fmt)
    torch.cuda.synchronize()
    return host(codes), host(sc)


def qf8_check(q, w, pos, cache, hpad, scale_fmt, what, max_frac=None, **kw):
    print(f"[case] qnorm_rope_fp8 {what} N={q.shape[0]} Hq={q.shape[1]} Hpad={hpad} "
          f"fmt={scale_fmt}", flush=True)
    gc, gs = qf8_gpu(q, w, pos, cache, hpad, scale_fmt, **kw)
    assert_q_fp8_parity(gc, gs, q, w, pos, cache, hpad, 1e-6, scale_fmt, f"qf8 {what}",
                        max_frac=max_frac)


def test_qf8_forward_full_size():
    q, w, pos, cache = synth.qnr_inputs(synth.QNR_FORWARD)
    qf8_check(q, w, pos, cache, 128, "fp32", "forward 8192x64->128", Q_DEF_FRAC_CODES)


def test_qf8_forward_ue8m0_token_slice():
    q, w, pos, cache = synth.qnr_inputs(synth.QNR_FORWARD, 4096, 5120)
    qf8_check(q, w, pos, cache, 128, "ue8m0", "forward slice", Q_DEF_FRAC_CODES)


@pytest.mark.parametrize("scale_fmt", ["fp32", "ue8m0"])
@pytest.mark.parametrize("shape", SHAPES)
def test_qf8_ragged_no_weight(scale_fmt, shape):
    cfg = dict(synth.QNR_FORWARD, N=table_tokens(shape, 7), Hq=5, Hpad=7, seed=98)
    q, _, pos, cache = synth.qnr_inputs(cfg)
    qf8_check(q, None, pos, cache, 7, scale_fmt, f"ragged {shape}")


@pytest.mark.parametrize("N", synth.DECODE_NS)
def test_qf8_decode_sizes(N):
    cfg = dict(synth.QNR_FORWARD, N=N, Hq=32, Hpad=128, seed=99 + N)
    q, w, pos, cache = synth.qnr_inputs(cfg)
    qf8_check(q, w, pos, cache, 128, "fp32", "decode")


@pytest.mark.parametrize("scale_fmt", ["fp32", "ue8m0"])
@pytest.mark.parametrize("quant_eps", [2.0 ** -116, 1e-10, 1e-4, 3.0, 1000.0])
def test_qf8_pad_only_waves_take_the_zero_head_scales(scale_fmt, quant_eps):
    # Hq = 4, Hpad = 12: two of every three waves hold pad heads only, and
    # their scales come from the host; both kinds must match the oracle
    cfg = dict(synth.QNR_FORWARD, N=9, Hq=4, Hpad=12, seed=125)
    q, w, pos, cache = synth.qnr_inputs(cfg)
    print(f"[case] qnorm_rope_fp8 pad waves eps={quant_eps} {scale_fmt}", flush=True)
    codes, sc = rq.empty_qnorm_rope_fp8_outputs(9, 12, DEV, scale_fmt)
    rq.qnorm_rope_fp8(dev(q), dev(w), dev(pos), dev(cache), codes, sc, 1e-6, scale_fmt,
                      quant_eps)
    torch.cuda.synchronize()
    assert_q_fp8_parity(host(codes), host(sc), q, w, pos, cache, 12, 1e-6, scale_fmt,
                        "pad waves", quant_eps)


def test_qf8_strided_input():
    cfg = dict(synth.QNR_FORWARD, N=19, Hq=6, Hpad=8, seed=120)
    q, w, pos, cache = synth.qnr_inputs(cfg)
    big = torch.zeros((19, 9, 512), dtype=torch.bfloat16, device=DEV)
    big[:, 2:8] = dev(q)
    qf8_check(q, w, pos, cache, 8, "fp32", "strided", q_dev=big[:, 2:8])


def test_qf8_bad_position_poisons_live_heads_only():
    cfg = dict(synth.QNR_FORWARD, N=5, Hq=3, Hpad=4, seed=121)
    q, w, pos, cache = synth.qnr_inputs(cfg)
    bad = pos.copy()
    bad[1] = -3
    gc, gs = qf8_gpu(q, w, bad, cache, 4)
    ec, es = oracle.qnorm_rope_fp8(q, w, pos, cache, 4, 1e-6)  # its pad head, below
    good = [0, 2, 3, 4]
    assert_q_fp8_parity(gc[good], gs[good], q[good].copy(), w, pos[good].copy(), cache, 4, 1e-6,
                        "fp32", "good tokens")
    assert np.isnan(gs[1, :3]).all()
    assert (gs[1, 3].view(np.uint32) == es[1, 3].view(np.uint32)).all() and (gc[1, 3] == 0).all()


# ----------------------------------------------------- kv_rope_insert_full

def kvf_inputs(N, ns, seed, holes=(), max_pos=65536):
    kv = synth.normal_bf16((N, 512), seed, synth.T_KV)
    pos = synth.uniform_positions(N, max_pos, seed)
    slots = synth.slot_permutation(N, ns, seed)
    for i in holes:
        slots[i] = -1
    return kv, pos, slots, synth.cos_sin_cache(max_pos)


def kvf_check(kv, pos, slots, cache, ns, row, what):
    print(f"[case] kv_rope_insert_full {what} N={kv.shape[0]} slots={ns} row={row}", flush=True)
    full = torch.full((ns, row), -21846, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    rq.kv_rope_insert_full(dev(kv), dev(pos), dev(cache), dev(slots), full)
    torch.cuda.synchronize()
    exp = oracle.kv_rope_insert_full(kv, pos, cache, slots, np.full((ns, row), 0xAAAA, np.uint16))
    assert_bits_equal(host(full), exp, f"kvf {what}")


def test_kvf_forward_full_size():
    kv, pos, slots, _ = synth.kvi_inputs(synth.KVI_FORWARD)
    kvf_check(kv, pos, slots, synth.cos_sin_cache(8192), 256 * 64, 512, "forward 8192")


@pytest.mark.parametrize("shape", SHAPES)
def test_kvf_ragged_holes_gap_rows(shape):
    N = table_tokens(shape, 1)
    kvf_check(*kvf_inputs(N, N + 13, 122, holes=(0, 11, 36)), N + 13, 576, f"ragged {shape}")


@pytest.mark.parametrize("N", synth.DECODE_NS)
def test_kvf_decode_sizes(N):
    kvf_check(*kvf_inputs(N, 4 * 64, 123 + N), 4 * 64, 512, "decode")


def test_kvf_bad_slot_skipped_bad_position_nan():
    kv, pos, slots, cache = kvf_inputs(6, 8, 124)
    slots = np.array([0, 9, 2, 3, 4, 5], np.int64)  # 9 >= num_slots: skipped
    bad = pos.copy()
    bad[3] = cache.shape[0]
    full = torch.full((8, 512), -21846, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    rq.kv_rope_insert_full(dev(kv), dev(bad), dev(cache), dev(slots), full)
    torch.cuda.synchronize()
    got = host(full)
    ok = np.array([0, 2, 4, 5])
    exp = oracle.kv_rope_insert_full(kv[ok].copy(), pos[ok].copy(), cache, slots[ok].copy(),
                                     np.full((8, 512), 0xAAAA, np.uint16))
    assert (got[[0, 2, 4, 5]] == exp[[0, 2, 4, 5]]).all()
    assert (got[3] == 0x7FC0).all()
    assert (got[[1, 6, 7]] == 0xAAAA).all()


# ------------------------------------------------ fused full-cache forms

def fused_full_inputs(N, Hq, ns, seed, holes=()):
    q = synth.normal_bf16((N, Hq, 512), seed, synth.T_Q, std=2.0)
    w = synth.uniform_bf16((512,), seed, synth.T_W, 0.5, 1.5)
    kv, pos, slots, cache = kvf_inputs(N, ns, seed, holes)
    return q, w, kv, pos, slots, cache


@pytest.mark.parametrize("N,Hq,hpad", [(8192, 64, 64), (37, 5, 5), (3, 32, 32)])
def test_fused_full_bf16_in_place(N, Hq, hpad):
    ns = max(2 * N, 64)
    q, w, kv, pos, slots, cache = fused_full_inputs(N, Hq, ns, 130 + N, holes=(1,))
    print(f"[case] fused full bf16 in place N={N} Hq={Hq}", flush=True)
    qd = dev(q)
    full = torch.full((ns, 512), -21846, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    rq.qnorm_rope_kv_rope_insert_full(qd, dev(w), dev(kv), dev(pos), dev(cache), dev(slots),
                                      qd, full)
    torch.cuda.synchronize()
    assert_q_out_parity(host(qd), q, w, pos, cache, hpad, 1e-6, "fused q")
    exp = oracle.kv_rope_insert_full(kv, pos, cache, slots, np.full((ns, 512), 0xAAAA, np.uint16))
    assert_bits_equal(host(full), exp, "fused kv")


@pytest.mark.parametrize("scale_fmt", ["fp32", "ue8m0"])
@pytest.mark.parametrize("N,Hq,hpad", [(2048, 64, 128), (37, 5, 7), (1, 32, 128)])
def test_fused_full_fp8_matches_oracle_and_separate_calls(scale_fmt, N, Hq, hpad):
    ns = max(2 * N, 64)
    q, w, kv, pos, slots, cache = fused_full_inputs(N, Hq, ns, 140 + N, holes=(0,))
    print(f"[case] fused full fp8 N={N} Hq={Hq} Hpad={hpad} {scale_fmt}", flush=True)
    qd, wd, kd, pd, cd, sd = dev(q), dev(w), dev(kv), dev(pos), dev(cache), dev(slots)
    res = []
    for fused in (True, False):
        codes, sc = rq.empty_qnorm_rope_fp8_outputs(N, hpad, DEV, scale_fmt)
        codes.fill_(0xCD)
        full = torch.full((ns, 512), -21846, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        if fused:
            rq.qnorm_rope_fp8_kv_rope_insert_full(qd, wd, kd, pd, cd, sd, codes, sc, full,
                                                  1e-6, scale_fmt)
        else:
            rq.qnorm_rope_fp8(qd, wd, pd, cd, codes, sc, 1e-6, scale_fmt)
            rq.kv_rope_insert_full(kd, pd, cd, sd, full)
        torch.cuda.synchronize()
        res.append((host(codes), host(sc), host(full)))
    for a, b in zip(*res):
        assert (a.view(np.uint8) == b.view(np.uint8)).all(), "fused differs from separate calls"
    assert_q_fp8_parity(res[0][0], res[0][1], q, w, pos, cache, hpad, 1e-6, scale_fmt,
                        "fused fp8")
    exp = oracle.kv_rope_insert_full(kv, pos, cache, slots, np.full((ns, 512), 0xAAAA, np.uint16))
    assert_bits_equal(res[0][2], exp, "fused fp8 kv rows")


# ----------------------------------------------------- graph capture

def test_graph_replays_of_the_other_entry_points_match_eager():
    # inv_rope_bf16, qnorm_rope_fp8, kv_rope_insert_full, the fused ops and
    # the indexer captured in one HIP graph, replayed four times with eager
    # scribbles over every output in between.  Slots are a permutation of all
    # cache rows, so every output byte is rewritten by each replay.
    N = 24
    o, pos, cache = synth.irq_inputs(dict(synth.IRQ_TINY, N=N, H=16, hpg=4, seed=160))
    q, w, qpos, qcache = synth.qnr_inputs(dict(synth.QNR_FORWARD, N=N, Hq=8, Hpad=12, seed=161))
    kv = synth.normal_bf16((N, 512), 162, synth.T_KV)
    slots = synth.slot_permutation(N, N, 162)
    iq = synth.normal_bf16((N, 8, 128), 163, synth.T_Q)
    iw = np.random.default_rng([163, 9]).uniform(0, 1, (N, 8)).astype(np.float32)
    od, pd, cd = dev(o), dev(pos), dev(cache)
    qd, wd, qpd, qcd = dev(q), dev(w), dev(qpos), dev(qcache)
    kd, sd, iqd, iwd = dev(kv), dev(slots), dev(iq), dev(iw)
    bf = lambda *shape: torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    outs = dict(
        irb=bf(4, N, 4 * 512),
        qf8_codes=torch.empty((N, 12, 512), dtype=torch.uint8, device=DEV),
        qf8_sc=torch.empty((N, 12, 4), dtype=torch.float32, device=DEV),
        kvf=bf(N, 512),
        fq=bf(N, 12, 512),
        fk=torch.empty((3, 8 * 528), dtype=torch.uint8, device=DEV),
        ffc=torch.empty((N, 12, 512), dtype=torch.uint8, device=DEV),
        ffs=torch.empty((N, 12), dtype=torch.int32, device=DEV),
        ffk=bf(N, 512),
        iq8=torch.empty((N, 8, 128), dtype=torch.uint8, device=DEV),
        iwo=torch.empty((N, 8), dtype=torch.float32, device=DEV),
    )

    def step():
        rq.inv_rope_bf16(od, pd, cd, 4, outs["irb"])
        rq.qnorm_rope_fp8(qd, wd, qpd, qcd, outs["qf8_codes"], outs["qf8_sc"], 1e-6)
        rq.kv_rope_insert_full(kd, qpd, qcd, sd, outs["kvf"])
        rq.qnorm_rope_kv_rope_quant_insert(qd, wd, kd, qpd, qcd, sd, outs["fq"], outs["fk"], 8)
        rq.qnorm_rope_fp8_kv_rope_insert_full(qd, wd, kd, qpd, qcd, sd, outs["ffc"], outs["ffs"],
                                              outs["ffk"], 1e-6, "ue8m0")
        rq.indexer_q_rope_quant(iqd, qpd, qcd, iwd, outs["iq8"], outs["iwo"], 128 ** -0.5)

    print("[case] graph of every other entry point", flush=True)
    step()
    torch.cuda.synchronize()
    eager = {k: host(t).copy() for k, t in outs.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs.values():  # eager work between replays
            t.view(torch.uint8).fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, t in outs.items():
            assert_bits_equal(host(t), eager[k], f"replay {rep} {k}")
    # and the eager results are the oracle's
    assert_bits_equal(eager["irb"], oracle.inv_rope_bf16(o, pos, cache, 4), "graph irb")
    exp = oracle.kv_rope_insert_full(kv, qpos, qcache, slots, np.zeros((N, 512), np.uint16))
    assert_bits_equal(eager["kvf"], exp, "graph kvf")


@pytest.mark.parametrize("shape", SHAPES)
def test_irq_scales_at_a_4_byte_offset(shape):
    # FP32 scales that are 4- but not 16-byte aligned take the per-block
    # stores; the default-aligned ones take the gathered 16-byte store
    N, G, hpg = table_tokens(shape, 16, base=23), 2, 8
    cfg = dict(synth.IRQ_TINY, N=N, H=16, hpg=hpg, max_pos=65536, seed=170)
    o, pos, cache = synth.irq_inputs(cfg)
    print(f"[case] irq scales at +4 bytes {shape}", flush=True)
    out = torch.full((G, N, hpg * 512), 0xCD, dtype=torch.uint8, device=DEV)
    raw = torch.full((G * N * hpg * 4 + 1,), -7.0, dtype=torch.float32, device=DEV)
    sc = raw[1:].view(G, N, hpg * 4)
    assert sc.data_ptr() % 16 == 4
    rq.inv_rope_fp8_quant(dev(o), dev(pos), dev(cache), hpg, out, sc)
    torch.cuda.synchronize()
    eo, es = oracle.inv_rope_fp8_quant(o, pos, cache, hpg)
    assert_bits_equal(host(sc), es, "offset scales")
    assert host(raw)[0] == np.float32(-7.0)
    assert_codes_match(host(out), eo, "offset codes")
