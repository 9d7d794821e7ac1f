"""Prepared calls (rq.prepare): checked and marshalled once, relaunched with
no further checks, on torch's current stream or a given one.  Each relaunch
must equal the regular call bit for bit."""
import numpy as np
import pytest
import torch

import rope_fp8_quant_amd as rq
from rope_fp8_quant_amd import synth
from tests.gpu_util import DEV, assert_bits_equal, dev, host

pytestmark = pytest.mark.gpu


def test_prepared_calls_match_regular_calls():
    o, pos, cache = synth.irq_inputs(dict(synth.IRQ_TINY, N=5, H=32, hpg=8, max_pos=65536,
                                          seed=180))
    q, w, qpos, qcache = synth.qnr_inputs(dict(synth.QNR_FORWARD, N=5, Hq=32, Hpad=128,
                                               seed=181))
    kv = synth.normal_bf16((5, 512), 182, synth.T_KV)
    slots = synth.slot_permutation(5, 64, 182)
    iq = synth.normal_bf16((5, 64, 128), 183, synth.T_Q)
    iw = np.random.default_rng([183, 9]).uniform(0, 1, (5, 64)).astype(np.float32)
    od, pd, cd = dev(o), dev(pos), dev(cache)
    qd, wd, qpd, qcd = dev(q), dev(w), dev(qpos), dev(qcache)
    kd, sd, iqd, iwd = dev(kv), dev(slots), dev(iq), dev(iw)

    def outputs():
        out, sc = rq.empty_inv_rope_fp8_quant_outputs(5, 32, 8, DEV)
        return dict(out=out, sc=sc,
                    q_out=torch.empty((5, 128, 512), dtype=torch.bfloat16, device=DEV),
                    k_cache=rq.empty_kv_cache(4, 16, DEV, fill=0xAA),
                    i8=torch.empty((5, 64, 128), dtype=torch.uint8, device=DEV),
                    iwo=torch.empty((5, 64), dtype=torch.float32, device=DEV))

    def calls(x):
        return [(rq.inv_rope_fp8_quant, (od, pd, cd, 8, x["out"], x["sc"])),
                (rq.qnorm_rope, (qd, wd, qpd, qcd, x["q_out"], 1e-6)),
                (rq.kv_rope_quant_insert, (kd, qpd, qcd, sd, x["k_cache"], 16)),
                (rq.indexer_q_rope_quant, (iqd, qpd, qcd, iwd, x["i8"], x["iwo"],
                                           128 ** -0.5))]

    print("[case] prepared calls: irq, qnr, kvi, indexer", flush=True)
    ref = outputs()
    for op, args in calls(ref):
        op(*args)
    torch.cuda.synchronize()
    got = outputs()
    prepared = [rq.prepare(op, *args) for op, args in calls(got)]
    for t in got.values():
        t.view(torch.uint8).fill_(0x5A)
    torch.cuda.synchronize()  # prepare() launched nothing: outputs still 0x5A
    assert all((host(t.view(torch.uint8)) == 0x5A).all() for t in got.values())
    side = torch.cuda.Stream()
    for rep in range(3):
        for t in got.values():
            t.view(torch.uint8).fill_(0x5A)
        torch.cuda.synchronize()
        if rep == 2:
            side.wait_stream(torch.cuda.current_stream())
            for call in prepared:
                call(stream=side)
            side.synchronize()
        else:
            for call in prepared:
                call()
            torch.cuda.synchronize()
        for k in ref:
            if k == "k_cache":  # bytes outside the records were refilled
                continue
            assert_bits_equal(host(got[k]), host(ref[k]), f"prepared {k} rep {rep}")
        kc, rc = host(got["k_cache"]), host(ref["k_cache"])
        for s in slots:
            off = (s // 16) * 16 * 528 + (s % 16) * 528
            assert (kc.reshape(-1)[off:off + 528] == rc.reshape(-1)[off:off + 528]).all()
