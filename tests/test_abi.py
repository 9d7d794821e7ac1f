"""The C ABI on the host: exported symbols, status codes, argument validation.

No kernel runs here.  The validation cases pass fake (never dereferenced)
device addresses, so they are skipped where a GPU is visible: a validation
bug there would launch a kernel on them.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

from rope_fp8_quant_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ropequant.h")

OK, NULL, SHAPE, STRIDE, ALIGN, VALUE = 0, -1, -2, -3, -4, -5

host_only = pytest.mark.skipif(torch.cuda.is_available(),
                               reason="passes fake device pointers; host-only check")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", text, flags=re.M)


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert set(names) >= {"inv_rope_fp8_quant", "qnorm_rope", "kv_rope_quant_insert"}
    syms = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                          text=True, check=True).stdout
    exported = {line.split()[-1] for line in syms.splitlines() if " T " in line}
    missing = [n for n in names if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    L = _lib.lib()
    for n in names:
        getattr(L, n)


def test_abi_version_matches_header():
    m = re.search(r"#define\s+ROPEQUANT_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert _lib.lib().ropequant_abi_version() == int(m.group(1))


def test_status_strings_distinct():
    L = _lib.lib()
    msgs = [L.ropequant_strerror(s).decode() for s in range(0, -7, -1)]
    assert len(set(msgs)) == 7 and all(msgs)
    assert L.ropequant_strerror(-99).decode() == "unknown status"


def test_exports_are_exactly_the_declared_functions():
    # nothing beyond the header: in particular no process-wide setting that
    # one caller could change under another
    syms = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                          text=True, check=True).stdout
    exported = {line.split()[-1] for line in syms.splitlines() if line.split()[1:2] == ["T"]}
    assert exported == set(declared_functions())
    assert set(_lib.EXPORTS) == exported


A = 0x100000  # fake, 256-byte aligned "device" addresses
B = 0x900000  # a second one, for outputs that must not alias an input


def irq(**kw):
    a = dict(o=A, ost=32 * 512, osh=512, pos=A, cs=A, max_pos=4096, n=16, h=32, hpg=8, fmt=0,
             eps=1e-10, out=A, osg=16 * 8 * 512, ost2=8 * 512, sc=A, ssg=16 * 32, sst=32, ssb=1)
    a.update(kw)
    return _lib.lib().inv_rope_fp8_quant(
        a["o"], a["ost"], a["osh"], a["pos"], a["cs"], a["max_pos"], a["n"], a["h"], a["hpg"],
        a["fmt"], a["eps"], a["out"], a["osg"], a["ost2"], a["sc"], a["ssg"], a["sst"],
        a["ssb"], None)


def qnr(**kw):
    a = dict(q=A, qst=64 * 512, qsh=512, w=A, pos=A, cs=A, max_pos=8192, n=8, hq=64, hpad=128,
             eps=1e-6, out=B)
    a.update(kw)
    return _lib.lib().qnorm_rope(a["q"], a["qst"], a["qsh"], a["w"], a["pos"], a["cs"],
                                 a["max_pos"], a["n"], a["hq"], a["hpad"], a["eps"], a["out"],
                                 None)


def kvi(**kw):
    a = dict(kv=A, kst=512, pos=A, cs=A, max_pos=8192, slots=A, n=8, cache=A, nb=256,
             stride=64 * 528, bs=64, fmt=0, eps=1e-10)
    a.update(kw)
    return _lib.lib().kv_rope_quant_insert(a["kv"], a["kst"], a["pos"], a["cs"], a["max_pos"],
                                           a["slots"], a["n"], a["cache"], a["nb"], a["stride"],
                                           a["bs"], a["fmt"], a["eps"], None)


def test_zero_tokens_is_ok_without_pointers():
    assert irq(n=0, o=None, pos=None, cs=None, out=None, sc=None) == OK
    assert qnr(n=0, q=None, w=None, pos=None, cs=None, out=None) == OK
    assert kvi(n=0, kv=None, pos=None, cs=None, slots=None, cache=None) == OK


@host_only
@pytest.mark.parametrize("kw,status", [
    (dict(hpg=7), SHAPE), (dict(n=-1), SHAPE), (dict(max_pos=0), SHAPE),
    (dict(h=0), SHAPE), (dict(n=1 << 26, h=32), SHAPE),
    (dict(fmt=2), VALUE), (dict(eps=0.0), VALUE), (dict(eps=float("nan")), VALUE),
    (dict(eps=1e-40), VALUE), (dict(eps=float("inf")), VALUE),
    (dict(o=None), NULL), (dict(pos=None), NULL), (dict(cs=None), NULL),
    (dict(out=None), NULL), (dict(sc=None), NULL),
    (dict(ost=0), STRIDE), (dict(ssb=0), STRIDE),
    (dict(o=A + 8), ALIGN), (dict(osh=516), ALIGN), (dict(ost=32 * 512 + 4), ALIGN),
    (dict(cs=A + 4), ALIGN), (dict(pos=A + 4), ALIGN), (dict(out=A + 8), ALIGN),
    (dict(ost2=8 * 512 + 8), ALIGN), (dict(sc=A + 2), ALIGN),
    (dict(ost2=4 * 512), STRIDE),                 # token rows overlap (hpg*512 bytes each)
    (dict(osg=8 * 512, ost2=16 * 512), STRIDE),   # group rows collide with token rows
    (dict(sst=16), STRIDE),                       # scale rows overlap
])
def test_irq_validation(kw, status):
    assert irq(**kw) == status


@host_only
def test_irq_token_major_strides_are_accepted_by_validation():
    # [N, H, 512] token-major strides pass validation; with no GPU the launch
    # itself is refused by the runtime, which must come back as RQ_ERR_HIP.
    assert irq(osg=8 * 512, ost2=32 * 512, ssg=32, sst=128, ssb=1) == -6


@host_only
@pytest.mark.parametrize("kw,status", [
    (dict(hpad=63), SHAPE), (dict(hq=0), SHAPE), (dict(max_pos=0), SHAPE),
    (dict(n=1 << 25, hpad=128), SHAPE),
    (dict(eps=0.0), VALUE), (dict(eps=-1.0), VALUE), (dict(eps=1e-50), VALUE),
    (dict(q=None), NULL), (dict(out=None), NULL), (dict(pos=None), NULL), (dict(cs=None), NULL),
    (dict(qst=0), STRIDE),
    (dict(q=A + 2), ALIGN), (dict(qsh=500), ALIGN), (dict(w=A + 8), ALIGN),
    (dict(out=B + 4), ALIGN), (dict(cs=A + 8), ALIGN),
    (dict(out=A), STRIDE),                                # in place needs hpad == hq
    (dict(out=A, hpad=64, qsh=1024, qst=128 * 512), STRIDE),  # ... and contiguous q
])
def test_qnr_validation(kw, status):
    assert qnr(**kw) == status


@host_only
@pytest.mark.parametrize("kw,status", [
    (dict(bs=0), SHAPE), (dict(nb=0), SHAPE), (dict(n=-3), SHAPE), (dict(max_pos=0), SHAPE),
    (dict(nb=1 << 26, bs=64), SHAPE),
    (dict(stride=64 * 528 - 16), STRIDE), (dict(kst=0), STRIDE),
    (dict(fmt=5), VALUE), (dict(eps=0.0), VALUE),
    (dict(kv=None), NULL), (dict(slots=None), NULL), (dict(cache=None), NULL),
    (dict(stride=64 * 528 + 8), ALIGN), (dict(cache=A + 8), ALIGN), (dict(kv=A + 8), ALIGN),
    (dict(kst=516), ALIGN), (dict(slots=A + 4), ALIGN),
])
def test_kvi_validation(kw, status):
    assert kvi(**kw) == status


def fused(**kw):
    a = dict(q=A, qst=64 * 512, qsh=512, w=A, kv=A, kst=512, pos=A, cs=A, max_pos=8192,
             slots=A, n=8, hq=64, hpad=128, eps=1e-6, out=B, cache=A, nb=256, stride=64 * 528,
             bs=64, fmt=0, qeps=1e-10)
    a.update(kw)
    return _lib.lib().qnorm_rope_kv_rope_quant_insert(
        a["q"], a["qst"], a["qsh"], a["w"], a["kv"], a["kst"], a["pos"], a["cs"], a["max_pos"],
        a["slots"], a["n"], a["hq"], a["hpad"], a["eps"], a["out"], a["cache"], a["nb"],
        a["stride"], a["bs"], a["fmt"], a["qeps"], None)


def test_fused_zero_tokens_is_ok_without_pointers():
    assert fused(n=0, q=None, w=None, kv=None, pos=None, cs=None, slots=None, out=None,
                 cache=None) == OK


@host_only
@pytest.mark.parametrize("kw,status", [
    (dict(hpad=63), SHAPE), (dict(bs=0), SHAPE), (dict(eps=0.0), VALUE), (dict(qeps=0.0), VALUE),
    (dict(fmt=3), VALUE), (dict(q=None), NULL), (dict(kv=None), NULL), (dict(slots=None), NULL),
    (dict(cache=None), NULL), (dict(stride=100), STRIDE), (dict(kv=A + 8), ALIGN),
    (dict(out=B + 8), ALIGN), (dict(out=A), STRIDE),
])
def test_fused_validation(kw, status):
    assert fused(**kw) == status


def idx(**kw):
    a = dict(q=A, qst=64 * 128, qsh=128, pos=A, cs=A, max_pos=4096, w=A, wst=64, n=8, h=64,
             ss=128 ** -0.5, hs=1.0, eps=1e-10, out=A, ost=64 * 128, osh=128, wo=A, wost=64)
    a.update(kw)
    return _lib.lib().indexer_q_rope_quant(a["q"], a["qst"], a["qsh"], a["pos"], a["cs"],
                                           a["max_pos"], a["w"], a["wst"], a["n"], a["h"],
                                           a["ss"], a["hs"], a["eps"], a["out"], a["ost"],
                                           a["osh"], a["wo"], a["wost"], None)


def test_indexer_zero_tokens_is_ok_without_pointers():
    assert idx(n=0, q=None, pos=None, cs=None, w=None, out=None, wo=None) == OK


@host_only
@pytest.mark.parametrize("kw,status", [
    (dict(h=0), SHAPE), (dict(n=-1), SHAPE), (dict(max_pos=0), SHAPE),
    (dict(n=1 << 25, h=64), SHAPE),
    (dict(eps=0.0), VALUE), (dict(ss=float("inf")), VALUE), (dict(hs=float("nan")), VALUE),
    (dict(ss=1e300), VALUE),
    (dict(q=None), NULL), (dict(w=None), NULL), (dict(out=None), NULL), (dict(wo=None), NULL),
    (dict(qst=0), STRIDE), (dict(wost=0), STRIDE), (dict(osh=64), STRIDE), (dict(wost=32), STRIDE),
    # per-lane offsets inside a 4-head item must fit in 32 bits
    (dict(qsh=(1 << 28) + 8), STRIDE), (dict(osh=(1 << 30) + 8), STRIDE),
    (dict(q=A + 8), ALIGN), (dict(qsh=132), ALIGN), (dict(out=A + 4), ALIGN),
    (dict(osh=132), ALIGN), (dict(w=A + 2), ALIGN), (dict(cs=A + 4), ALIGN),
])
def test_indexer_validation(kw, status):
    assert idx(**kw) == status


def irb(**kw):
    a = dict(o=A, ost=32 * 512, osh=512, pos=A, cs=A, max_pos=4096, n=16, h=32, hpg=8, out=B,
             osg=16 * 8 * 512, ost2=8 * 512)
    a.update(kw)
    return _lib.lib().inv_rope_bf16(a["o"], a["ost"], a["osh"], a["pos"], a["cs"], a["max_pos"],
                                    a["n"], a["h"], a["hpg"], a["out"], a["osg"], a["ost2"], None)


def test_irb_zero_tokens_is_ok_without_pointers():
    assert irb(n=0, o=None, pos=None, cs=None, out=None) == OK


@host_only
@pytest.mark.parametrize("kw,status", [
    (dict(hpg=7), SHAPE), (dict(n=-1), SHAPE), (dict(max_pos=0), SHAPE),
    (dict(o=None), NULL), (dict(out=None), NULL), (dict(pos=None), NULL),
    (dict(ost=0), STRIDE), (dict(osg=0), STRIDE),
    (dict(o=A + 8), ALIGN), (dict(out=B + 8), ALIGN), (dict(osg=16 * 8 * 512 + 4), ALIGN),
    (dict(ost2=4 * 512), STRIDE),                 # token rows overlap
    (dict(out=A), STRIDE),                        # group-major over o is not in place
    (dict(out=A, osg=8 * 512, ost2=32 * 512, osh=1024, ost=64 * 512), STRIDE),
])
def test_irb_validation(kw, status):
    assert irb(**kw) == status


@host_only
def test_irb_token_major_in_place_passes_validation():
    # out == o with the token-major strides: each head overwrites its own row;
    # without a GPU the launch itself comes back as RQ_ERR_HIP
    assert irb(out=A, osg=8 * 512, ost2=32 * 512) == -6


def qf8(**kw):
    a = dict(q=A, qst=64 * 512, qsh=512, w=A, pos=A, cs=A, max_pos=8192, n=8, hq=64, hpad=128,
             eps=1e-6, fmt=0, qeps=1e-10, codes=B, sc=B)
    a.update(kw)
    return _lib.lib().qnorm_rope_fp8(a["q"], a["qst"], a["qsh"], a["w"], a["pos"], a["cs"],
                                     a["max_pos"], a["n"], a["hq"], a["hpad"], a["eps"],
                                     a["fmt"], a["qeps"], a["codes"], a["sc"], None)


def test_qf8_zero_tokens_is_ok_without_pointers():
    assert qf8(n=0, q=None, w=None, pos=None, cs=None, codes=None, sc=None) == OK


@host_only
@pytest.mark.parametrize("kw,status", [
    (dict(hpad=63), SHAPE), (dict(fmt=2), VALUE), (dict(qeps=0.0), VALUE), (dict(eps=0.0), VALUE),
    (dict(codes=None), NULL), (dict(sc=None), NULL), (dict(q=None), NULL),
    (dict(codes=B + 8), ALIGN), (dict(sc=B + 2), ALIGN), (dict(q=A + 8), ALIGN),
])
def test_qf8_validation(kw, status):
    assert qf8(**kw) == status


def kvf(**kw):
    a = dict(kv=A, kst=512, pos=A, cs=A, max_pos=8192, slots=A, n=8, cache=B, ns=1024, cst=512)
    a.update(kw)
    return _lib.lib().kv_rope_insert_full(a["kv"], a["kst"], a["pos"], a["cs"], a["max_pos"],
                                          a["slots"], a["n"], a["cache"], a["ns"], a["cst"], None)


def test_kvf_zero_tokens_is_ok_without_pointers():
    assert kvf(n=0, kv=None, pos=None, cs=None, slots=None, cache=None) == OK


@host_only
@pytest.mark.parametrize("kw,status", [
    (dict(ns=0), SHAPE), (dict(n=-2), SHAPE), (dict(max_pos=0), SHAPE),
    (dict(ns=1 << 60), SHAPE),
    (dict(cst=504), STRIDE), (dict(kst=0), STRIDE),
    (dict(kv=None), NULL), (dict(slots=None), NULL), (dict(cache=None), NULL),
    (dict(cache=B + 8), ALIGN), (dict(cst=516), ALIGN), (dict(slots=A + 4), ALIGN),
])
def test_kvf_validation(kw, status):
    assert kvf(**kw) == status


def fused_full(fp8=False, **kw):
    a = dict(q=A, qst=64 * 512, qsh=512, w=A, kv=A, kst=512, pos=A, cs=A, max_pos=8192,
             slots=A, n=8, hq=64, hpad=128, eps=1e-6, out=B, fmt=0, qeps=1e-10, sc=B,
             cache=B + 0x100000, ns=1024, cst=512)
    a.update(kw)
    L = _lib.lib()
    if fp8:
        return L.qnorm_rope_fp8_kv_rope_insert_full(
            a["q"], a["qst"], a["qsh"], a["w"], a["kv"], a["kst"], a["pos"], a["cs"],
            a["max_pos"], a["slots"], a["n"], a["hq"], a["hpad"], a["eps"], a["fmt"], a["qeps"],
            a["out"], a["sc"], a["cache"], a["ns"], a["cst"], None)
    return L.qnorm_rope_kv_rope_insert_full(
        a["q"], a["qst"], a["qsh"], a["w"], a["kv"], a["kst"], a["pos"], a["cs"], a["max_pos"],
        a["slots"], a["n"], a["hq"], a["hpad"], a["eps"], a["out"], a["cache"], a["ns"],
        a["cst"], None)


@pytest.mark.parametrize("fp8", [False, True])
def test_fused_full_zero_tokens_is_ok_without_pointers(fp8):
    assert fused_full(fp8, n=0, q=None, w=None, kv=None, pos=None, cs=None, slots=None,
                      out=None, sc=None, cache=None) == OK


@host_only
@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(hpad=63), SHAPE), (dict(ns=0), SHAPE), (dict(eps=0.0), VALUE),
    (dict(q=None), NULL), (dict(kv=None), NULL), (dict(cache=None), NULL),
    (dict(cst=100), STRIDE), (dict(kv=A + 8), ALIGN), (dict(out=B + 8), ALIGN),
])
def test_fused_full_validation(fp8, kw, status):
    assert fused_full(fp8, **kw) == status


@host_only
def test_fused_full_fp8_scale_format_checked():
    assert fused_full(True, fmt=7) == VALUE
    assert fused_full(True, qeps=0.0) == VALUE
    assert fused_full(True, sc=None) == NULL


def test_python_binding_rejects_host_tensors():
    import rope_fp8_quant_amd as rq
    o = torch.zeros((2, 8, 512), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        rq.inv_rope_fp8_quant(o, torch.zeros(2, dtype=torch.int64), torch.zeros(4, 64), 8,
                              torch.empty(1, 2, 4096, dtype=torch.uint8),
                              torch.empty(1, 2, 32))


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()


@host_only
@pytest.mark.parametrize("call,kw", [
    (irq, dict(ost=1 << 56)), (irq, dict(osh=1 << 56)), (irq, dict(osg=1 << 60)),
    (irq, dict(ost2=1 << 59)), (irq, dict(ssg=1 << 62)), (irq, dict(ssb=1 << 61)),
    (irb, dict(ost=1 << 56)), (irb, dict(osg=1 << 60)),
    (qnr, dict(qst=1 << 58)), (qnr, dict(qsh=1 << 55)),
    (qf8, dict(qst=1 << 58)),
    (kvi, dict(kst=1 << 58)), (kvi, dict(stride=1 << 60)),
    (kvf, dict(kst=1 << 58)),
    (idx, dict(qst=1 << 58)), (idx, dict(wst=1 << 62)), (idx, dict(ost=1 << 60)),
    (idx, dict(wost=1 << 61)),
], ids=lambda v: getattr(v, "__name__", None) or str(v))
def test_strides_beyond_any_address_space_are_rejected(call, kw):
    # a tensor whose strides reach past 2^56 bytes (or overflow int64 on the
    # way) cannot exist; without this the kernels' address arithmetic wraps
    assert call(**kw) == STRIDE
