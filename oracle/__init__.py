"""ctypes wrapper around the CPU oracle ``libropequant_oracle.so``.

TEST INFRASTRUCTURE ONLY: the plain single-threaded C definition of the fused
RoPE + block-FP8 hot path (see ``oracle.c`` for the method, its sources and the
readings it takes).  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  It shares no code
with the HIP library and takes all inputs as host numpy arrays.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None

SCALE_FP32 = 0
SCALE_UE8M0 = 1
RECORD_BYTES = 528
# RMSNorm summation orders: "index" is the definition (left to right over the
# 512 dims); "pairwise" adds the same squares by recursive pairwise summation
# (each half-range's sum added to the other's).
SUM_ORDERS = {"index": 0, "pairwise": 1}


def _order(sum_order):
    if sum_order not in SUM_ORDERS:
        raise ValueError(f"sum_order must be one of {sorted(SUM_ORDERS)}")
    return SUM_ORDERS[sum_order]


# A test may point the wrapper at another build of oracle.c (the mutation
# check builds altered copies and expects the pins to fail on each).
LIB_ENV = "ROPEQUANT_ORACLE_LIB"


def lib():
    """Load the compiled oracle, compiling it first if it is not there."""
    global _LIB
    if _LIB is None:
        path = os.environ.get(LIB_ENV)
        if path is None:
            path = _build.LIB
            if not os.path.exists(path):
                _build.build()
        L = ctypes.CDLL(path)
        P, I64, I32, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_to_f32.restype = ctypes.c_float
        L.orc_f32_to_e4m3.argtypes = [ctypes.c_float]
        L.orc_f32_to_e4m3.restype = ctypes.c_uint8
        L.orc_pow2_ceil_exp.argtypes = [ctypes.c_float]
        L.orc_pow2_ceil_exp.restype = ctypes.c_int
        for nm in ("orc_f32_to_e4m3_n", "orc_f32_to_bf16_n", "orc_bf16_to_f32_n",
                   "orc_pow2_ceil_exp_n"):
            getattr(L, nm).argtypes = [P, P, I64]
            getattr(L, nm).restype = None
        L.orc_rope_head.argtypes = [P, P, P, ctypes.c_int]
        L.orc_rope_head.restype = None
        L.orc_quant_head.argtypes = [P, ctypes.c_int, ctypes.c_float, P, P, P]
        L.orc_quant_head.restype = None
        L.orc_sum_squares.argtypes = [P, I32, I32]
        L.orc_sum_squares.restype = ctypes.c_float
        for nm in ("orc_rmsnorm_head", "orc_rmsnorm_head_pairwise"):
            getattr(L, nm).argtypes = [P, P, ctypes.c_float, P]
            getattr(L, nm).restype = None
        L.orc_inv_rope_fp8_quant.argtypes = [P, I64, I64, P, P, I64, I64, I32, I32, I32, D,
                                             P, I64, I64, P, I64, I64, I64]
        L.orc_inv_rope_fp8_quant.restype = ctypes.c_int
        L.orc_qnorm_rope.argtypes = [P, I64, I64, P, P, P, I64, I64, I32, I32, D, P, I32]
        L.orc_qnorm_rope.restype = ctypes.c_int
        L.orc_qnorm_rope_f32.argtypes = [P, I64, I64, P, P, P, I64, I64, I32, D, P, I32]
        L.orc_qnorm_rope_f32.restype = ctypes.c_int
        L.orc_kv_rope_quant_insert.argtypes = [P, I64, P, P, I64, P, I64, P, I64, I64, I32,
                                               I32, D]
        L.orc_kv_rope_quant_insert.restype = ctypes.c_int
        L.orc_inv_rope_bf16.argtypes = [P, I64, I64, P, P, I64, I64, I32, I32, P, I64, I64]
        L.orc_inv_rope_bf16.restype = ctypes.c_int
        L.orc_qnorm_rope_fp8.argtypes = [P, I64, I64, P, P, P, I64, I64, I32, I32, D, I32, D,
                                         P, P, I32]
        L.orc_qnorm_rope_fp8.restype = ctypes.c_int
        L.orc_kv_rope_insert_full.argtypes = [P, I64, P, P, I64, P, I64, P, I64, I64]
        L.orc_kv_rope_insert_full.restype = ctypes.c_int
        F = ctypes.c_float
        L.orc_indexer_rope.argtypes = [P, P, P]
        L.orc_indexer_rope.restype = None
        L.orc_indexer_head.argtypes = [P, P, F, F, F, F, P, P, P]
        L.orc_indexer_head.restype = None
        L.orc_indexer_q_rope_quant.argtypes = [P, I64, I64, P, P, I64, P, I64, I64, I32, D, D,
                                               D, P, I64, I64, P, I64]
        L.orc_indexer_q_rope_quant.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _ptr(a):
    return None if a is None else a.ctypes.data


def _need(a, dtype, name):
    if a is None:
        return None
    if a.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {a.dtype}")
    if not a.flags.c_contiguous:
        raise ValueError(f"{name}: must be C-contiguous")
    return a


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what}: oracle status {rc}")


# ----------------------------------------------------------------- codecs

def bf16_to_f32(bits):
    """bf16 bit patterns (uint16 array) -> float32 values."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float32)
    lib().orc_bf16_to_f32_n(_ptr(bits), _ptr(out), bits.size)
    return out


def f32_to_bf16(x):
    """float32 values -> bf16 bit patterns (uint16), RNE."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_f32_to_bf16_n(_ptr(x), _ptr(out), x.size)
    return out


def e4m3_to_f32(codes):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    f = lib().orc_e4m3_to_f32
    return np.array([f(int(c)) for c in codes.ravel()], dtype=np.float32).reshape(codes.shape)


def f32_to_e4m3(x):
    """float32 values in [-448, 448] -> e4m3 codes (uint8), RNE."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().orc_f32_to_e4m3_n(_ptr(x), _ptr(out), x.size)
    return out


def pow2_ceil_exp(t):
    """Smallest k with 2**k >= t, elementwise over float32 values."""
    t = np.ascontiguousarray(t, dtype=np.float32)
    out = np.empty(t.shape, dtype=np.int32)
    lib().orc_pow2_ceil_exp_n(_ptr(t), _ptr(out), t.size)
    return out


# ------------------------------------------------------------ head steps

def rope_head(x, cs_row, inverse):
    """One 512-dim fp32 head through GPT-J RoPE on its last 64 dims."""
    x = _need(np.ascontiguousarray(x, dtype=np.float32), np.float32, "x")
    cs_row = _need(np.ascontiguousarray(cs_row, dtype=np.float32), np.float32, "cs_row")
    assert x.shape == (512,) and cs_row.shape == (64,)
    y = np.empty(512, dtype=np.float32)
    lib().orc_rope_head(_ptr(x), _ptr(y), _ptr(cs_row), 1 if inverse else 0)
    return y


def quant_head(x, scale_fmt=SCALE_FP32, eps=1e-10):
    """One 512-dim fp32 head -> (codes[512] uint8, scales[4] f32, ue8m0 word)."""
    x = _need(np.ascontiguousarray(x, dtype=np.float32), np.float32, "x")
    assert x.shape == (512,)
    codes = np.empty(512, dtype=np.uint8)
    sc = np.empty(4, dtype=np.float32)
    word = np.zeros(1, dtype=np.uint32)
    lib().orc_quant_head(_ptr(x), scale_fmt, float(np.float32(eps)), _ptr(codes), _ptr(sc),
                         _ptr(word))
    return codes, sc, int(word[0])


def sum_squares(x, sum_order="index"):
    """RMSNorm's fp32 sum of squares of x (1-D, at least one value), the
    squares added in `sum_order`."""
    x = _need(np.ascontiguousarray(x, dtype=np.float32), np.float32, "x")
    if x.ndim != 1 or x.size < 1:
        raise ValueError("x must be a non-empty vector")
    return np.float32(lib().orc_sum_squares(_ptr(x), x.size, _order(sum_order)))


def rmsnorm_head(x, weight_bits, eps, sum_order="index"):
    """RMSNorm of one 512-dim fp32 head; the squares are added in `sum_order`."""
    x = _need(np.ascontiguousarray(x, dtype=np.float32), np.float32, "x")
    w = None if weight_bits is None else np.ascontiguousarray(weight_bits, dtype=np.uint16)
    y = np.empty(512, dtype=np.float32)
    fn = lib().orc_rmsnorm_head_pairwise if _order(sum_order) else lib().orc_rmsnorm_head
    fn(_ptr(x), _ptr(w), float(np.float32(eps)), _ptr(y))
    return y


# ---------------------------------------------------------- whole ops

def inv_rope_fp8_quant(o_bits, positions, cos_sin_cache, heads_per_group,
                       scale_fmt=SCALE_FP32, eps=1e-10, layout="group"):
    """Oracle IRQ on host arrays.

    o_bits: uint16 [N, H, 512] bf16 bits; positions int64 [N];
    cos_sin_cache float32 [max_pos, 64].
    layout "group": out [G, N, hpg*512] uint8, scales [G, N, hpg*4] f32
    (UE8M0: [G, N, hpg] uint32).  layout "token": out [N, H, 512],
    scales [N, H*4] (UE8M0: [N, H]).
    """
    o_bits = _need(o_bits, np.uint16, "o")
    positions = _need(positions, np.int64, "positions")
    cos_sin_cache = _need(cos_sin_cache, np.float32, "cos_sin_cache")
    N, H, D = o_bits.shape
    assert D == 512
    hpg = int(heads_per_group)
    G = H // hpg
    if layout == "group":
        out = np.zeros((G, N, hpg * 512), dtype=np.uint8)
        osg, ost = N * hpg * 512, hpg * 512
        if scale_fmt == SCALE_UE8M0:
            sc = np.zeros((G, N, hpg), dtype=np.uint32)
            ssg, sst, ssb = N * hpg, hpg, 1
        else:
            sc = np.zeros((G, N, hpg * 4), dtype=np.float32)
            ssg, sst, ssb = N * hpg * 4, hpg * 4, 1
    else:
        out = np.zeros((N, H, 512), dtype=np.uint8)
        osg, ost = hpg * 512, H * 512
        if scale_fmt == SCALE_UE8M0:
            sc = np.zeros((N, H), dtype=np.uint32)
            ssg, sst, ssb = hpg, H, 1
        else:
            sc = np.zeros((N, H * 4), dtype=np.float32)
            ssg, sst, ssb = hpg * 4, H * 4, 1
    rc = lib().orc_inv_rope_fp8_quant(
        _ptr(o_bits), H * 512, 512, _ptr(positions), _ptr(cos_sin_cache),
        cos_sin_cache.shape[0], N, H, hpg, scale_fmt, eps,
        _ptr(out), osg, ost, _ptr(sc), ssg, sst, ssb)
    _check(rc, "inv_rope_fp8_quant")
    return out, sc


def inv_rope_bf16(o_bits, positions, cos_sin_cache, heads_per_group, layout="group"):
    """Oracle inverse RoPE with bf16 output (the IRQ kernel without quantization).

    layout "group": out uint16 [G, N, hpg*512]; layout "token": out [N, H, 512].
    """
    o_bits = _need(o_bits, np.uint16, "o")
    positions = _need(positions, np.int64, "positions")
    cos_sin_cache = _need(cos_sin_cache, np.float32, "cos_sin_cache")
    N, H, D = o_bits.shape
    assert D == 512
    hpg = int(heads_per_group)
    G = H // hpg
    if layout == "group":
        out = np.full((G, N, hpg * 512), 0xFFFF, dtype=np.uint16)
        osg, ost = N * hpg * 512, hpg * 512
    else:
        out = np.full((N, H, 512), 0xFFFF, dtype=np.uint16)
        osg, ost = hpg * 512, H * 512
    rc = lib().orc_inv_rope_bf16(_ptr(o_bits), H * 512, 512, _ptr(positions),
                                 _ptr(cos_sin_cache), cos_sin_cache.shape[0], N, H, hpg,
                                 _ptr(out), osg, ost)
    _check(rc, "inv_rope_bf16")
    return out


def qnorm_rope(q_bits, weight_bits, positions, cos_sin_cache, q_head_padded, eps,
               sum_order="index"):
    """Oracle QNR: q_bits uint16 [N, Hq, 512] -> q_out uint16 [N, Hpad, 512].
    sum_order: "index" (the RMSNorm definition) or "pairwise" (see SUM_ORDERS)."""
    q_bits = _need(q_bits, np.uint16, "q_in")
    positions = _need(positions, np.int64, "positions")
    cos_sin_cache = _need(cos_sin_cache, np.float32, "cos_sin_cache")
    if weight_bits is not None:
        weight_bits = _need(weight_bits, np.uint16, "weight")
    N, Hq, D = q_bits.shape
    assert D == 512
    q_out = np.full((N, q_head_padded, 512), 0xFFFF, dtype=np.uint16)
    rc = lib().orc_qnorm_rope(_ptr(q_bits), Hq * 512, 512, _ptr(weight_bits), _ptr(positions),
                              _ptr(cos_sin_cache), cos_sin_cache.shape[0], N, Hq,
                              q_head_padded, eps, _ptr(q_out), _order(sum_order))
    _check(rc, "qnorm_rope")
    return q_out


def qnorm_rope_f32(q_bits, weight_bits, positions, cos_sin_cache, eps, sum_order="index"):
    """The fp32 values the q paths round (RMSNorm, then forward RoPE): float32
    [N, Hq, 512] for the live heads of q_bits uint16 [N, Hq, 512]."""
    q_bits = _need(q_bits, np.uint16, "q_in")
    positions = _need(positions, np.int64, "positions")
    cos_sin_cache = _need(cos_sin_cache, np.float32, "cos_sin_cache")
    if weight_bits is not None:
        weight_bits = _need(weight_bits, np.uint16, "weight")
    N, Hq, D = q_bits.shape
    assert D == 512
    z = np.empty((N, Hq, 512), dtype=np.float32)
    rc = lib().orc_qnorm_rope_f32(_ptr(q_bits), Hq * 512, 512, _ptr(weight_bits),
                                  _ptr(positions), _ptr(cos_sin_cache), cos_sin_cache.shape[0],
                                  N, Hq, eps, _ptr(z), _order(sum_order))
    _check(rc, "qnorm_rope_f32")
    return z


def qnorm_rope_fp8(q_bits, weight_bits, positions, cos_sin_cache, q_head_padded, eps,
                   scale_fmt=SCALE_FP32, quant_eps=1e-10, sum_order="index"):
    """Oracle q path into FP8: q_bits uint16 [N, Hq, 512] -> (codes uint8
    [N, Hpad, 512], scales f32 [N, Hpad, 4] or, UE8M0, uint32 [N, Hpad])."""
    q_bits = _need(q_bits, np.uint16, "q_in")
    positions = _need(positions, np.int64, "positions")
    cos_sin_cache = _need(cos_sin_cache, np.float32, "cos_sin_cache")
    if weight_bits is not None:
        weight_bits = _need(weight_bits, np.uint16, "weight")
    N, Hq, D = q_bits.shape
    assert D == 512
    codes = np.full((N, q_head_padded, 512), 0xCD, dtype=np.uint8)
    if scale_fmt == SCALE_UE8M0:
        sc = np.full((N, q_head_padded), 0xDEADBEEF, dtype=np.uint32)
    else:
        sc = np.full((N, q_head_padded, 4), -1.0, dtype=np.float32)
    rc = lib().orc_qnorm_rope_fp8(_ptr(q_bits), Hq * 512, 512, _ptr(weight_bits),
                                  _ptr(positions), _ptr(cos_sin_cache), cos_sin_cache.shape[0],
                                  N, Hq, q_head_padded, eps, scale_fmt, quant_eps, _ptr(codes),
                                  _ptr(sc), _order(sum_order))
    _check(rc, "qnorm_rope_fp8")
    return codes, sc


def kv_rope_insert_full(kv_bits, positions, cos_sin_cache, slot_mapping, cache):
    """Oracle kv path into a token-strided bf16 cache: writes rows of ``cache``
    (uint16 [num_slots, row_elems], row_elems >= 512) in place and returns it."""
    kv_bits = _need(kv_bits, np.uint16, "kv")
    positions = _need(positions, np.int64, "positions")
    cos_sin_cache = _need(cos_sin_cache, np.float32, "cos_sin_cache")
    slot_mapping = _need(slot_mapping, np.int64, "slot_mapping")
    cache = _need(cache, np.uint16, "cache")
    N, D = kv_bits.shape
    assert D == 512
    ns, row = cache.shape
    rc = lib().orc_kv_rope_insert_full(_ptr(kv_bits), 512, _ptr(positions),
                                       _ptr(cos_sin_cache), cos_sin_cache.shape[0],
                                       _ptr(slot_mapping), N, _ptr(cache), ns, row)
    _check(rc, "kv_rope_insert_full")
    return cache


def kv_rope_quant_insert(kv_bits, positions, cos_sin_cache, slot_mapping, k_cache,
                         cache_block_size, block_stride_bytes=None, scale_fmt=SCALE_FP32,
                         eps=1e-10):
    """Oracle KVI: writes records into ``k_cache`` (uint8 [num_blocks, block_bytes])
    in place and returns it."""
    kv_bits = _need(kv_bits, np.uint16, "kv")
    positions = _need(positions, np.int64, "positions")
    cos_sin_cache = _need(cos_sin_cache, np.float32, "cos_sin_cache")
    slot_mapping = _need(slot_mapping, np.int64, "slot_mapping")
    k_cache = _need(k_cache, np.uint8, "k_cache")
    N, D = kv_bits.shape
    assert D == 512
    nb, bb = k_cache.shape
    stride = bb if block_stride_bytes is None else int(block_stride_bytes)
    rc = lib().orc_kv_rope_quant_insert(_ptr(kv_bits), 512, _ptr(positions),
                                        _ptr(cos_sin_cache), cos_sin_cache.shape[0],
                                        _ptr(slot_mapping), N, _ptr(k_cache), nb, stride,
                                        cache_block_size, scale_fmt, eps)
    _check(rc, "kv_rope_quant_insert")
    return k_cache


# ------------------------------------------------------------- indexer

def indexer_rope(x, cs_row):
    """Rotate-half RoPE (with the bf16 round trip) of one 128-dim fp32 head."""
    x = _need(np.ascontiguousarray(x, dtype=np.float32), np.float32, "x")
    cs_row = _need(np.ascontiguousarray(cs_row, dtype=np.float32), np.float32, "cs_row")
    assert x.shape == (128,) and cs_row.shape == (64,)
    y = np.empty(128, dtype=np.float32)
    lib().orc_indexer_rope(_ptr(x), _ptr(cs_row), _ptr(y))
    return y


def indexer_head(x, cs_row, w, softmax_scale, head_scale=1.0, eps=1e-10):
    """One 128-dim fp32 head -> (codes[128] uint8, w_out f32, q_scale f32)."""
    x = _need(np.ascontiguousarray(x, dtype=np.float32), np.float32, "x")
    cs_row = _need(np.ascontiguousarray(cs_row, dtype=np.float32), np.float32, "cs_row")
    assert x.shape == (128,) and cs_row.shape == (64,)
    codes = np.empty(128, dtype=np.uint8)
    wo = np.zeros(1, dtype=np.float32)
    qs = np.zeros(1, dtype=np.float32)
    lib().orc_indexer_head(_ptr(x), _ptr(cs_row), float(np.float32(eps)),
                           float(np.float32(softmax_scale)), float(np.float32(head_scale)),
                           float(np.float32(w)), _ptr(codes), _ptr(wo), _ptr(qs))
    return codes, wo[0], qs[0]


def indexer_q_rope_quant(q_bits, positions, cos_sin_cache, weights, softmax_scale,
                         head_scale=1.0, eps=1e-10):
    """Oracle indexer path: q_bits uint16 [N, H, 128], weights f32 [N, H] ->
    (q_fp8 uint8 [N, H, 128], weights_out f32 [N, H])."""
    q_bits = _need(q_bits, np.uint16, "q")
    positions = _need(positions, np.int64, "positions")
    cos_sin_cache = _need(cos_sin_cache, np.float32, "cos_sin_cache")
    weights = _need(weights, np.float32, "weights")
    N, H, D = q_bits.shape
    assert D == 128 and weights.shape == (N, H)
    out = np.zeros((N, H, 128), dtype=np.uint8)
    wo = np.zeros((N, H), dtype=np.float32)
    rc = lib().orc_indexer_q_rope_quant(_ptr(q_bits), H * 128, 128, _ptr(positions),
                                        _ptr(cos_sin_cache), cos_sin_cache.shape[0],
                                        _ptr(weights), H, N, H, softmax_scale, head_scale, eps,
                                        _ptr(out), H * 128, 128, _ptr(wo), H)
    _check(rc, "indexer_q_rope_quant")
    return out, wo


def qnorm_rope_kv_rope_quant_insert(q_bits, weight_bits, kv_bits, positions, cos_sin_cache,
                                    slot_mapping, k_cache, q_head_padded, cache_block_size,
                                    eps=1e-6, scale_fmt=SCALE_FP32, quant_eps=1e-10,
                                    block_stride_bytes=None, sum_order="index"):
    """The fused op is, by definition, both ops on the same positions."""
    q_out = qnorm_rope(q_bits, weight_bits, positions, cos_sin_cache, q_head_padded, eps,
                       sum_order)
    kv_rope_quant_insert(kv_bits, positions, cos_sin_cache, slot_mapping, k_cache,
                         cache_block_size, block_stride_bytes, scale_fmt, quant_eps)
    return q_out, k_cache
