"""ctypes loader for libropequant.so (the gfx950 HIP library).

The library is loaded on first use.  If it is missing the call raises: there
is no fallback path of any kind.
"""
import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libropequant.so")

RQ_OK = 0
RQ_SCALE_FP32 = 0
RQ_SCALE_UE8M0 = 1

EXPORTS = ("inv_rope_fp8_quant", "inv_rope_bf16", "qnorm_rope", "qnorm_rope_fp8",
           "kv_rope_quant_insert", "kv_rope_insert_full", "qnorm_rope_kv_rope_quant_insert",
           "qnorm_rope_kv_rope_insert_full", "qnorm_rope_fp8_kv_rope_insert_full",
           "indexer_q_rope_quant", "ropequant_strerror", "ropequant_abi_version")

_lock = threading.Lock()
_lib = None


class RopeQuantError(RuntimeError):
    """A libropequant entry point returned a negative status."""

    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


def lib():
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libropequant is not built ({LIB_PATH} missing); run "
                "`python -m rope_fp8_quant_amd.build` (needs hipcc for gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, D, I = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double,
                             ctypes.c_int)
        L.inv_rope_fp8_quant.argtypes = [P, I64, I64, P, P, I64, I64, I32, I32, I32, D,
                                         P, I64, I64, P, I64, I64, I64, P]
        L.inv_rope_fp8_quant.restype = I
        L.inv_rope_bf16.argtypes = [P, I64, I64, P, P, I64, I64, I32, I32, P, I64, I64, P]
        L.inv_rope_bf16.restype = I
        L.qnorm_rope.argtypes = [P, I64, I64, P, P, P, I64, I64, I32, I32, D, P, P]
        L.qnorm_rope.restype = I
        L.qnorm_rope_fp8.argtypes = [P, I64, I64, P, P, P, I64, I64, I32, I32, D, I32, D, P, P,
                                     P]
        L.qnorm_rope_fp8.restype = I
        L.kv_rope_insert_full.argtypes = [P, I64, P, P, I64, P, I64, P, I64, I64, P]
        L.kv_rope_insert_full.restype = I
        L.qnorm_rope_kv_rope_insert_full.argtypes = [P, I64, I64, P, P, I64, P, P, I64, P, I64,
                                                     I32, I32, D, P, P, I64, I64, P]
        L.qnorm_rope_kv_rope_insert_full.restype = I
        L.qnorm_rope_fp8_kv_rope_insert_full.argtypes = [P, I64, I64, P, P, I64, P, P, I64, P,
                                                         I64, I32, I32, D, I32, D, P, P, P, I64,
                                                         I64, P]
        L.qnorm_rope_fp8_kv_rope_insert_full.restype = I
        L.kv_rope_quant_insert.argtypes = [P, I64, P, P, I64, P, I64, P, I64, I64, I32, I32, D,
                                           P]
        L.kv_rope_quant_insert.restype = I
        L.qnorm_rope_kv_rope_quant_insert.argtypes = [P, I64, I64, P, P, I64, P, P, I64, P, I64,
                                                      I32, I32, D, P, P, I64, I64, I32, I32, D,
                                                      P]
        L.qnorm_rope_kv_rope_quant_insert.restype = I
        L.indexer_q_rope_quant.argtypes = [P, I64, I64, P, P, I64, P, I64, I64, I32, D, D, D,
                                           P, I64, I64, P, I64, P]
        L.indexer_q_rope_quant.restype = I
        L.ropequant_strerror.argtypes = [I]
        L.ropequant_strerror.restype = ctypes.c_char_p
        L.ropequant_abi_version.argtypes = []
        L.ropequant_abi_version.restype = I
        _lib = L
    return _lib


_fns = None


def functions():
    """The exported C entry points by name (looked up once)."""
    global _fns
    if _fns is None:
        L = lib()
        _fns = {n: getattr(L, n) for n in EXPORTS}
    return _fns


def check(fn, status):
    if status != RQ_OK:
        raise RopeQuantError(fn, status, lib().ropequant_strerror(status).decode())
