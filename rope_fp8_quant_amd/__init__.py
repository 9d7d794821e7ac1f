"""Python binding of libropequant: fused RoPE + block-FP8 ops for MI355X.

Thin argument marshalling only: each function checks the tensors the way the
op's C++ entry checks them (dtype, device, shape, contiguity where required),
then passes raw device pointers, strides and torch's current HIP stream to the
C entry point of the same name.  Every step of the computation runs in the
library's gfx950 kernels; there is no other path.  Outputs are preallocated by
the caller and written in place (the ``_out`` convention); the ``empty_*``
helpers allocate correctly shaped outputs.

Sources: the op semantics follow the analyses of vLLM PR #63540
("한 프로그램이 4개 head를 처리하게 하라: DeepSeek-V4 inverse RoPE + FP8 quant
커널 3.5배 가속기", sections 1-4) for ``inv_rope_fp8_quant`` and ``inv_rope_bf16``
and of vLLM PR
#49236 ("vLLM DeepSeek-V4 성능 최적화: Eager Break 시 Workspace 재사용 개선",
sections 1-2) for ``qnorm_rope`` and ``kv_rope_quant_insert`` and their
full-cache forms (section 2), and of vLLM PR
#46862 ("vLLM의 GLM5.2 성능 최적화: Triton 커널 융합을 통한 E2E Throughput 향상",
section 1) for ``indexer_q_rope_quant``.
"""
import threading

import torch

from ._lib import RQ_SCALE_FP32, RQ_SCALE_UE8M0, RopeQuantError, check, functions, lib

__all__ = [
    "inv_rope_fp8_quant", "inv_rope_bf16", "qnorm_rope", "qnorm_rope_fp8",
    "kv_rope_quant_insert", "kv_rope_insert_full", "qnorm_rope_kv_rope_quant_insert",
    "qnorm_rope_kv_rope_insert_full", "qnorm_rope_fp8_kv_rope_insert_full",
    "indexer_q_rope_quant", "empty_inv_rope_fp8_quant_outputs", "empty_qnorm_rope_fp8_outputs",
    "empty_kv_cache", "abi_version", "prepare", "Prepared", "RopeQuantError", "RECORD_BYTES",
    "SCALE_FMTS",
]

RECORD_BYTES = 528
SCALE_FMTS = {"fp32": RQ_SCALE_FP32, "ue8m0": RQ_SCALE_UE8M0}
_BYTE_DTYPES = (torch.uint8, torch.float8_e4m3fn)
_WORD_DTYPES = (torch.int32, torch.uint32)


def _fmt(scale_fmt):
    if scale_fmt not in SCALE_FMTS:
        raise ValueError(f"scale_fmt must be one of {sorted(SCALE_FMTS)}")
    return SCALE_FMTS[scale_fmt]


def _cuda(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _same_device(ref, *named):
    """Checks that every named tensor is on ref's device; returns its index."""
    # device indices as ints: cheaper than building torch.device objects, and
    # a CPU tensor (index -1) fails too
    d = ref.get_device()
    for t, name in named:
        if t is not None and t.get_device() != d:
            raise ValueError(f"{name} must be on {ref.device}")
    return d


# torch's handle of the current stream of a device and its current device
# index, without building Stream / device objects (the public API where this
# build lacks them)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_get_device = getattr(torch._C, "_cuda_getDevice", None) or torch.cuda.current_device

# A prepare() call in progress on this thread collects the launch here
# instead of launching it.
_capture = threading.local()


def _launch(name, fn, idx, stream, args):
    if stream is None:
        handle = (_raw_stream(idx) if _raw_stream is not None
                  else torch.cuda.current_stream(idx).cuda_stream)
    else:
        if stream.device.index != idx:
            raise ValueError(f"stream is on {stream.device}, the tensors on cuda:{idx}")
        handle = stream.cuda_stream
    if idx != _get_device():
        with torch.cuda.device(idx):
            rc = fn(*args, handle)
    else:
        rc = fn(*args, handle)
    if rc:
        check(name, rc)


def _call(name, idx, stream, *args):
    """Launch C entry point `name` on `stream` (default: torch's current stream
    of device `idx`), with that device current during the call, and raise on a
    non-OK status.  The library launches on the current HIP device, so a
    stream or tensors on another device would hand it foreign pointers."""
    if getattr(_capture, "slot", None) is not None:
        _capture.slot.append((name, idx, args))
        return
    _launch(name, functions()[name], idx, stream, args)


class Prepared:
    """One op call with its arguments checked and marshalled once: calling it
    launches the same work again (on `stream`, default torch's current stream
    of the tensors' device) with no further checks.  It keeps its tensors
    alive; they must keep their storage (no resize or set_) and are read and
    written again on every call."""

    __slots__ = ("name", "_fn", "_idx", "_args", "_keep")

    def __init__(self, name, idx, args, keep):
        self.name, self._fn, self._idx, self._args, self._keep = (
            name, functions()[name], idx, args, keep)

    def __call__(self, stream=None):
        _launch(self.name, self._fn, self._idx, stream, self._args)


def prepare(op, *args, **kwargs):
    """Check and marshal `op(*args, **kwargs)` once (any op of this module) and
    return a Prepared call that relaunches it: for loops that run the same op
    on the same buffers, where the per-call checks would cost more host time
    than the kernel."""
    _capture.slot = []
    try:
        op(*args, **kwargs)
        (name, idx, cargs), = _capture.slot
    finally:
        _capture.slot = None
    return Prepared(name, idx, cargs, (args, kwargs))


def _check_rope_inputs(positions, cos_sin_cache, n_tokens):
    """Checks positions and the table; returns the table's row count."""
    if positions.dtype != torch.int64 or positions.shape != (n_tokens,):
        raise ValueError("positions must be int64 [N]")
    if not positions.is_contiguous():
        raise ValueError("positions must be contiguous")
    cs_shape = cos_sin_cache.shape
    if (cos_sin_cache.dtype != torch.float32 or len(cs_shape) != 2 or cs_shape[1] != 64
            or not cos_sin_cache.is_contiguous()):
        raise ValueError("cos_sin_cache must be contiguous float32 [max_pos, 64]")
    return cs_shape[0]


def abi_version():
    return lib().ropequant_abi_version()


def empty_inv_rope_fp8_quant_outputs(n_tokens, n_heads, heads_per_group, device,
                                     scale_fmt="fp32"):
    """Group-major outputs: codes uint8 [G, N, hpg*512] and scales
    float32 [G, N, hpg*4] (fp32) or int32 [G, N, hpg] (ue8m0 words)."""
    G = n_heads // heads_per_group
    out = torch.empty((G, n_tokens, heads_per_group * 512), dtype=torch.uint8, device=device)
    if _fmt(scale_fmt) == RQ_SCALE_UE8M0:
        sc = torch.empty((G, n_tokens, heads_per_group), dtype=torch.int32, device=device)
    else:
        sc = torch.empty((G, n_tokens, heads_per_group * 4), dtype=torch.float32, device=device)
    return out, sc


def empty_qnorm_rope_fp8_outputs(n_tokens, q_head_padded, device, scale_fmt="fp32"):
    """Codes uint8 [N, Hpad, 512] and scales float32 [N, Hpad, 4] (fp32) or
    int32 [N, Hpad] (ue8m0 words)."""
    codes = torch.empty((n_tokens, q_head_padded, 512), dtype=torch.uint8, device=device)
    if _fmt(scale_fmt) == RQ_SCALE_UE8M0:
        sc = torch.empty((n_tokens, q_head_padded), dtype=torch.int32, device=device)
    else:
        sc = torch.empty((n_tokens, q_head_padded, 4), dtype=torch.float32, device=device)
    return codes, sc


def empty_kv_cache(num_blocks, cache_block_size, device, fill=None):
    """uint8 [num_blocks, cache_block_size * 528] paged cache."""
    if fill is None:
        return torch.empty((num_blocks, cache_block_size * RECORD_BYTES), dtype=torch.uint8,
                           device=device)
    return torch.full((num_blocks, cache_block_size * RECORD_BYTES), fill, dtype=torch.uint8,
                      device=device)


def inv_rope_fp8_quant(o, positions, cos_sin_cache, heads_per_group, out, scales,
                       scale_fmt="fp32", eps=1e-10, stream=None):
    """Inverse RoPE + block-128 e4m3 quantization of o [N, H, 512] bf16.

    out: uint8 / float8_e4m3fn [G, N, hpg*512] (any strides on the first two
    dims, last dim contiguous) - e.g. ``t.view(N, G, hpg*512).transpose(0, 1)``
    of a token-major [N, H, 512] tensor.  scales: float32 [G, N, hpg*4] for
    "fp32" or int32/uint32 [G, N, hpg] words for "ue8m0" (any strides).
    """
    fmt = _fmt(scale_fmt)
    N, H, hpg, G, o_st = _check_o(o, heads_per_group)
    max_pos = _check_rope_inputs(positions, cos_sin_cache, N)
    out_st = out.stride()
    if out.dtype not in _BYTE_DTYPES or out.shape != (G, N, hpg * 512) or out_st[2] != 1:
        raise ValueError(f"out must be uint8/float8_e4m3fn [{G}, {N}, {hpg * 512}], last dim "
                         "contiguous")
    if fmt == RQ_SCALE_UE8M0:
        if scales.dtype not in _WORD_DTYPES or scales.shape != (G, N, hpg):
            raise ValueError(f"ue8m0 scales must be int32/uint32 [{G}, {N}, {hpg}]")
    elif scales.dtype != torch.float32 or scales.shape != (G, N, hpg * 4):
        raise ValueError(f"fp32 scales must be float32 [{G}, {N}, {hpg * 4}]")
    idx = _same_device(o, (positions, "positions"), (cos_sin_cache, "cos_sin_cache"),
                       (out, "out"), (scales, "scales"))
    sc_st = scales.stride()
    _call("inv_rope_fp8_quant", idx, stream,
        o.data_ptr(), o_st[0], o_st[1], positions.data_ptr(), cos_sin_cache.data_ptr(),
        max_pos, N, H, hpg, fmt, float(eps), out.data_ptr(), out_st[0], out_st[1],
        scales.data_ptr(), sc_st[0], sc_st[1], sc_st[2])


def _check_o(o, heads_per_group):
    """Checks o; returns N, H, heads per group, groups and o's strides."""
    _cuda(o, "o")
    shape, st = o.shape, o.stride()
    if o.dtype != torch.bfloat16 or len(shape) != 3 or shape[2] != 512 or st[2] != 1:
        raise ValueError("o must be bf16 [N, H, 512] with a contiguous last dim")
    N, H, _ = shape
    hpg = int(heads_per_group)
    if hpg < 1 or H % hpg:
        raise ValueError("heads_per_group must divide the head count")
    return N, H, hpg, H // hpg, st


def inv_rope_bf16(o, positions, cos_sin_cache, heads_per_group, out, stream=None):
    """Inverse RoPE alone (the quantize-off form of inv_rope_fp8_quant): o
    [N, H, 512] bf16 into out bf16 [G, N, hpg*512] (any strides on the first
    two dims, last dim contiguous; the token-major view
    ``t.view(N, G, hpg*512).transpose(0, 1)`` of a [N, H, 512] tensor works,
    and that view of o itself rotates o in place)."""
    N, H, hpg, G, o_st = _check_o(o, heads_per_group)
    max_pos = _check_rope_inputs(positions, cos_sin_cache, N)
    out_st = out.stride()
    if out.dtype != torch.bfloat16 or out.shape != (G, N, hpg * 512) or out_st[2] != 1:
        raise ValueError(f"out must be bf16 [{G}, {N}, {hpg * 512}], last dim contiguous")
    idx = _same_device(o, (positions, "positions"), (cos_sin_cache, "cos_sin_cache"),
                       (out, "out"))
    _call("inv_rope_bf16", idx, stream,
        o.data_ptr(), o_st[0], o_st[1], positions.data_ptr(), cos_sin_cache.data_ptr(),
        max_pos, N, H, hpg, out.data_ptr(), out_st[0], out_st[1])


def _check_q_in(q_in, norm_weight, positions, cos_sin_cache):
    """Checks q_in, the norm weight and the rope inputs; returns N, Hq,
    q_in's strides, the table's row count and the device index."""
    _cuda(q_in, "q_in")
    shape, st = q_in.shape, q_in.stride()
    if q_in.dtype != torch.bfloat16 or len(shape) != 3 or shape[2] != 512 or st[2] != 1:
        raise ValueError("q_in must be bf16 [N, Hq, 512] with a contiguous last dim")
    N, Hq, _ = shape
    max_pos = _check_rope_inputs(positions, cos_sin_cache, N)
    if norm_weight is not None and (norm_weight.dtype != torch.bfloat16
                                    or norm_weight.shape != (512,)
                                    or not norm_weight.is_contiguous()):
        raise ValueError("norm_weight must be contiguous bf16 [512] or None")
    idx = _same_device(q_in, (positions, "positions"), (cos_sin_cache, "cos_sin_cache"),
                       (norm_weight, "norm_weight"))
    return N, Hq, st, max_pos, idx


def _check_q_fp8(q_in, q_fp8, q_scales, fmt, N, Hq):
    if (q_fp8.dtype not in _BYTE_DTYPES or q_fp8.dim() != 3 or q_fp8.shape[0] != N
            or q_fp8.shape[2] != 512 or not q_fp8.is_contiguous()):
        raise ValueError("q_fp8 must be contiguous uint8/float8_e4m3fn [N, q_head_padded, 512]")
    hpad = q_fp8.shape[1]
    if hpad < Hq:
        raise ValueError("q_head_padded must be >= num_heads_q")
    if fmt == RQ_SCALE_UE8M0:
        if q_scales.dtype not in _WORD_DTYPES or q_scales.shape != (N, hpad) or (
                not q_scales.is_contiguous()):
            raise ValueError(f"ue8m0 q_scales must be contiguous int32/uint32 [{N}, {hpad}]")
    elif q_scales.dtype != torch.float32 or q_scales.shape != (N, hpad, 4) or (
            not q_scales.is_contiguous()):
        raise ValueError(f"fp32 q_scales must be contiguous float32 [{N}, {hpad}, 4]")
    _same_device(q_in, (q_fp8, "q_fp8"), (q_scales, "q_scales"))
    return hpad


def _check_qnr(q_in, norm_weight, positions, cos_sin_cache, q_out):
    """_check_q_in and q_out; returns N, Hq, q_head_padded, q_in's strides,
    the table's row count and the device index."""
    N, Hq, st, max_pos, idx = _check_q_in(q_in, norm_weight, positions, cos_sin_cache)
    shape = q_out.shape
    if (q_out.dtype != q_in.dtype or len(shape) != 3 or shape[0] != N or shape[2] != 512
            or not q_out.is_contiguous()):
        raise ValueError("q_out must be contiguous bf16 [N, q_head_padded, 512]")
    if shape[1] < Hq:
        raise ValueError("q_head_padded must be >= num_heads_q")
    _same_device(q_in, (q_out, "q_out"))
    return N, Hq, shape[1], st, max_pos, idx


def _check_kvi(kv, positions, cos_sin_cache, slot_mapping, k_cache, cache_block_size):
    _cuda(kv, "kv")
    if kv.dtype != torch.bfloat16 or kv.dim() != 2 or kv.shape[1] != 512 or kv.stride(1) != 1:
        raise ValueError("kv must be bf16 [N, 512] with a contiguous last dim")
    N = kv.shape[0]
    _check_rope_inputs(positions, cos_sin_cache, N)
    if (slot_mapping.dtype != torch.int64 or slot_mapping.shape != (N,)
            or not slot_mapping.is_contiguous()):
        raise ValueError("slot_mapping must be contiguous int64 [N]")
    if k_cache.dtype != torch.uint8 or k_cache.dim() != 2 or k_cache.stride(1) != 1:
        raise ValueError("k_cache must be uint8 [num_blocks, block_bytes]")
    if k_cache.shape[1] < int(cache_block_size) * RECORD_BYTES:
        raise ValueError("k_cache block_bytes must hold cache_block_size * 528 bytes")
    _same_device(kv, (positions, "positions"), (cos_sin_cache, "cos_sin_cache"),
                 (slot_mapping, "slot_mapping"), (k_cache, "k_cache"))
    return N


def _check_kvf(kv, positions, cos_sin_cache, slot_mapping, cache):
    _cuda(kv, "kv")
    if kv.dtype != torch.bfloat16 or kv.dim() != 2 or kv.shape[1] != 512 or kv.stride(1) != 1:
        raise ValueError("kv must be bf16 [N, 512] with a contiguous last dim")
    N = kv.shape[0]
    _check_rope_inputs(positions, cos_sin_cache, N)
    if (slot_mapping.dtype != torch.int64 or slot_mapping.shape != (N,)
            or not slot_mapping.is_contiguous()):
        raise ValueError("slot_mapping must be contiguous int64 [N]")
    if (cache.dtype != torch.bfloat16 or cache.dim() != 2 or cache.shape[1] < 512
            or cache.stride(1) != 1):
        raise ValueError("cache must be bf16 [num_slots, >= 512] with a contiguous last dim")
    _same_device(kv, (positions, "positions"), (cos_sin_cache, "cos_sin_cache"),
                 (slot_mapping, "slot_mapping"), (cache, "cache"))
    return N


def qnorm_rope(q_in, norm_weight, positions, cos_sin_cache, q_out, eps=1e-6, stream=None):
    """Per-head RMSNorm + forward RoPE of q_in [N, Hq, 512] bf16 into the
    contiguous q_out [N, q_head_padded, 512] bf16; pad heads are zeroed.
    norm_weight: bf16 [512] or None.  With q_head_padded == Hq, q_out may be
    q_in itself (contiguous): each head is read before it is written."""
    N, Hq, hpad, st, max_pos, idx = _check_qnr(q_in, norm_weight, positions, cos_sin_cache,
                                               q_out)
    _call("qnorm_rope", idx, stream,
        q_in.data_ptr(), st[0], st[1], None if norm_weight is None else norm_weight.data_ptr(),
        positions.data_ptr(), cos_sin_cache.data_ptr(), max_pos, N, Hq, hpad, float(eps),
        q_out.data_ptr())


def qnorm_rope_fp8(q_in, norm_weight, positions, cos_sin_cache, q_fp8, q_scales, eps=1e-6,
                   scale_fmt="fp32", quant_eps=1e-10, stream=None):
    """qnorm_rope's q path written to FP8: block-128 e4m3 codes q_fp8
    [N, q_head_padded, 512] and scales q_scales (float32 [N, Hpad, 4], or
    int32/uint32 [N, Hpad] UE8M0 words); pad heads are quantized zero heads."""
    fmt = _fmt(scale_fmt)
    N, Hq, _, _, _ = _check_q_in(q_in, norm_weight, positions, cos_sin_cache)
    hpad = _check_q_fp8(q_in, q_fp8, q_scales, fmt, N, Hq)
    _call("qnorm_rope_fp8", q_in.get_device(), stream,
        q_in.data_ptr(), q_in.stride(0), q_in.stride(1),
        None if norm_weight is None else norm_weight.data_ptr(), positions.data_ptr(),
        cos_sin_cache.data_ptr(), cos_sin_cache.shape[0], N, Hq, hpad, float(eps), fmt,
        float(quant_eps), q_fp8.data_ptr(), q_scales.data_ptr())


def kv_rope_insert_full(kv, positions, cos_sin_cache, slot_mapping, cache, stream=None):
    """Forward RoPE of kv [N, 512] bf16 into the token-strided bf16 cache
    [num_slots, >= 512]: token t's row goes to cache[slot_mapping[t], :512]
    (skipped for a negative slot)."""
    N = _check_kvf(kv, positions, cos_sin_cache, slot_mapping, cache)
    _call("kv_rope_insert_full", kv.get_device(), stream,
        kv.data_ptr(), kv.stride(0), positions.data_ptr(), cos_sin_cache.data_ptr(),
        cos_sin_cache.shape[0], slot_mapping.data_ptr(), N, cache.data_ptr(), cache.shape[0],
        cache.stride(0))


def kv_rope_quant_insert(kv, positions, cos_sin_cache, slot_mapping, k_cache, cache_block_size,
                         scale_fmt="fp32", eps=1e-10, stream=None):
    """Forward RoPE + block-128 e4m3 quantization of kv [N, 512] bf16, each
    token's 528-byte record written at its slot of the paged uint8 cache
    k_cache [num_blocks, block_bytes] (block stride = k_cache.stride(0))."""
    fmt = _fmt(scale_fmt)
    N = _check_kvi(kv, positions, cos_sin_cache, slot_mapping, k_cache, cache_block_size)
    _call("kv_rope_quant_insert", kv.get_device(), stream,
        kv.data_ptr(), kv.stride(0), positions.data_ptr(), cos_sin_cache.data_ptr(),
        cos_sin_cache.shape[0], slot_mapping.data_ptr(), N, k_cache.data_ptr(), k_cache.shape[0],
        k_cache.stride(0), int(cache_block_size), fmt, float(eps))


def qnorm_rope_kv_rope_quant_insert(q_in, norm_weight, kv, positions, cos_sin_cache,
                                    slot_mapping, q_out, k_cache, cache_block_size, eps=1e-6,
                                    scale_fmt="fp32", quant_eps=1e-10, stream=None):
    """qnorm_rope and kv_rope_quant_insert in one launch (same results)."""
    fmt = _fmt(scale_fmt)
    N, Hq = _check_qnr(q_in, norm_weight, positions, cos_sin_cache, q_out)[:2]
    if _check_kvi(kv, positions, cos_sin_cache, slot_mapping, k_cache, cache_block_size) != N:
        raise ValueError("q_in and kv must have the same number of tokens")
    _call("qnorm_rope_kv_rope_quant_insert", q_in.get_device(), stream,
        q_in.data_ptr(), q_in.stride(0), q_in.stride(1),
        None if norm_weight is None else norm_weight.data_ptr(), kv.data_ptr(), kv.stride(0),
        positions.data_ptr(), cos_sin_cache.data_ptr(), cos_sin_cache.shape[0],
        slot_mapping.data_ptr(), N, Hq, q_out.shape[1], float(eps), q_out.data_ptr(),
        k_cache.data_ptr(), k_cache.shape[0], k_cache.stride(0), int(cache_block_size), fmt,
        float(quant_eps))


def qnorm_rope_kv_rope_insert_full(q_in, norm_weight, kv, positions, cos_sin_cache,
                                   slot_mapping, q_out, cache, eps=1e-6, stream=None):
    """Full-cache form of the fused op in one launch: qnorm_rope (q_out may be
    q_in itself) and kv_rope_insert_full."""
    N, Hq = _check_qnr(q_in, norm_weight, positions, cos_sin_cache, q_out)[:2]
    if _check_kvf(kv, positions, cos_sin_cache, slot_mapping, cache) != N:
        raise ValueError("q_in and kv must have the same number of tokens")
    _call("qnorm_rope_kv_rope_insert_full", q_in.get_device(), stream,
        q_in.data_ptr(), q_in.stride(0), q_in.stride(1),
        None if norm_weight is None else norm_weight.data_ptr(), kv.data_ptr(), kv.stride(0),
        positions.data_ptr(), cos_sin_cache.data_ptr(), cos_sin_cache.shape[0],
        slot_mapping.data_ptr(), N, Hq, q_out.shape[1], float(eps), q_out.data_ptr(),
        cache.data_ptr(), cache.shape[0], cache.stride(0))


def qnorm_rope_fp8_kv_rope_insert_full(q_in, norm_weight, kv, positions, cos_sin_cache,
                                       slot_mapping, q_fp8, q_scales, cache, eps=1e-6,
                                       scale_fmt="fp32", quant_eps=1e-10, stream=None):
    """Full-cache form of the fused op with q to FP8, in one launch:
    qnorm_rope_fp8 and kv_rope_insert_full."""
    fmt = _fmt(scale_fmt)
    N, Hq = _check_q_in(q_in, norm_weight, positions, cos_sin_cache)[:2]
    hpad = _check_q_fp8(q_in, q_fp8, q_scales, fmt, N, Hq)
    if _check_kvf(kv, positions, cos_sin_cache, slot_mapping, cache) != N:
        raise ValueError("q_in and kv must have the same number of tokens")
    _call("qnorm_rope_fp8_kv_rope_insert_full", q_in.get_device(), stream,
        q_in.data_ptr(), q_in.stride(0), q_in.stride(1),
        None if norm_weight is None else norm_weight.data_ptr(), kv.data_ptr(), kv.stride(0),
        positions.data_ptr(), cos_sin_cache.data_ptr(), cos_sin_cache.shape[0],
        slot_mapping.data_ptr(), N, Hq, hpad, float(eps), fmt, float(quant_eps),
        q_fp8.data_ptr(), q_scales.data_ptr(), cache.data_ptr(), cache.shape[0], cache.stride(0))


def indexer_q_rope_quant(q, positions, cos_sin_cache, weights, q_fp8, weights_out,
                         softmax_scale, head_scale=1.0, eps=1e-10, stream=None):
    """Indexer query path: rotate-half RoPE on dims 0..63 of q [N, H, 128] bf16
    (rotated values rounded through bf16), per-head power-of-two e4m3
    quantization into q_fp8 [N, H, 128] (uint8 / float8_e4m3fn), and the scale
    folded into weights_out[N, H] = ((weights * q_scale) * softmax_scale) *
    head_scale (float32; may be ``weights`` itself)."""
    _cuda(q, "q")
    if q.dtype != torch.bfloat16 or q.dim() != 3 or q.shape[2] != 128 or q.stride(2) != 1:
        raise ValueError("q must be bf16 [N, H, 128] with a contiguous last dim")
    N, H, _ = q.shape
    _check_rope_inputs(positions, cos_sin_cache, N)
    for t, name in ((weights, "weights"), (weights_out, "weights_out")):
        if (t.dtype != torch.float32 or t.shape != (N, H)
                or (H > 1 and t.stride(1) != 1)):
            raise ValueError(f"{name} must be float32 [N, H] with contiguous heads")
    if q_fp8.dtype not in _BYTE_DTYPES or q_fp8.shape != (N, H, 128) or (
            q_fp8.stride(2) != 1):
        raise ValueError("q_fp8 must be uint8/float8_e4m3fn [N, H, 128], last dim contiguous")
    _same_device(q, (positions, "positions"), (cos_sin_cache, "cos_sin_cache"),
                 (weights, "weights"), (q_fp8, "q_fp8"), (weights_out, "weights_out"))
    _call("indexer_q_rope_quant", q.get_device(), stream,
        q.data_ptr(), q.stride(0), q.stride(1), positions.data_ptr(), cos_sin_cache.data_ptr(),
        cos_sin_cache.shape[0], weights.data_ptr(), weights.stride(0), N, H,
        float(softmax_scale), float(head_scale), float(eps), q_fp8.data_ptr(), q_fp8.stride(0),
        q_fp8.stride(1), weights_out.data_ptr(), weights_out.stride(0))
