"""Seeded synthetic inputs for the fused RoPE + block-FP8 ops.

This module only draws inputs; it holds none of the ops' arithmetic, and both
the GPU path's tests and the CPU oracle's tests take their inputs from it.

Recipe (every tensor is reproducible from (seed, tensor id, token chunk)):
  * random numbers: numpy's PCG64 generator seeded with
    ``[seed, tensor_id, chunk]`` where ``chunk`` = token index // 1024, so any
    token range can be drawn without drawing the tokens before it;
  * bf16 tensors: float64 draws scaled as asked, rounded to float32 by numpy,
    then to bf16 by torch's round-to-nearest-even cast; returned as uint16 bit
    patterns;
  * cos/sin cache: ``cache[p, i] = cos(p * theta**(-2i/64))`` and
    ``cache[p, 32+i] = sin(...)`` for i < 32, evaluated in float64 and
    rounded once to float32 (the standard RoPE frequency table for a 64-dim
    rotary part, theta = 10000).
"""
import numpy as np
import torch

CHUNK = 1024

# tensor ids (keep distinct per draw so tensors are independent)
T_O, T_POS, T_OUTLIER, T_Q, T_W, T_KV, T_SLOT, T_POS2 = range(8)


def _rng(seed, tensor_id, chunk=0):
    return np.random.Generator(np.random.PCG64([int(seed), int(tensor_id), int(chunk)]))


def f32_to_bf16_bits(x):
    """float32 array -> bf16 bit patterns (uint16) with torch's RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def cos_sin_cache(max_pos, theta=10000.0, rope_dim=64):
    half = rope_dim // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / rope_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def normal_bf16(shape, seed, tensor_id, std=1.0, outlier_frac=0.0, outlier_mult=20.0,
                tok_lo=0, tok_hi=None):
    """bf16 bits of N(0, std^2) draws; ``shape[0]`` is the token axis.

    With ``outlier_frac`` > 0 each element is independently (Bernoulli) scaled
    by ``outlier_mult`` before rounding.  ``tok_lo``/``tok_hi`` draw only that
    token range of the full tensor (same values as a full draw).
    """
    n = shape[0]
    tok_hi = n if tok_hi is None else tok_hi
    inner = tuple(shape[1:])
    out = np.empty((tok_hi - tok_lo,) + inner, dtype=np.uint16)
    c0 = tok_lo // CHUNK
    c1 = (tok_hi + CHUNK - 1) // CHUNK
    for c in range(c0, c1):
        a, b = c * CHUNK, min((c + 1) * CHUNK, n)
        x = _rng(seed, tensor_id, c).standard_normal((b - a,) + inner) * std
        if outlier_frac > 0:
            m = _rng(seed, T_OUTLIER * 1000 + tensor_id, c).random((b - a,) + inner)
            x = np.where(m < outlier_frac, x * outlier_mult, x)
        bits = f32_to_bf16_bits(x.astype(np.float32))
        lo, hi = max(a, tok_lo), min(b, tok_hi)
        out[lo - tok_lo:hi - tok_lo] = bits[lo - a:hi - a]
    return out


def uniform_bf16(shape, seed, tensor_id, lo, hi):
    x = _rng(seed, tensor_id).uniform(lo, hi, size=shape)
    return f32_to_bf16_bits(x.astype(np.float32))


def uniform_positions(n, max_pos, seed, tensor_id=T_POS):
    return _rng(seed, tensor_id).integers(0, max_pos, size=n, dtype=np.int64)


def slot_permutation(n, num_slots, seed, tensor_id=T_SLOT):
    """First n entries of a seeded random permutation of 0..num_slots-1."""
    return _rng(seed, tensor_id).permutation(num_slots)[:n].astype(np.int64)


# --------------------------------------------------------------- workloads
# The configurations the ops are tested and measured on (sizes as in the
# workload list; each is a plain dict so tests and the benchmark agree).

IRQ_TINY = dict(name="irq_tiny_n16_h8", N=16, H=8, hpg=8, max_pos=4096, pos="uniform",
                outliers=0.0, seed=1)
IRQ_PREFILL = dict(name="irq_prefill_n16384_h32_g4", N=16384, H=32, hpg=8, max_pos=65536,
                   pos="arange", outliers=0.01, seed=2)
IRQ_IRREGULAR = dict(name="irq_irregular_n4096_h48_hpg6", N=4096, H=48, hpg=6,
                     max_pos=4096, pos="arange", outliers=0.0, seed=5)
QNR_FORWARD = dict(name="qnr_forward_n8192_hq64_hpad128", N=8192, Hq=64, Hpad=128,
                   max_pos=8192, std=2.0, eps=1e-6, seed=3)
KVI_FORWARD = dict(name="kvi_forward_n8192_256x64", N=8192, num_blocks=256, block_size=64,
                   max_pos=8192, seed=3)
DECODE_NS = (1, 2, 4, 8, 16)


def irq_inputs(cfg, tok_lo=0, tok_hi=None):
    """(o_bits [n, H, 512], positions [n], cos_sin_cache) for an IRQ config."""
    N, H = cfg["N"], cfg["H"]
    tok_hi = N if tok_hi is None else tok_hi
    o = normal_bf16((N, H, 512), cfg["seed"], T_O, outlier_frac=cfg.get("outliers", 0.0),
                    tok_lo=tok_lo, tok_hi=tok_hi)
    if cfg["pos"] == "arange":
        pos = np.arange(N, dtype=np.int64) % cfg["max_pos"]
    else:
        pos = uniform_positions(N, cfg["max_pos"], cfg["seed"])
    return o, pos[tok_lo:tok_hi].copy(), cos_sin_cache(cfg["max_pos"])


def qnr_inputs(cfg, tok_lo=0, tok_hi=None):
    N, Hq = cfg["N"], cfg["Hq"]
    tok_hi = N if tok_hi is None else tok_hi
    q = normal_bf16((N, Hq, 512), cfg["seed"], T_Q, std=cfg.get("std", 1.0),
                    tok_lo=tok_lo, tok_hi=tok_hi)
    w = uniform_bf16((512,), cfg["seed"], T_W, 0.5, 1.5)
    pos = np.arange(N, dtype=np.int64) % cfg["max_pos"]
    return q, w, pos[tok_lo:tok_hi].copy(), cos_sin_cache(cfg["max_pos"])


def kvi_inputs(cfg):
    N = cfg["N"]
    kv = normal_bf16((N, 512), cfg["seed"], T_KV)
    pos = np.arange(N, dtype=np.int64) % cfg["max_pos"]
    slots = slot_permutation(N, cfg["num_blocks"] * cfg["block_size"], cfg["seed"])
    return kv, pos, slots, cos_sin_cache(cfg["max_pos"])
