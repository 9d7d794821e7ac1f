"""Small numpy helpers shared by the tests (no op arithmetic lives here)."""
import math

import numpy as np
import torch


def f32_bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def from_bits(u):
    return np.ascontiguousarray(u, dtype=np.uint32).view(np.float32)


def torch_e4m3(x):
    """torch's float8_e4m3fn cast (RNE) as uint8 codes."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_e4m3_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).float().numpy()


def torch_bf16(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_value(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def e4m3_ulp(v):
    """Spacing of e4m3 values at |v| (v a float64 array, |v| <= 448)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3))


def rope_angles(positions, theta=10000.0):
    """fp64 RoPE angles p * theta^(-2i/64), shape [len(positions), 32]."""
    i = np.arange(32, dtype=np.float64)
    return np.asarray(positions, dtype=np.float64)[:, None] * theta ** (-2.0 * i / 64.0)
