"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle runs.

This module draws numbers and encodes them; it holds none of the method's
arithmetic.  Every tensor is drawn from its own counter-style seed

    SeedSequence([0x4C4C, config, layer, chunk, pass, tensor])

as float64 N(0, 1), rounded to float32 and then, for bfloat16 inputs, to the
nearest bfloat16 (ties to even).  The arrays returned are float32 holding
exactly representable values, so both sides consume identical numbers.
"""

import numpy as np

# tensor ids inside the seed
Q, K, V, K_TXT, V_TXT, RK, RV = range(7)

SEED_TAG = 0x4C4C


def generator(config, layer=0, chunk=0, pass_=0, tensor=0):
    """The numpy Generator for one tensor of one (config, layer, chunk, pass)."""
    ss = np.random.SeedSequence([SEED_TAG, int(config), int(layer), int(chunk),
                                 int(pass_), int(tensor)])
    return np.random.default_rng(ss)


def bf16_bits(x32):
    """float32 array -> uint16 bfloat16 bit patterns, round to nearest even."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return ((u >> 16) & 0xFFFF).astype(np.uint16)


def bf16_to_f32(bits):
    """uint16 bfloat16 bit patterns -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(shape, dtype, config, layer=0, chunk=0, pass_=0, tensor=0):
    """N(0,1) draw of ``shape`` rounded to ``dtype`` ("f32" or "bf16").

    Returns a float32 array of exactly representable values.
    """
    x = generator(config, layer, chunk, pass_, tensor).standard_normal(shape)
    x32 = x.astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return bf16_to_f32(bf16_bits(x32))
    raise ValueError(dtype)


def to_torch(x32, dtype, device="cpu"):
    """float32 array of representable values -> torch tensor of ``dtype``."""
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(device)
    if dtype == "bf16":
        bits = bf16_bits(x32).view(np.int16)
        return torch.from_numpy(bits).view(torch.bfloat16).to(device)
    raise ValueError(dtype)
