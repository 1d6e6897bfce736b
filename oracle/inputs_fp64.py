"""Widening of the seeded inputs to fp64 (oracle; test infrastructure).

bf16 bit patterns widen exactly (the value is the top 16 bits of a float32);
e4m3 codes widen through the format definition in ``e4m3`` times their
per-(batch, head) scale, also exactly.
"""
import numpy as np

from .e4m3 import dequantize


def bf16_to_fp64(bits):
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def inputs_to_fp64(inp):
    """Return (q, k, v) fp64 [B,N,H,D] for an ``Inputs`` record."""
    if inp.scales is None:
        return bf16_to_fp64(inp.q), bf16_to_fp64(inp.k), bf16_to_fp64(inp.v)
    s = inp.scales
    return dequantize(inp.q, s[0]), dequantize(inp.k, s[1]), dequantize(inp.v, s[2])
