"""OCP 8-bit floating point e4m3 ("e4m3fn") decoding (oracle; test infrastructure).

Format definition (OCP 8-bit Floating Point Specification, OFP8, E4M3):
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds
subnormals m/8 * 2^-6; there are no infinities; S.1111.111 is NaN, so the
largest finite magnitude is 1.110b * 2^8 = 448.

Used for the FP8 workload of "Optimizing FLUX 3 Image Klein inference on NVIDIA
Blackwell GPUs" (section "How it works": query, key and value in FP8).
"""
import numpy as np


def e4m3_decode(codes):
    """Decode uint8 codes to fp64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, val)
    return sign * val


def e4m3_table():
    """All 256 code values, index = code."""
    return e4m3_decode(np.arange(256, dtype=np.uint8))


def dequantize(codes, scales):
    """codes [B,N,H,D] uint8, scales [B,H] -> fp64 values codes * scale per (b,h)."""
    vals = e4m3_table()[np.asarray(codes, dtype=np.uint8)]
    return vals * np.asarray(scales, dtype=np.float64)[:, None, :, None]


def e4m3_round(x):
    """Round fp64 values to the nearest e4m3 value (ties to the even code, that
    is the one whose mantissa's last bit is 0), saturating at +-448 (the
    e4m3fn conversion with saturation: there is no infinity to round to).

    Written from the format: the finite non-negative values in code order are
    increasing, so the nearest one is found by a search over that sorted list.
    Returns fp64 values (the decoded rounded codes); NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    pos = e4m3_table()[:127]                      # codes 0x00..0x7E: 0 .. 448, increasing
    a = np.minimum(np.abs(x), pos[-1])
    hi = np.clip(np.searchsorted(pos, a, side="left"), 1, len(pos) - 1)
    lo = hi - 1
    d_lo, d_hi = a - pos[lo], pos[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    r = np.where(take_hi, pos[hi], pos[lo])
    r = np.where(a == pos[hi], pos[hi], r)
    return np.where(np.isnan(x), np.nan, np.copysign(r, x))

