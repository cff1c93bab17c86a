"""Oracle: OCP FP8 E4M3 ("e4m3fn") decoding and 128x128 block dequantisation --
TEST INFRASTRUCTURE ONLY.

Format (OCP 8-bit floating point specification, E4M3): 1 sign bit, 4
exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
subnormals m/8 * 2^-6; S.1111.111 is NaN; there are no infinities, so the
largest finite magnitude is 1.75 * 2^8 = 448.

Block scaling of the weights (reading of the "per-128 block scales" of the
fp8 workload): weight element (n, c) of an expert is code(n, c) *
scale[n // 128][c // 128], one fp32 scale per 128 x 128 block.
"""
from __future__ import annotations

import numpy as np


def decode_e4m3(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = c & 0x7
    normal = sign * (1.0 + man / 8.0) * np.power(2.0, ex - 7.0)
    sub = sign * (man / 8.0) * 2.0 ** -6
    out = np.where(ex == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


_TABLE = None


def dequant_blocks(codes, scales) -> np.ndarray:
    """codes uint8 [..., N, K], scales fp32 [..., N/128, K/128] -> fp64 [..., N, K]."""
    global _TABLE
    if _TABLE is None:
        _TABLE = decode_e4m3(np.arange(256, dtype=np.uint8))   # every code, decoded once
    v = _TABLE[np.asarray(codes, dtype=np.uint8)]
    s = np.asarray(scales, dtype=np.float64)
    s = np.repeat(np.repeat(s, 128, axis=-2), 128, axis=-1)
    return v * s
