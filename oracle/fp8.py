"""Oracle: OCP FP8 E4M3 ("e4m3fn") decoding and 128x128 block dequantisation --
TEST INFRASTRUCTURE ONLY.

Format (OCP 8-bit floating point specification, E4M3): 1 sign bit, 4
exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
subnormals m/8 * 2^-6; S.1111.111 is NaN; there are no infinities, so the
largest finite magnitude is 1.75 * 2^8 = 448.

Block scaling of the weights (reading of the "per-128 block scales" of the
fp8 workload): weight element (n, c) of an expert is code(n, c) *
scale[n // 128][c // 128], one fp32 scale per 128 x 128 block.

Token-axis requantization (MegaFlux summary, "Backward", overlapped
requantization of D_e and dZ_e; reading: the weight-gradient operands, whose
contraction runs over tokens, are quantized in blocks of beta consecutive
slots -- one planner block -- times one column): scale = amax / 448 over the
block's column and code = e4m3(value / scale), every step in fp32 (the
quantized code is an integer decided by floating point, so the oracle and the
device both decide it in fp32); an all-zero block column has scale 0 and
codes 0.

Activation rows for an fp8 x fp8 product (the fp8 MFMA path of FC1; reading:
the "per-1x128 e4m3 activations" of a block-scaled fp8 GEMM): each row is cut
into blocks of 128 consecutive features, and each block gets a power-of-two
scale 2^e, e the smallest integer with amax <= 448 * 2^e (so the largest
value maps into the top binade of e4m3), clamped to [-127, 127]; an all-zero
block has e = -127.  code = e4m3(value * 2^-e), the product exact in fp32.
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


def encode_e4m3(values) -> np.ndarray:
    """fp32 values -> e4m3fn codes: round to nearest on the e4m3 grid, ties to
    even; magnitudes above 448 saturate to 448 (no value reaches NaN)."""
    v = np.asarray(values, dtype=np.float32).astype(np.float64)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    a = np.minimum(np.abs(v), 448.0)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))        # binade; the subnormals share 2^-6's step
    step = np.power(2.0, e - 3)                              # 3 mantissa bits
    q = np.rint(a / step).astype(np.int64)                  # half-way cases to even
    up = q == 16                                             # rounded into the next binade
    e = np.where(up, e + 1, e)
    q = np.where(up, 8, q)
    normal = q >= 8
    code = np.where(normal, ((e.astype(np.int64) + 7) << 3) | (q - 8), q)
    return (sign | code).astype(np.uint8)


def quantize_token_blocks(values, block_rows: int):
    """values fp32 [rows, cols] -> (codes uint8 [rows, cols], scales fp32
    [ceil(rows / block_rows), cols]): one scale per block of block_rows
    consecutive rows and one column."""
    v = np.asarray(values, dtype=np.float32)
    rows, cols = v.shape
    nblk = (rows + block_rows - 1) // block_rows
    codes = np.zeros((rows, cols), dtype=np.uint8)
    scales = np.zeros((nblk, cols), dtype=np.float32)
    for b in range(nblk):
        blk = v[b * block_rows:(b + 1) * block_rows]
        amax = np.max(np.abs(blk), axis=0).astype(np.float32)
        sc = (amax / np.float32(448.0)).astype(np.float32)
        scales[b] = sc
        safe = np.where(sc > 0, sc, np.float32(1.0)).astype(np.float32)
        q = np.where(sc > 0, (blk / safe).astype(np.float32), np.float32(0.0))
        codes[b * block_rows:(b + 1) * block_rows] = encode_e4m3(q)
    return codes, scales


def quantize_row_blocks_pow2(values, block_cols: int = 128):
    """values fp32 [rows, cols] (cols a multiple of block_cols) -> (codes
    uint8 [rows, cols], exps int32 [rows, cols / block_cols]): per row and
    block of block_cols columns, e = ceil(log2(amax / 448)) clamped to
    [-127, 127] (-127 for a zero block), code = e4m3(value * 2^-e)."""
    v = np.asarray(values, dtype=np.float32)
    rows, cols = v.shape
    assert cols % block_cols == 0
    nb = cols // block_cols
    blk = v.reshape(rows, nb, block_cols)
    amax = np.max(np.abs(blk), axis=2).astype(np.float64)
    # ceil(log2(x)) from x = m * 2^E, m in [0.5, 1): E - 1 when m is exactly 0.5
    m, E = np.frexp(amax / 448.0)
    e = np.where(m == 0.5, E - 1, E).astype(np.int64)
    e = np.where(amax > 0, e, -127)
    e = np.clip(e, -127, 127)
    scaled = (blk.astype(np.float64) * np.power(2.0, -e)[:, :, None]).astype(np.float32)
    codes = encode_e4m3(scaled).reshape(rows, cols)
    return codes, e.astype(np.int32)


def dequant_row_blocks_pow2(codes, exps, block_cols: int = 128) -> np.ndarray:
    """Inverse of quantize_row_blocks_pow2 up to the rounding: fp64 values."""
    global _TABLE
    if _TABLE is None:
        _TABLE = decode_e4m3(np.arange(256, dtype=np.uint8))
    v = _TABLE[np.asarray(codes, dtype=np.uint8)]
    return v * np.repeat(np.power(2.0, np.asarray(exps, dtype=np.float64)), block_cols, axis=1)


def dequant_token_blocks(codes, scales, block_rows: int) -> np.ndarray:
    """Inverse of quantize_token_blocks up to the rounding: fp64 values."""
    global _TABLE
    if _TABLE is None:
        _TABLE = decode_e4m3(np.arange(256, dtype=np.uint8))
    v = _TABLE[np.asarray(codes, dtype=np.uint8)]
    s = np.repeat(np.asarray(scales, dtype=np.float64), block_rows, axis=0)[: v.shape[0]]
    return v * s
