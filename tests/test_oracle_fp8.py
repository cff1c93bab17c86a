"""Pins for the e4m3 decoder (oracle/fp8.py): every code against torch's
float8_e4m3fn conversion (a library routine implementing the OCP format), plus
the block-scale layout against an explicit loop."""
import numpy as np
import torch

from oracle.fp8 import decode_e4m3, dequant_blocks


def test_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = decode_e4m3(codes)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all() and nan.sum() == 2
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert np.nanmax(got) == 448.0 and decode_e4m3(np.uint8(1)) == 2.0 ** -9


def test_block_scales_layout():
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 0x7E, size=(2, 256, 384)).astype(np.uint8)
    scales = rng.random((2, 2, 3)).astype(np.float32) + 0.1
    got = dequant_blocks(codes, scales)
    vals = decode_e4m3(codes)
    for e in range(2):
        for n in (0, 127, 128, 255):
            for c in (0, 5, 128, 300, 383):
                assert got[e, n, c] == vals[e, n, c] * np.float64(scales[e, n // 128, c // 128])


# ---- token-axis requantization (encoder and block quantizer) ----------------

def test_encode_matches_torch_cast():
    from oracle.fp8 import encode_e4m3
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-4, 2.6, 100000)).astype(np.float32)
    v = np.clip(v, -448, 448)
    # half-way points between neighbouring codes go to the even mantissa
    grid = decode_e4m3(np.arange(0, 0x7F, dtype=np.uint8))
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(encode_e4m3(v), ref)


def test_encode_round_trip_and_saturation():
    from oracle.fp8 import encode_e4m3
    codes = np.arange(256, dtype=np.uint8)
    vals = decode_e4m3(codes)
    ok = ~np.isnan(vals)
    np.testing.assert_array_equal(encode_e4m3(vals[ok].astype(np.float32)), codes[ok])
    assert encode_e4m3(np.float32(1000.0)) == 0x7E and encode_e4m3(np.float32(-449.0)) == 0xFE


def test_quantize_token_blocks():
    from oracle.fp8 import dequant_token_blocks, quantize_token_blocks
    rng = np.random.default_rng(4)
    v = (rng.standard_normal((300, 40)) * 3).astype(np.float32)
    v[128:256, 7] = 0.0                               # an all-zero block column
    codes, scales = quantize_token_blocks(v, 128)
    assert scales.shape == (3, 40)
    for b in range(3):
        blk = v[b * 128:(b + 1) * 128]
        amax = np.abs(blk).max(axis=0)
        np.testing.assert_array_equal(scales[b], (amax / np.float32(448)).astype(np.float32))
        # the largest magnitude of a block column lands on the top code
        for c in range(40):
            if amax[c] > 0:
                i = int(np.argmax(np.abs(blk[:, c])))
                assert codes[b * 128 + i, c] & 0x7F == 0x7E
    assert scales[1, 7] == 0 and not codes[128:256, 7].any()
    back = dequant_token_blocks(codes, scales, 128)
    # within half a step of e4m3: 2^-4 relative, or 2^-10 of the scale below 2^-6
    bound = np.maximum(np.abs(v) * 2.0 ** -4, np.repeat(scales, 128, axis=0)[:300] * 2.0 ** -10)
    assert np.all(np.abs(back - v) <= bound * (1 + 1e-6))


# ---- activation rows: per-row blocks of 128 with power-of-two scales ----------

def test_row_blocks_pow2_exponent_boundaries():
    """e is the smallest integer with amax <= 448 * 2^e: amax = 448 * 2^k
    and one ulp below give k, one ulp above gives k + 1; 256 * 2^k still
    needs k, and 128 * 2^k fits k - 1."""
    from oracle.fp8 import quantize_row_blocks_pow2
    rows = []
    want = []
    for k in (-20, -3, 0, 1, 7):
        top = np.float32(448.0 * 2.0 ** k)
        for amax, e in ((top, k), (np.nextafter(top, np.float32(np.inf)), k + 1),
                        (np.nextafter(top, np.float32(0)), k), (np.float32(2.0 ** (k + 8)), k),
                        (np.float32(2.0 ** (k + 7)), k - 1)):
            r = np.zeros(128, dtype=np.float32)
            r[5] = -amax
            rows.append(r)
            want.append(e)
    codes, exps = quantize_row_blocks_pow2(np.stack(rows))
    np.testing.assert_array_equal(exps[:, 0], want)
    # the block maximum lands in the top binade [256, 448] of e4m3
    top = decode_e4m3(codes[np.arange(len(rows)), 5])
    assert (np.abs(top) >= 224).all() and (np.abs(top) <= 448).all()


def test_row_blocks_pow2_codes_match_torch_cast():
    """Codes are torch's e4m3fn cast of value * 2^-e (an independent encoder),
    zero blocks have e = -127 and codes 0, and every value comes back within
    half an e4m3 step of its scaled grid."""
    from oracle.fp8 import dequant_row_blocks_pow2, quantize_row_blocks_pow2
    rng = np.random.default_rng(9)
    v = (rng.standard_normal((64, 512)) * 10.0 ** rng.uniform(-3, 3, (64, 1))).astype(np.float32)
    v[3, 128:256] = 0.0
    codes, exps = quantize_row_blocks_pow2(v)
    assert exps.shape == (64, 4) and exps[3, 1] == -127 and (codes[3, 128:256] == 0).all()
    scaled = (v.reshape(64, 4, 128) * np.power(2.0, -exps.astype(np.float64))[:, :, None]).astype(np.float32)
    ref = torch.from_numpy(scaled.reshape(64, 512)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes, ref)
    back = dequant_row_blocks_pow2(codes, exps)
    step = np.repeat(np.power(2.0, exps.astype(np.float64)), 128, axis=1) * 2.0 ** -9
    grid_step = np.maximum(np.abs(back), np.abs(v)) * 2.0 ** -3
    assert (np.abs(back - v) <= np.maximum(grid_step / 2 * 1.0001, step)).all()
    # power-of-two scales change the exponent only: a block scaled by 2^j
    # gets the same codes and e + j
    c2, e2 = quantize_row_blocks_pow2((v * np.float32(2.0 ** 5)).astype(np.float32))
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(e2[exps > -127], exps[exps > -127] + 5)
