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
