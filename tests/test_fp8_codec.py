"""Pins for the oracle's E4M3FN decode and FP8 record layout."""
import math

import numpy as np
import torch

import oracle
import workloads as W


def test_all_256_codes_match_closed_form_and_torch():
    torch_vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        v = oracle.e4m3_value(c)
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 15
        m = c & 7
        if e == 15 and m == 7:
            assert math.isnan(v) and math.isnan(torch_vals[c])
            continue
        closed = s * (2.0 ** (e - 7) * (1 + m / 8) if e else 2.0 ** -6 * (m / 8))
        assert v == closed == torch_vals[c], c


def test_landmark_codes():
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0xFE) == -448.0
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x00) == 0.0


def test_record_dequantises_within_e4m3_rounding():
    rng = np.random.Generator(np.random.PCG64(5))
    x = rng.standard_normal((8, 576), dtype=np.float32)
    x[3, 128:256] = 0.0          # an all-zero tile: scale 0, codes 0
    x[4, :128] *= 1000.0         # tiles with very different ranges
    bits = W.bf16_bits(x)
    recs = W.quantize_fp8_records(bits)
    vals = W.bf16_to_f32(bits).astype(np.float64)
    for t in range(8):
        k = oracle.fp8_record_values(recs[t])
        # RoPE slice is bf16 and exact
        np.testing.assert_array_equal(k[512:], vals[t, 512:])
        for tile in range(4):
            sl = slice(128 * tile, 128 * tile + 128)
            amax = np.abs(vals[t, sl]).max()
            scale = amax / 448.0
            err = np.abs(k[sl] - vals[t, sl])
            bound = np.maximum(2.0 ** -4 * np.abs(vals[t, sl]), 2.0 ** -10 * scale) * (1 + 1e-6) + 1e-30
            assert np.all(err <= bound), (t, tile)
            if amax > 0:
                j = int(np.argmax(np.abs(vals[t, sl])))
                assert abs(abs(k[sl][j]) - amax) <= 2e-7 * amax
            else:
                assert np.all(k[sl] == 0)


def test_scale_of_each_tile_sits_at_its_offset():
    rec = np.zeros(656, dtype=np.uint8)
    rec[:512] = 0x38  # every code decodes to 1.0
    rec[512:528] = np.array([1.0, 2.0, 4.0, 8.0], dtype="<f4").view(np.uint8)
    rec[528:656] = W.bf16_bits(np.arange(64, dtype=np.float32)).astype("<u2").view(np.uint8)
    k = oracle.fp8_record_values(rec)
    for tile, s in enumerate([1.0, 2.0, 4.0, 8.0]):
        assert np.all(k[128 * tile:128 * tile + 128] == s)
    np.testing.assert_array_equal(k[512:], np.arange(64))
