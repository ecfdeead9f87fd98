"""Pins of the oracle's cache writer and E4M3FN encoder against what the
format and the mathematics fix: the code table itself, torch's float8_e4m3fn
cast (a library round-to-nearest-even conversion), hand-derived records, the
independent quantiser of the input generator, and error bounds."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

FINITE = [c for c in range(256) if c not in (0x7F, 0xFF)]


def test_every_finite_code_round_trips():
    for c in FINITE:
        assert oracle.e4m3_encode(oracle.e4m3_value(c)) == c, hex(c)


def test_hand_derived_ties_and_limits():
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39): the even code wins
    assert oracle.e4m3_encode(1.0625) == 0x38
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A)
    assert oracle.e4m3_encode(1.1875) == 0x3A
    # 2^-10 is half the smallest subnormal 2^-9: tie between 0 and 0x01
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00
    # 3 * 2^-10 lies halfway between 0x01 and 0x02
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02
    # the largest finite magnitude and its negative; signed zero keeps its sign
    assert oracle.e4m3_encode(448.0) == 0x7E and oracle.e4m3_encode(-448.0) == 0xFE
    assert oracle.e4m3_encode(0.0) == 0x00 and oracle.e4m3_encode(-0.0) == 0x80
    # 432 lies halfway between 416 (0x7D) and 448 (0x7E)
    assert oracle.e4m3_encode(432.0) == 0x7E


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_encoder_matches_torch_rounding_on_midpoints_and_random_values():
    vals = np.array([oracle.e4m3_value(c) for c in range(127)], dtype=np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # exact in fp32
    rng = np.random.default_rng(5)
    rand = np.concatenate([
        rng.uniform(-448, 448, 3000), rng.normal(0, 1, 3000), rng.normal(0, 0.01, 2000),
        mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1000))
    ]).astype(np.float32)
    ref = _torch_e4m3(rand)
    got = np.array([oracle.e4m3_encode(float(x)) for x in rand], dtype=np.uint8)
    np.testing.assert_array_equal(got, ref)


def test_record_of_a_hand_built_row():
    row = np.zeros(576, dtype=np.float32)
    row[0:4] = [448.0, -448.0, 1.0, -0.0]           # tile 0: amax 448 -> scale 1
    # tile 1 stays zero -> scale 0, codes 0
    row[256:260] = [2.0, 1.0, 0.5, -2.0]             # tile 2: amax 2 -> scale 2/448
    row[384] = 3.0                                   # tile 3: amax 3
    row[385] = 3.0 * 2.0 ** -12                      # -> 448 * 2^-12 = 0.109375
    row[386] = 3.0 * 2.0 ** -15                      # -> 448 * 2^-15 = 7 * 2^-9, subnormal
    row[512:] = np.arange(64, dtype=np.float32) - 32  # RoPE, copied
    bits = W.bf16_bits(row)
    rec = oracle.fp8_record_from_row(bits)
    scales = rec[512:528].view("<f4")
    assert scales[0] == np.float32(1.0) and scales[1] == 0.0
    assert scales[2] == np.float32(2.0) / np.float32(448.0)
    assert scales[3] == np.float32(3.0) / np.float32(448.0)
    assert list(rec[0:4]) == [0x7E, 0xFE, 0x38, 0x80]
    assert not rec[4:128].any() and not rec[128:256].any()
    # 2 / s = 448 (0x7E), 1 / s = 224 = 1.75 * 2^7 (0x76), 0.5 / s = 112 (0x6E)
    assert list(rec[256:260]) == [0x7E, 0x76, 0x6E, 0xFE]
    # 448 * 2^-12 = 0.109375 = 1.75 * 2^-4 -> exponent field 3, mantissa 6: 0x1E
    assert rec[384] == 0x7E and rec[385] == 0x1E
    # 7 * 2^-9 = (7 / 8) * 2^-6: exponent field 0, mantissa 7
    assert rec[386] == 0x07
    np.testing.assert_array_equal(rec[528:].view("<u2"), bits[512:])


def test_oracle_records_equal_the_input_generators_quantiser():
    # two independent implementations of the same rule: the generator's (numpy
    # fp32 division + torch cast) and the oracle's (C fp32 + code search)
    rng = np.random.default_rng(8)
    x = rng.normal(0, 1, (300, 576)).astype(np.float32)
    x[:, :128] *= np.exp2(rng.integers(-20, 8, size=(300, 1))).astype(np.float32)
    x[7, 128:256] = 0.0   # an all-zero tile
    x[9, 256] = -0.0
    bits = W.bf16_bits(x)
    ref = W.quantize_fp8_records(bits)
    got = np.stack([oracle.fp8_record_from_row(r) for r in bits])
    np.testing.assert_array_equal(got, ref)


def test_dequantised_record_is_within_half_a_code_step():
    rng = np.random.default_rng(9)
    bits = W.bf16_bits(rng.normal(0, 3, (64, 576)).astype(np.float32))
    vals = np.array([oracle.e4m3_value(c) for c in range(127)])
    for r in bits:
        rec = oracle.fp8_record_from_row(r)
        deq = oracle.fp8_record_values(rec)[:512]
        x = W.bf16_to_f32(r)[:512].astype(np.float64)
        scale = np.repeat(rec[512:528].view("<f4").astype(np.float64), 128)
        # the gap between neighbouring codes around |x / scale| bounds the error
        idx = np.searchsorted(vals, np.abs(x / scale)).clip(1, 126)
        gap = vals[idx] - vals[idx - 1]
        assert np.all(np.abs(deq - x) <= 0.5 * gap * scale * (1 + 1e-6) + 1e-30)


@pytest.mark.parametrize("kind", [0, 1])
def test_writer_places_rows_at_the_end_of_each_request_and_nothing_else(kind):
    rng = np.random.default_rng(10 + kind)
    seqlens = np.array([1, 70, 0, 130], dtype=np.int32)
    n_new = 2
    pages = 8
    bt = np.full((4, 3), -1, dtype=np.int32)
    perm = rng.permutation(pages).astype(np.int32)
    bt[0, 0], bt[1, :2], bt[3, :3] = perm[0], perm[1:3], perm[3:6]
    shape = (pages, 64, 576) if kind == 0 else (pages, 64, 656)
    dtype = np.uint16 if kind == 0 else np.uint8
    cache = rng.integers(0, 1 << (16 if kind == 0 else 8), size=shape).astype(dtype)
    k_new = W.bf16_bits(rng.normal(0, 1, (4, n_new, 576)).astype(np.float32))
    out = oracle.kv_write(k_new, bt, seqlens, cache, kind)
    expect = cache.copy()
    for b, L in enumerate(seqlens):
        for i in range(n_new):
            pos = L - n_new + i
            if pos < 0:
                continue  # request 0 has one token: its first new row has no place
            slot = expect[bt[b, pos // 64], pos % 64]
            slot[:] = k_new[b, i] if kind == 0 else oracle.fp8_record_from_row(k_new[b, i])
    np.testing.assert_array_equal(out, expect)
    # exactly the written slots changed: 1 + 2 + 0 + 2 tokens
    changed = np.any(out != cache, axis=-1).sum()
    assert changed == 5
