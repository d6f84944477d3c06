"""Pins of the oracle's 8-bit latent cache (E4M3 codes, per-128 fp32 scales).

The E4M3 decoding is pinned to torch's float8_e4m3fn (a library routine) and
to closed-form values; the rounding to torch's conversion and to hand-made
ties; the quantiser to its defining bounds.
"""
import numpy as np
import pytest
import torch

import oracle as O


def test_e4m3_decode_matches_library_and_closed_forms():
    v = O.e4m3_value(np.arange(256))
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(v), np.isnan(lib))
    assert np.array_equal(v[~np.isnan(v)], lib[~np.isnan(lib)])
    assert v[0x7E] == 448.0 and v[0x38] == 1.0 and v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6
    assert v[0x07] == 7 / 8 * 2.0 ** -6 and np.signbit(v[0x80]) and v[0x80] == 0.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.all(np.diff(v[:0x7F]) > 0)          # codes 0..126 increase


def test_e4m3_rounding_matches_library_conversion():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-448, 448, 60000),
                        np.sign(rng.standard_normal(60000)) * np.exp2(rng.uniform(-13, 8.8, 60000))])
    x = np.clip(x, -448, 448).astype(np.float32)
    got = O.round_to_e4m3(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_e4m3_ties_go_to_the_even_code():
    assert O.round_to_e4m3(np.array([1.0625]))[0] == 0x38      # between 1 (0x38) and 1.125 (0x39)
    assert O.round_to_e4m3(np.array([1.1875]))[0] == 0x3A      # between 1.125 and 1.25 (0x3A)
    assert O.round_to_e4m3(np.array([0.5 * 2.0 ** -9]))[0] == 0x00
    assert O.round_to_e4m3(np.array([1.5 * 2.0 ** -9]))[0] == 0x02
    assert O.round_to_e4m3(np.array([7.5 / 8 * 2.0 ** -6]))[0] == 0x08   # subnormal max / min normal
    assert O.round_to_e4m3(np.array([-1.0625]))[0] == 0xB8
    exact = O.e4m3_value(np.arange(0x7F))
    assert np.array_equal(O.round_to_e4m3(exact), np.arange(0x7F, dtype=np.uint8))
    with pytest.raises(ValueError):
        O.round_to_e4m3(np.array([449.0]))


def test_quantiser_scale_bounds_and_layout():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((64, 512)) * np.exp2(rng.uniform(-6, 6, (64, 1)))).astype(np.float32)
    x[3, 128:256] = 0.0                               # an all-zero group
    codes, scales = O.quantize_latent_fp8(x)
    assert codes.dtype == np.uint8 and scales.dtype == np.float32 and scales.shape == (64, 4)
    amax = np.abs(x.reshape(64, 4, 128)).max(axis=-1)
    np.testing.assert_array_equal(scales, (amax / np.float32(448.0)).astype(np.float32))
    assert scales[3, 1] == 0 and np.all(codes[3, 128:256] == 0)
    deq = O.dequantize_latent_fp8(codes, scales)
    err = np.abs(deq - x.astype(np.float64))
    sc = np.repeat(scales.astype(np.float64), 128, axis=1)
    # three mantissa bits: half a step is 2^-4 of the value above 2^-6 * scale,
    # 2^-10 * scale below it
    bound = np.maximum(np.abs(x) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)
    # the group maximum lands on the largest code
    g = x.reshape(64, 4, 128)
    top = np.abs(g).argmax(axis=-1)
    c4 = codes.reshape(64, 4, 128)
    for r in range(64):
        for k in range(4):
            if scales[r, k] > 0:
                assert c4[r, k, top[r, k]] & 0x7F == 0x7E
    row = O.fp8_cache_row_bytes(codes[:2], scales[:2], np.arange(128, dtype=np.uint16).reshape(2, 64))
    assert row.shape == (2, 656)
    assert np.array_equal(row[:, :512], codes[:2])
    assert np.array_equal(row[:, 512:528].view("<f4"), scales[:2])
    assert np.array_equal(row[:, 528:].view("<u2"), np.arange(128).reshape(2, 64))


def test_planted_rounding_mistakes_are_caught():
    # rounding half away from zero, or truncation, must fail the pins above
    x = np.array([1.0625, 1.1875, 1.03])
    good = O.round_to_e4m3(x)
    away = np.array([0x39, 0x3A, 0x38], dtype=np.uint8)      # what half-away-from-zero gives
    trunc = np.array([0x38, 0x39, 0x38], dtype=np.uint8)
    assert not np.array_equal(good, away) and not np.array_equal(good, trunc)
