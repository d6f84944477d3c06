"""Pins of the oracle's YaRN scale, YaRN frequencies, rotation and bf16 rounding.

Each check compares with something other than the oracle's own formula: the
textbook RoPE frequencies, YaRN's wavelength thresholds, complex-number
rotation, group properties of rotations, or torch's own bf16 conversion.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

SIGMA_LITERAL = 0.14467962580268925      # (0.1 ln 64 + 1)^2 / sqrt(192), fp64
MSCALE_LITERAL = 1.4158883083359672      # 0.1 ln 64 + 1


def test_mscale_and_softmax_scale_values():
    assert O.yarn_get_mscale(64.0, 1.0) == pytest.approx(MSCALE_LITERAL, rel=1e-15)
    assert O.softmax_scale() == pytest.approx(SIGMA_LITERAL, rel=1e-15)
    # no YaRN: the plain 1/sqrt(d_k) of scaled dot-product attention, d_k = 128 + 64
    assert O.yarn_get_mscale(1.0, 1.0) == 1.0
    no_yarn = dict(O.ROPE_SCALING, factor=1.0)
    assert O.softmax_scale(rope_scaling=no_yarn) == pytest.approx(1 / math.sqrt(192), rel=1e-15)


def test_factor_one_is_textbook_rope():
    # RoFormer frequencies theta_i = base^(-2i/d)
    no_yarn = dict(O.ROPE_SCALING, factor=1.0)
    f = O.yarn_inv_freq(64, 10000.0, no_yarn)
    want = np.array([10000.0 ** (-2.0 * i / 64) for i in range(32)])
    np.testing.assert_allclose(f, want, rtol=1e-15)


def test_yarn_frequency_regions_follow_the_wavelength_thresholds():
    # YaRN: a pair that turns more than beta_fast times over the original
    # context keeps its frequency; one that turns fewer than beta_slow times is
    # interpolated by the full factor.  Turns r_i = orig / wavelength_i.
    f = O.yarn_inv_freq()
    base = np.array([10000.0 ** (-2.0 * i / 64) for i in range(32)])
    turns = 4096 * base / (2 * math.pi)
    keep = turns > 32
    interp = turns < 1
    assert keep.sum() == 11 and interp.sum() == 9          # pairs 0..10 and 23..31
    np.testing.assert_allclose(f[keep], base[keep], rtol=1e-15)
    np.testing.assert_allclose(f[interp], base[interp] / 64, rtol=1e-15)
    mid = ~keep & ~interp
    assert np.all(f[mid] < base[mid]) and np.all(f[mid] > base[mid] / 64)
    assert np.all(np.diff(f) < 0)
    assert O.yarn_correction_range() == (10, 23)


GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "yarn_ramp_page1.json")


def _interp_weight(f):
    """Weight w_i of the interpolated frequency in f_i = base_i (1 - w_i) + base_i / 64 w_i."""
    base = np.array([10000.0 ** (-2.0 * i / 64) for i in range(32)])
    return (base - f) / (base - base / 64)


def test_yarn_ramp_interior_is_linear_in_the_pair_index():
    # Fixture: the interpolation weights of the index-linear reading at ramp
    # pairs, as exact fractions (i - 10) / 13; the ramp ends 10 and 23 follow
    # from the printed beta_fast / beta_slow (see the region test above).
    with open(GOLDEN) as fh:
        g = json.load(fh)
    w = _interp_weight(O.yarn_inv_freq())
    for pair, (num, den) in g["interpolated_weight"].items():
        assert w[int(pair)] == pytest.approx(num / den, abs=1e-12), pair


def test_a_ramp_over_the_rotation_count_fails_the_ramp_pin():
    # The same blend with the weight written over the rotation count r (the
    # paper's gamma(r)) agrees at the region ends and disagrees inside: the pin
    # above tells the two forms apart.
    with open(GOLDEN) as fh:
        g = json.load(fh)
    base = np.array([10000.0 ** (-2.0 * i / 64) for i in range(32)])
    r = 4096 * base / (2 * math.pi)
    gamma = np.clip((r - 1.0) / (32.0 - 1.0), 0.0, 1.0)
    f_r = base * gamma + base / 64 * (1.0 - gamma)
    w_r = _interp_weight(f_r)
    wrong = [p for p, (num, den) in g["interpolated_weight"].items() if abs(w_r[int(p)] - num / den) > 1e-3]
    assert {"13", "16", "20"} <= set(wrong)


def _rot_complex(x, pos, inv_freq):
    k = x.shape[-1] // 2
    z = (x[..., :k] + 1j * x[..., k:]) * np.exp(1j * np.asarray(pos, float)[..., None] * inv_freq)
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rotation_equals_complex_multiplication():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64))
    pos = np.array([0, 1, 4095, 131071, 262143])
    f = O.yarn_inv_freq()
    np.testing.assert_allclose(O.rope_rotate(x, pos, f), _rot_complex(x, pos, f), rtol=0, atol=1e-12)


def test_rotation_group_properties():
    rng = np.random.default_rng(2)
    f = O.yarn_inv_freq()
    q = rng.standard_normal(64)
    k = rng.standard_normal(64)
    np.testing.assert_array_equal(O.rope_rotate(q, 0, f), q)                  # identity at 0
    r = O.rope_rotate(q, 12345, f)
    np.testing.assert_allclose(r[:32] ** 2 + r[32:] ** 2, q[:32] ** 2 + q[32:] ** 2, rtol=1e-13)
    np.testing.assert_allclose(O.rope_rotate(O.rope_rotate(q, 700, f), 300, f),
                               O.rope_rotate(q, 1000, f), atol=1e-12)
    for m, n, d in [(10, 3, 5), (1000, 999, 200000), (262143, 0, -7)]:
        a = O.rope_rotate(q, m, f) @ O.rope_rotate(k, n, f)
        b = O.rope_rotate(q, m + d, f) @ O.rope_rotate(k, n + d, f)
        assert a == pytest.approx(b, abs=1e-9)


def test_round_to_bf16_matches_torch_and_ties_to_even():
    rng = np.random.default_rng(3)
    x32 = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_to_bf16(x32.astype(np.float64)), want)
    assert O.round_to_bf16(np.array([1 + 2 ** -8]))[0] == 1.0               # tie -> even
    assert O.round_to_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6   # tie -> even (up)
    assert O.round_to_bf16(np.array([-(1 + 2 ** -8 + 2 ** -30)]))[0] == -(1 + 2 ** -7)


def test_bf16_bit_helpers_round_trip():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F], dtype=np.uint16)
    vals = O.bf16_bits_to_float(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[2] == 3.140625
    np.testing.assert_array_equal(O.float_to_bf16_bits(vals), bits)
