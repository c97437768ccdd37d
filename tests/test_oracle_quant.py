"""Pins of the oracle's asymmetric RTN group quantizer (KIVI keys/values,
Kitty boosted channels) against facts the pages and the arithmetic fix.

* Kitty summary, "Observation 1": a channel spanning [0, 10] quantized to
  2 bits has steps of 10/3; one spanning [0, 1] has steps of 1/3
  (tests/golden/kitty_obs1_steps.json).
* Round-to-nearest: each code is a nearest level (brute force over all
  2^b levels), and |x - x_hat| <= s/2 for every element.
* Special cases: constant groups reconstruct exactly; equally spaced
  levels reconstruct exactly; minimum -> code 0, maximum -> 2^b - 1.
"""
import json
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def f16(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def f32(h):
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float32)


def _check_group(O, x, bits):
    s16, z16, codes = O.quant_asym(x, bits)
    s = float(f32(s16)); z = float(f32(z16))
    xv = f32(x).astype(np.float64)
    lmax = (1 << bits) - 1
    assert codes.max() <= lmax
    xhat = np.array([O.dequant_asym(c, s16, z16) for c in codes], np.float64)
    # x_hat is code*s + z rounded once to binary32
    assert np.array_equal(xhat.astype(np.float32),
                          (codes.astype(np.float32) * np.float32(s) + np.float32(z)))
    # |x - x_hat| <= s/2, exact fp64 with one binary32 half-ulp of slack
    slack = np.abs(xhat) * 2.0 ** -24 + 2.0 ** -149
    assert np.all(np.abs(xv - xhat) <= s / 2 + slack), (s, np.max(np.abs(xv - xhat)))
    # brute force: the chosen level is a nearest level (up to rounding slack)
    levels = np.arange(lmax + 1, dtype=np.float64) * s + z
    dist = np.abs(xv[:, None] - levels[None, :])
    best = dist.min(axis=1)
    chosen = dist[np.arange(xv.size), codes]
    assert np.all(chosen <= best + 2.0 ** -20 * max(s, 2.0 ** -24) + slack)
    return s16, z16, codes, s, z


@pytest.mark.parametrize("bits", [2, 4])
def test_random_groups_nearest_level_and_half_step_bound(O, bits):
    rng = np.random.default_rng(7)
    for trial in range(400):
        scale = 2.0 ** rng.uniform(-20, 12)
        x = f16(rng.standard_normal(32) * scale + rng.standard_normal() * scale)
        s16, z16, codes, s, z = _check_group(O, x, bits)
        xv = f32(x)
        assert z16 == f16(xv.min() + np.float32(0.0))     # z = group minimum
        assert codes[np.argmin(xv)] == 0
        if s >= 2.0 ** -14:       # fp16-normal step: the maximum takes the top level
            assert codes[np.argmax(xv)] == (1 << bits) - 1


def test_kitty_observation1_steps(O):
    with open(os.path.join(GOLD, "kitty_obs1_steps.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        lo, hi = case["span"]
        x = f16(np.linspace(lo, hi, 32))
        s16, z16, codes, s, z = _check_group(O, x, case["bits"])
        assert z == lo
        assert abs(s - case["step"]) <= case["step"] * 2.0 ** -11
        assert abs(s - case["step_printed"]) < case["printed_tolerance"]


def test_constant_group_reconstructs_exactly(O):
    for v in [0.0, -0.0, 1.5, -3.25, 65504.0, 2.0 ** -24]:
        x = f16(np.full(32, v))
        s16, z16, codes = O.quant_asym(x, 2)
        assert s16 == 0 and np.all(codes == 0)
        assert O.dequant_asym(0, s16, z16) == float(f32(x[0]))


@pytest.mark.parametrize("bits", [2, 4])
def test_equally_spaced_levels_are_exact(O, bits):
    lmax = (1 << bits) - 1
    for z, s in [(-1.0, 0.5), (0.0, 1.0), (2.0, 0.125), (-8.0, 3.0)]:
        lv = z + s * np.arange(lmax + 1)
        x = f16(np.resize(lv, 32))
        s16, z16, codes, ss, zz = _check_group(O, x, bits)
        assert ss == s and zz == z
        assert np.array_equal(codes, np.resize(np.arange(lmax + 1), 32))


def test_exact_ties_round_to_even(O):
    # z = 0, s = 1 (range 3): x = k + 1/2 is an exact tie between k and k+1
    x = f16([0.0, 3.0, 0.5, 1.5, 2.5] + [1.0] * 27)
    s16, z16, codes = O.quant_asym(x, 2)
    assert f32(s16) == 1.0
    assert list(codes[2:5]) == [0, 2, 2]


def test_subnormal_scale_guard_keeps_half_step_bound(O):
    # range 4 * 2^-24: plain rounding would give s = 2^-24 and the top element
    # would land a whole step away; the guard raises s to 2 * 2^-24
    x = f16(np.resize([0.0, 4 * 2.0 ** -24], 32))
    s16, z16, codes, s, z = _check_group(O, x, 2)
    assert s == 2 * 2.0 ** -24
    assert set(codes.tolist()) == {0, 2}


def test_codes_fill_all_levels_on_uniform_data(O):
    x = f16(np.linspace(-5, 7, 32))
    s16, z16, codes = O.quant_asym(x, 2)
    assert set(codes.tolist()) == {0, 1, 2, 3}
