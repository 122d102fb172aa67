"""Pins of the export oracle (oracle/export.py) against values fixed by the
definition z = e^gamma * rho * a / RMS(a) stored as IEEE binary16 with
round-half-to-even ("DuoLM: Fast and Effective Personalized Recommendation
with Language Models", 核心方法 and 方法步骤详情 step 3).  Every expected value
below is worked out by hand from that definition or from the binary16 format,
not by calling the oracle's own formula again.
"""
import math

import numpy as np
import pytest

from oracle.export import (
    export_table,
    interface_vectors,
    midpoint_distance,
    reference_scale,
    rms,
    to_fp16_bits,
)


def test_hand_worked_row():
    # a = [3, 4, 0, 0]: mean square 25/4, RMS 2.5, a / RMS = [1.2, 1.6, 0, 0].
    # With rho = 0.5 and gamma = 0: z = [0.6, 0.8, 0, 0].  A sum in place of the
    # mean (RMS 5), a dropped square root (6.25) or a missing rho all move it.
    z = interface_vectors(np.array([[3.0, 4.0, 0.0, 0.0]]), rho=0.5, gamma=0.0)
    np.testing.assert_allclose(z, [[0.6, 0.8, 0.0, 0.0]], rtol=0, atol=1e-15)
    # fp16 codes worked out by hand: [0.5, 1) has spacing 2^-11 and exponent
    # field 14 (0x3800); 0.6 = 0.5 + 204.8 steps -> 205 -> 0x38CD,
    # 0.8 = 0.5 + 614.4 steps -> 614 -> 0x3A66.
    bits = export_table(np.array([[3.0, 4.0, 0.0, 0.0]]), rho=0.5, gamma=0.0)
    assert bits.tolist() == [[0x38CD, 0x3A66, 0x0000, 0x0000]]


def test_gain_is_exponential():
    # gamma = ln 2 doubles the vector (e^gamma, not gamma, multiplies it)
    a = np.array([[3.0, 4.0, 0.0, 0.0]])
    z = interface_vectors(a, rho=0.5, gamma=math.log(2.0))
    np.testing.assert_allclose(z, [[1.2, 1.6, 0.0, 0.0]], rtol=1e-15, atol=0)


def test_constant_row_closed_form():
    # a = c * 1 with c > 0 has RMS c, so every entry of z is rho * e^gamma
    for c in (1e-3, 0.25, 7.0, 3e4):
        a = np.full((1, 64), c)
        z = interface_vectors(a, rho=0.03, gamma=0.4)
        np.testing.assert_allclose(z, 0.03 * math.exp(0.4), rtol=1e-15)


def test_eps_enters_under_the_root():
    # a = [1, 1, 1, 1], eps = 3: RMS = sqrt(1 + 3) = 2, so z = rho e^gamma / 2
    z = interface_vectors(np.ones((1, 4)), rho=1.0, gamma=0.0, eps=3.0)
    np.testing.assert_allclose(z, 0.5, rtol=1e-15)
    np.testing.assert_allclose(rms(np.ones((1, 4)), 3.0), [2.0], rtol=1e-15)


def test_output_rms_is_the_calibrated_scale():
    # the purpose of the interface: every z row has RMS rho * e^gamma (eps = 0),
    # whatever the scale of a; with eps > 0 it shrinks by sqrt(ms / (ms + eps))
    rng = np.random.default_rng(5)
    a = rng.standard_normal((50, 96)) * np.exp(rng.standard_normal((50, 1)))
    z = interface_vectors(a, rho=0.028, gamma=-0.3)
    got = np.sqrt(np.mean(z * z, axis=1))
    np.testing.assert_allclose(got, 0.028 * math.exp(-0.3), rtol=1e-13)
    eps = 0.5
    ms = np.mean(a * a, axis=1)
    z = interface_vectors(a, rho=0.028, gamma=-0.3, eps=eps)
    got = np.sqrt(np.mean(z * z, axis=1))
    np.testing.assert_allclose(got, 0.028 * math.exp(-0.3) * np.sqrt(ms / (ms + eps)), rtol=1e-13)


def test_scale_invariance_and_odd_symmetry():
    rng = np.random.default_rng(6)
    a = rng.standard_normal((20, 32))
    z = interface_vectors(a, rho=0.02, gamma=0.1)
    np.testing.assert_allclose(interface_vectors(a * 37.5, rho=0.02, gamma=0.1), z, rtol=1e-14)
    np.testing.assert_allclose(interface_vectors(-a, rho=0.02, gamma=0.1), -z, rtol=0, atol=0)
    # rows are independent: changing one row leaves the others alone
    b = a.copy()
    b[3] *= -9.0
    b[3, 0] += 1.0
    zb = interface_vectors(b, rho=0.02, gamma=0.1)
    np.testing.assert_array_equal(np.delete(zb, 3, axis=0), np.delete(z, 3, axis=0))


def test_zero_row():
    z = interface_vectors(np.zeros((2, 16)), rho=0.02, gamma=0.0, eps=0.0)
    assert np.all(z == 0) and not np.any(np.isnan(z))
    z = interface_vectors(np.zeros((1, 16)), rho=0.02, gamma=0.0, eps=1e-6)
    assert np.all(z == 0)


# binary16 codes worked out from the format: 1.0 = 0x3C00, spacing 2^-10 in
# [1, 2); largest finite 65504 = 0x7BFF; +inf = 0x7C00; smallest subnormal
# 2^-24 = 0x0001.
FP16_CASES = [
    (1.0, 0x3C00),
    (1.0 + 2.0 ** -11, 0x3C00),       # tie between 0x3C00 and 0x3C01: even -> 0x3C00
    (1.0 + 3 * 2.0 ** -11, 0x3C02),   # tie between 0x3C01 and 0x3C02: even -> 0x3C02
    (1.0 + 2.0 ** -11 + 2.0 ** -30, 0x3C01),  # just above the tie
    (65504.0, 0x7BFF),
    (65519.0, 0x7BFF),                # below the overflow threshold 65520
    (65520.0, 0x7C00),                # tie with 2^16: even -> +inf
    (70000.0, 0x7C00),
    (2.0 ** -24, 0x0001),
    (2.0 ** -25, 0x0000),             # tie between 0 and 2^-24: even -> 0
    (3 * 2.0 ** -25, 0x0002),         # tie between 0x0001 and 0x0002: even -> 0x0002
    (2.0 ** -14, 0x0400),             # smallest normal
    (2.0 ** -14 - 2.0 ** -25, 0x0400),  # tie between 0x03FF and 0x0400: even -> 0x0400
    (-0.6, 0xB8CD),
]


@pytest.mark.parametrize("value,code", FP16_CASES)
def test_fp16_rounding_codes(value, code):
    assert int(to_fp16_bits(np.array([value]))[0]) == code
    # the same value produced by the export of a constant row of power-of-two
    # entries (every step exact in float64): a = 4 * 1, rho = value
    if value > 0:
        bits = export_table(np.full((1, 8), 4.0), rho=value, gamma=0.0)
        assert np.all(bits == code)


def test_midpoint_distance():
    assert midpoint_distance(np.array([1.0 + 2.0 ** -11]))[0] == 0.0
    assert midpoint_distance(np.array([65520.0]))[0] == 0.0
    assert midpoint_distance(np.array([3 * 2.0 ** -25]))[0] == 0.0
    # a representable value is half a cell from its cell's midpoint
    np.testing.assert_allclose(midpoint_distance(np.array([1.0])), [2.0 ** -11], rtol=1e-15)


def test_reference_scale():
    # E = [[3, 4], [0, 0]]: mean square 25/4 -> rho = 2.5; a constant table has rho = |c|
    assert reference_scale(np.array([[3.0, 4.0], [0.0, 0.0]])) == 2.5
    assert reference_scale(np.full((7, 5), -0.02)) == pytest.approx(0.02, rel=1e-15)
    # rho of a table whose rows were exported with gain 1 equals rho (the
    # calibration the pages describe): rows of RMS rho have overall RMS rho
    rng = np.random.default_rng(7)
    z = interface_vectors(rng.standard_normal((100, 64)), rho=0.03, gamma=0.0)
    assert reference_scale(z) == pytest.approx(0.03, rel=1e-13)
