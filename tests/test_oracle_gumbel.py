"""Pins for the oracle's word -> uniform -> Gumbel map, against closed forms.

Standard Gumbel: CDF F(g) = exp(-exp(-g)), mean = Euler-Mascheroni gamma,
variance = pi^2 / 6. The uniform is u = (x + 1/2) 2^-32, so the map must
invert F exactly (to fp64 rounding) at every lattice point, and the lattice
average of g is a midpoint-rule quadrature of the integral of F^-1 over (0, 1)
(= gamma).
"""
from fractions import Fraction

import numpy as np

from oracle.gumbel import gumbel_from_words, uniform_to_gumbel, word_to_uniform

EULER_GAMMA = 0.57721566490153286061


def test_uniform_is_exact_and_open():
    xs = np.array([0, 1, 2**31 - 1, 2**31, 2**32 - 2, 2**32 - 1], dtype=np.uint64)
    u = word_to_uniform(xs)
    for x, ui in zip(xs, u):
        assert Fraction(float(ui)) == (Fraction(int(x)) + Fraction(1, 2)) / 2**32
    assert u.min() > 0 and u.max() < 1
    assert u[0] == 2.0 ** -33 and u[-1] == 1 - 2.0 ** -33


def test_inverse_cdf_everywhere_on_the_lattice_sample():
    rng = np.random.default_rng(0)
    xs = np.concatenate([
        np.arange(0, 4096, dtype=np.uint64),
        np.arange(2**32 - 4096, 2**32, dtype=np.uint64),
        np.arange(2**31 - 2048, 2**31 + 2048, dtype=np.uint64),
        rng.integers(0, 2**32, 200000, dtype=np.uint64),
    ])
    g = gumbel_from_words(xs)
    u = (xs.astype(np.float64) + 0.5) * 2.0 ** -32
    one_minus_u = (2.0 ** 32 - xs.astype(np.float64) - 0.5) * 2.0 ** -32
    # F(g) = exp(-exp(-g)); compare in whichever tail keeps precision
    Fg = np.exp(-np.exp(-g))
    one_minus_Fg = -np.expm1(-np.exp(-g))
    lo = u <= 0.5
    assert np.all(np.abs(Fg[lo] - u[lo]) <= 1e-14 * u[lo] + 1e-300)
    assert np.all(np.abs(one_minus_Fg[~lo] - one_minus_u[~lo]) <= 2e-13 * one_minus_u[~lo])


def test_extremes_closed_form():
    g = gumbel_from_words(np.array([0, 2**32 - 1], dtype=np.uint64))
    # u = 2^-33: g = -ln(33 ln 2); 1 - u = 2^-33: g = -ln(-ln(1 - 2^-33)) ~= 33 ln 2
    assert abs(g[0] - (-np.log(33 * np.log(2.0)))) < 1e-14
    assert abs(g[1] - 33 * np.log(2.0)) < 1e-8
    assert -3.1300 < g[0] < -3.1299 and 22.8738 < g[1] < 22.8739


def test_lattice_moments_match_gumbel_law():
    # stride-2^12 midpoint lattice (2^20 points): quadrature error ~ h log(1/h), h = 2^-20
    k = 2**12
    xs = (np.arange(2**20, dtype=np.uint64) * np.uint64(k)) + np.uint64(k // 2)
    g = gumbel_from_words(xs)
    assert abs(g.mean() - EULER_GAMMA) < 5e-6
    assert abs(g.var() - np.pi**2 / 6) < 1e-4


def test_uniform_to_gumbel_agrees_with_word_path():
    xs = np.random.default_rng(1).integers(0, 2**32, 10000, dtype=np.uint64)
    a = gumbel_from_words(xs)
    b = uniform_to_gumbel(word_to_uniform(xs))
    assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_monotone_in_the_word():
    xs = np.arange(0, 2**32, 2**20 + 7, dtype=np.uint64)
    g = gumbel_from_words(xs)
    assert np.all(np.diff(g) > 0)
