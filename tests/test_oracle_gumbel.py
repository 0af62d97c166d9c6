"""Exhaustive pins of the oracle's uniform and Gumbel maps (CPU only).

The sampler perturbs each scaled logit with a standard Gumbel variable
(wiki summary, "Key claims" and "Method"; the Gumbel-Max trick).  The oracle
maps the top 23 bits k of a noise word to u = (2k+1) 2^-24 and inverts the
Gumbel CDF, g = -log(-log u).  All 2^23 grid points are checked against the
closed-form CDF F(x) = exp(-exp(-x)), which a sign error, a swapped log or a
wrong bit count would violate.
"""
import math

import numpy as np
import pytest

K = np.arange(1 << 23, dtype=np.uint64)
WORDS = (K << np.uint64(9)).astype(np.uint32)          # low 9 bits zero


@pytest.fixture(scope="module")
def grid(orc):
    u = orc.uniform_array(WORDS)
    g = orc.gumbel_array(WORDS)
    return u, g


def test_uniform_grid_is_exact_open_interval(orc, grid):
    u, _ = grid
    expect = (2.0 * K.astype(np.float64) + 1.0) / 2.0**24
    assert np.array_equal(u.astype(np.float64), expect)
    assert u.min() > 0.0 and u.max() < 1.0
    # the low 9 bits of the word are ignored
    noisy = WORDS | np.uint32(0x1FF)
    assert np.array_equal(orc.uniform_array(noisy[:: 997]), u[:: 997])


def test_gumbel_finite_monotone_and_range(grid):
    _, g = grid
    assert np.all(np.isfinite(g))
    assert np.all(np.diff(g) > 0)                     # strictly increasing in k
    # extremes of the grid: -log(-log 2^-24) and -log(-log(1 - 2^-24))
    assert abs(g[0] - (-math.log(24 * math.log(2)))) < 1e-6
    assert abs(g[-1] - (-math.log(-math.log1p(-2.0**-24)))) < 1e-5
    assert -2.8116 < g[0] < -2.8115 and 16.6355 < g[-1] < 16.6356


def test_gumbel_matches_cdf_pointwise(grid):
    """F(g(k)) must give back u(k): the fp32 rounding of g moves F by at most
    the density (<= 1/e) times half an ulp of g."""
    u, g = grid
    g64 = g.astype(np.float64)
    F = np.exp(-np.exp(-g64))
    half_ulp = np.spacing(np.abs(g)).astype(np.float64) / 2
    bound = half_ulp * np.exp(-g64 - np.exp(-g64)) * 1.0001 + 1e-15
    assert np.all(np.abs(F - u.astype(np.float64)) <= bound)


def test_gumbel_empirical_cdf(grid):
    """The grid's empirical CDF equals exp(-exp(-x)) to within one grid step."""
    _, g = grid
    xs = np.linspace(-2.5, 15.0, 301)
    emp = np.searchsorted(g, xs, side="right") / g.size
    F = np.exp(-np.exp(-xs))
    assert np.max(np.abs(emp - F)) < 2.0 / g.size


def test_gumbel_moments(grid):
    """Mean is the Euler-Mascheroni constant, variance pi^2 / 6."""
    _, g = grid
    g64 = g.astype(np.float64)
    assert abs(g64.mean() - 0.5772156649) < 1e-4
    assert abs(g64.var() - math.pi**2 / 6) < 2e-3
