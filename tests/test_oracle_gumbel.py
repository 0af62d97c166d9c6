"""Pins of the oracle's uniform and Gumbel maps (CPU only).

The sampler perturbs each scaled logit with a standard Gumbel variable
(wiki summary, "Key claims" and "Method"; the Gumbel-Max trick).  The oracle
maps a 32-bit noise word x to the midpoint of its cell, u = (x + 1/2) 2^-32,
and inverts the Gumbel CDF, g = -log(-log u).  The 2^32 words are too many to
check one by one, so the pins cover:

  * the tail exhaustively: the top 2^24 words (u > 1 - 2^-8), where the
    winners of a large vocabulary draw their noise, and the bottom 2^20;
  * the bulk on a stratified grid: one word in every cell of 256, offset
    into the cell, 2^24 words spread evenly over the whole range;

against the closed-form CDF F(x) = exp(-exp(-x)), which a sign error, a
swapped log, a dropped bit or a shifted cell would violate; plus the
moments of the standard Gumbel law, and the tie rate of the whole noise
field at a production vocabulary size (the exactness the pages claim).
"""
import math

import numpy as np
import pytest

TOP = (np.uint64(1) << np.uint64(32)) - np.uint64(1 << 24) + np.arange(1 << 24, dtype=np.uint64)
TAIL_HI = TOP.astype(np.uint32)                                   # x >= 2^32 - 2^24
TAIL_LO = np.arange(1 << 20, dtype=np.uint32)                      # x < 2^20
STRAT = (np.arange(1 << 24, dtype=np.uint64) * np.uint64(256) + np.uint64(97)).astype(np.uint32)


@pytest.fixture(scope="module")
def maps(orc):
    out = {}
    for name, words in (("hi", TAIL_HI), ("lo", TAIL_LO), ("strat", STRAT)):
        out[name] = (words, orc.uniform_array(words), orc.gumbel_array(words))
    return out


def test_uniform_is_cell_midpoint(maps):
    """u(x) * 2^33 = 2x + 1 exactly, and 0 < u < 1."""
    for words, u, _ in maps.values():
        assert u.dtype == np.float64
        assert np.array_equal(u * 2.0**33, 2.0 * words.astype(np.float64) + 1.0)
        assert u.min() > 0.0 and u.max() < 1.0


def test_every_bit_of_the_word_counts(orc):
    """Flipping any single bit of the word moves u by exactly that bit's
    weight 2^(i-32): no bit is dropped (the low 9 bits included)."""
    rng = np.random.default_rng(3)
    words = rng.integers(0, 1 << 32, size=4096, dtype=np.uint64).astype(np.uint32)
    u = orc.uniform_array(words)
    for i in range(32):
        flipped = words ^ np.uint32(1 << i)
        du = orc.uniform_array(flipped) - u
        sign = np.where((words >> np.uint32(i)) & 1, -1.0, 1.0)
        assert np.array_equal(du, sign * 2.0 ** (i - 32))


def test_gumbel_finite_monotone_and_extremes(orc, maps):
    for words, _, g in maps.values():
        assert np.all(np.isfinite(g))
        order = np.argsort(words, kind="stable")
        assert np.all(np.diff(g[order].astype(np.float64)) >= 0)
    # the top 2^18 words give distinct fp32 values (spacing >> one ulp there)
    words, _, g = maps["hi"]
    assert np.all(np.diff(g[-(1 << 18):]) > 0)
    # extremes: -log(-log 2^-33) = -log(33 ln 2) and -log(-log(1 - 2^-33))
    assert orc.gumbel(0) == np.float32(-math.log(33 * math.log(2)))
    assert orc.gumbel(0xFFFFFFFF) == np.float32(-math.log(-math.log1p(-2.0**-33)))
    assert -3.1301 < orc.gumbel(0) < -3.1299 and 22.8738 < orc.gumbel(0xFFFFFFFF) < 22.8739


def test_gumbel_matches_cdf_pointwise(maps):
    """F(g(x)) must give back u(x): the fp32 rounding of g moves F by at most
    the density (<= 1/e) times half an ulp of g.  In the top tail the check
    is made on 1 - F against 1 - u, which keeps its relative accuracy."""
    for name, (words, u, g) in maps.items():
        g64 = g.astype(np.float64)
        half_ulp = np.spacing(np.abs(g)).astype(np.float64) / 2
        dens = np.exp(-g64 - np.exp(-g64))
        if name == "hi":
            got = -np.expm1(-np.exp(-g64))                                # 1 - F(g)
            want = ((2.0**32 - 1.0) - words.astype(np.float64) + 0.5) * 2.0**-32  # 1 - u
        else:
            got, want = np.exp(-np.exp(-g64)), u
        # plus a relative slack for the fp64 evaluation of F (far below a cell)
        bound = half_ulp * dens * 1.0001 + 1e-13 * want
        assert np.all(np.abs(got - want) <= bound)


def test_gumbel_empirical_cdf_on_stratified_grid(maps):
    """Over one word per 256-cell, evenly spread, the empirical CDF of g is
    exp(-exp(-x)) to within one stratum (2^-24)."""
    words, _, g = maps["strat"]
    gs = np.sort(g)
    xs = np.linspace(-3.0, 16.0, 381)
    emp = np.searchsorted(gs, xs, side="right") / gs.size
    F = np.exp(-np.exp(-xs))
    assert np.max(np.abs(emp - F)) < 2.0 / gs.size


def test_gumbel_moments(maps):
    """Mean is the Euler-Mascheroni constant, variance pi^2 / 6."""
    _, _, g = maps["strat"]
    g64 = g.astype(np.float64)
    assert abs(g64.mean() - 0.5772156649) < 1e-4
    assert abs(g64.var() - math.pi**2 / 6) < 2e-3


def test_equal_logits_tie_rate_at_full_vocabulary(orc):
    """With all logits equal (h = 0, duplicate or padding rows) the sample
    must be uniform over the vocabulary; a tie for the largest score goes to
    the smaller id and biases it.  At V = 128256 the field ties only when two
    words are equal, about V * 2^-33 = 1.5e-5 of draws; the tie rate over
    3 * 10^4 seeds must stay below 1e-4 (a noise map that drops bits of the
    word, e.g. a 23-bit grid, ties at V * 2^-24, about 0.76%)."""
    V, n = 128256, 30000
    z = np.zeros((1, V), np.float32)
    ids, val, gap = orc.sample_logits(z, np.ones(1, np.float32), seed0=0, step=0, n_seeds=n)
    ties = int((gap == 0).sum())
    assert ties / n < 1e-4, f"{ties} ties in {n} draws"
    # and the ids are uniform: the 16 equal-width id bins, chi-square at p > 0.001
    from scipy.stats import chisquare
    counts = np.bincount(ids[:, 0] * 16 // V, minlength=16)
    assert chisquare(counts).pvalue > 1e-3


def test_score_equals_its_parts(orc):
    """oracle_score (used to accept near-tie ids) is the fp32 add of the fp32
    scaled logit and the Gumbel value of the element's own noise word, and
    the plain logit for a greedy row."""
    rng = np.random.default_rng(17)
    for _ in range(200):
        z = np.float32(rng.normal() * 3)
        T = np.float32(rng.uniform(0.2, 2.0))
        seed, step = int(rng.integers(0, 2**63)), int(rng.integers(0, 2**63))
        row, gv = int(rng.integers(0, 4096)), int(rng.integers(0, 2**31 - 1))
        g = np.float32(orc.gumbel(orc.noise_bits(seed, step, row, gv)))
        scaled = np.float32(z * np.float32(np.float32(1.0) / T))
        assert orc.score(z, T, seed, step, row, gv) == np.float32(scaled + g)
        for greedy_T in (0.0, -0.0, -1.5, float("nan")):
            assert orc.score(z, greedy_T, seed, step, row, gv) == z


def test_score_equals_one_id_sampler(orc):
    """On a one-id vocabulary the sampler's winning score is that id's score:
    oracle_score and the sampler agree on the row and the global id that key
    the noise, and on the scaling, for scaled and greedy rows."""
    rng = np.random.default_rng(23)
    for _ in range(50):
        z = np.array([[rng.normal() * 2]], np.float32)
        row, gv = int(rng.integers(0, 512)), int(rng.integers(0, 2**31 - 1))
        seed, step = int(rng.integers(0, 2**40)), int(rng.integers(0, 2**40))
        for T in (np.float32(rng.uniform(0.3, 1.5)), np.float32(0.0)):
            ids, val, _ = orc.sample_logits(z, np.array([T], np.float32), seed0=seed,
                                            step=step, vocab_offset=gv,
                                            rows=np.array([row], np.int32))
            assert ids[0, 0] == gv
            assert val[0, 0] == np.float32(orc.score(float(z[0, 0]), float(T), seed, step,
                                                     row, gv))
