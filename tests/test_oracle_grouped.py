"""Pins for the oracle's grouped (hierarchical) sampler.

The pages state that grouped variants are exact by hierarchical
factorisation of the categorical distribution (arXiv abstract page; wiki
summary, "Key claims"): P(i) = P(G) P(i | G) with P(G) proportional to
exp(LSE_G).  Each pin checks the oracle against something other than
itself: a library routine (scipy's logsumexp on an independent numpy
matmul), the associativity of log-sum-exp, the closed-form group and token
distributions (chi-square), the standard Gumbel law (KS) and the greedy
limit (plain argmax).
"""
import numpy as np
import pytest
from scipy import stats
from scipy.special import logsumexp, softmax

import oracle
from lm_head_exact_amd import workloads as wl

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _np_logits(hb, Wb):
    """fp32 logits from an fp64 numpy matmul of the bf16 bit patterns."""
    h = (hb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    W = (Wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return (h @ W.T).astype(np.float32)


def _tiny(B=6, temps=(1.0, 0.5, 0.0, 2.0, 0.3, -1.0)):
    h, W, _ = wl.make_inputs(wl.TINY, B)
    hb, Wb = wl.bf16_bits(h), wl.bf16_bits(W)
    T = np.resize(np.asarray(temps, np.float32), B)
    return hb, Wb, T


def test_lse_matches_library_logsumexp():
    hb, Wb, T = _tiny()
    z = _np_logits(hb, Wb)
    ids, val, gap, lse = oracle.sample_lse(hb, Wb, T, seed=3, step=4)
    for b in range(len(T)):
        if T[b] > 0:
            inv_t = np.float32(1.0) / T[b]
            ref = logsumexp(z[b].astype(np.float64) * np.float64(inv_t))
            assert abs(lse[b] - ref) <= 2e-6 * max(1.0, abs(ref)), b
        else:
            assert lse[b] == z[b].max(), b  # greedy: the largest logit


def test_sample_lse_winner_is_the_plain_sampler():
    hb, Wb, T = _tiny()
    a = oracle.sample(hb, Wb, T, seed=11, step=2, vocab_offset=7)
    b = oracle.sample_lse(hb, Wb, T, seed=11, step=2, vocab_offset=7)
    for x, y in zip(a, b[:3]):
        assert np.array_equal(x, y)


def test_group_lse_merges_to_full_lse():
    """log-sum-exp is associative: the merge of the slices' LSEs is the LSE
    of the whole vocabulary; the merged sample is one of the slices'."""
    hb, Wb, T = _tiny()
    V = Wb.shape[0]
    cuts = [0, 1, 100, 333, 334, 800, V]
    full = oracle.sample_lse(hb, Wb, T, seed=5, step=6)
    parts = [oracle.sample_lse(hb, Wb[a:c], T, seed=5, step=6, vocab_offset=a)
             for a, c in zip(cuts[:-1], cuts[1:])]
    val = np.stack([p[1] for p in parts])
    ids = np.stack([p[0] for p in parts])
    lse = np.stack([p[3] for p in parts])
    out_id, out_val, out_lse, _ = oracle.merge_lse(val, ids, lse, T, seed=5, step=6)
    np.testing.assert_allclose(out_lse, full[3], rtol=2e-6, atol=2e-6)
    for b in range(len(T)):
        assert out_id[b] in ids[:, b]


def test_group_choice_follows_softmax_of_lse():
    """With fixed group partials, the chosen group is distributed as
    softmax(LSE_G); rows are independent draws (the noise is keyed on them)."""
    lse_groups = np.array([0.0, 1.0, -0.5, 2.0, 0.3], np.float32)
    P, N = lse_groups.size, 200_000
    lse = np.repeat(lse_groups[:, None], N, axis=1)
    ids = np.repeat(np.arange(P, dtype=np.int32)[:, None], N, axis=1)  # id = group
    val = np.zeros_like(lse)
    T = np.ones(N, np.float32)
    chosen, _, total, _ = oracle.merge_lse(val, ids, lse, T, seed=123, step=9)
    counts = np.bincount(chosen, minlength=P)
    expected = softmax(lse_groups.astype(np.float64)) * N
    chi2, p = stats.chisquare(counts, expected)
    assert p > 1e-3, (counts, expected, p)
    np.testing.assert_allclose(total, logsumexp(lse_groups.astype(np.float64)), rtol=1e-6)


@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_grouped_sampler_follows_softmax(T):
    """The whole grouped construction -- each group's Gumbel-max sample, its
    LSE, then the group draw -- samples softmax(z / T) exactly."""
    rng = np.random.default_rng(7)
    z = (1.2 * rng.standard_normal((1, 16))).astype(np.float32)
    cuts = [0, 5, 6, 12, 16]
    N = 100_000
    Tr = np.array([T], np.float32)
    vals, ids, lses = [], [], []
    for a, c in zip(cuts[:-1], cuts[1:]):
        i, v, _ = oracle.sample_logits(z[:, a:c], Tr, seed0=1000, step=1, n_seeds=N,
                                       vocab_offset=a)
        ids.append(i[:, 0])
        vals.append(v[:, 0])
        lses.append(np.full(N, oracle.lse_logits(z[:, a:c], Tr)[0], np.float32))
    # one merge row per seed: the group noise is keyed on the row
    out_id, _, total, _ = oracle.merge_lse(np.stack(vals), np.stack(ids), np.stack(lses),
                                           np.full(N, T, np.float32), seed=77, step=1)
    counts = np.bincount(out_id, minlength=16)
    inv_t = np.float64(np.float32(1.0) / np.float32(T))
    expected = softmax(z[0].astype(np.float64) * inv_t) * N
    chi2, p = stats.chisquare(counts, expected)
    assert p > 1e-3, (counts, expected, p)
    np.testing.assert_allclose(total[0], logsumexp(z[0].astype(np.float64) / T), rtol=1e-5)


def test_greedy_rows_pick_the_global_argmax():
    hb, Wb, _ = _tiny()
    B, V = hb.shape[0], Wb.shape[0]
    T = np.zeros(B, np.float32)
    z = _np_logits(hb, Wb)
    cuts = [0, 250, 500, 750, V]
    parts = [oracle.sample_lse(hb, Wb[a:c], T, seed=1, step=1, vocab_offset=a)
             for a, c in zip(cuts[:-1], cuts[1:])]
    out_id, out_val, out_lse, _ = oracle.merge_lse(
        np.stack([p[1] for p in parts]), np.stack([p[0] for p in parts]),
        np.stack([p[3] for p in parts]), T, seed=1, step=1)
    assert np.array_equal(out_id, np.argmax(z, axis=1))
    assert np.array_equal(out_lse, z.max(axis=1))


def test_group_noise_is_standard_gumbel():
    g = np.array([oracle.group_gumbel(99, 5, row, p) for row in range(200) for p in range(100)])
    assert stats.kstest(g, stats.gumbel_r.cdf).pvalue > 1e-3
    # independent of the token noise drawn at the same (seed, step, row)
    tok = np.array([oracle.gumbel(oracle.noise_bits(99, 5, row, 4 * p))
                    for row in range(200) for p in range(100)])
    assert abs(np.corrcoef(g, tok)[0, 1]) < 0.03
