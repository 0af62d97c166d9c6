"""Pins of the oracle's sampler against what the method and the mathematics
fix (CPU only).

FlashSampling (wiki summary, "Key claims" and "Method"; arXiv abstract)
samples a token id from the categorical softmax(z / T) as the argmax of the
scaled logits plus Gumbel noise, and is exact because that argmax decomposes
over any partition of the vocabulary.  Each check below is one of:
  * a closed form: P(id = i) = softmax(z/T)_i (Pearson chi-square, and the
    two-id logistic law), max score - logsumexp(z/T) ~ Gumbel(0,1);
  * an invariant: tiles/shards + merge reproduce the full run bit for bit,
    (2W, 2T) gives the same scores;
  * a special case that reduces to a library routine: greedy rows are
    numpy.argmax of an fp64 matmul; h = 0 samples uniformly.
"""
import math

import numpy as np
import pytest
import torch
from scipy import special, stats

from lm_head_exact_amd import workloads as wl

P_MIN = 1e-3  # acceptance threshold of every goodness-of-fit test


def _f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _rand_bf16(shape, std, seed):
    g = torch.Generator().manual_seed(seed)
    return wl.bf16_bits((std * torch.randn(*shape, generator=g)).to(torch.bfloat16))


def _chisq(counts, probs):
    """Pearson chi-square with bins of expected count < 5 pooled."""
    n = counts.sum()
    exp = probs * n
    order = np.argsort(exp)
    c, e = counts[order].astype(np.float64), exp[order]
    small = np.cumsum(e) < 5.0
    if small.any():
        k = int(small.sum()) + 1
        c = np.concatenate([[c[:k].sum()], c[k:]])
        e = np.concatenate([[e[:k].sum()], e[k:]])
    return stats.chisquare(c, e * (c.sum() / e.sum())).pvalue


@pytest.fixture(scope="module")
def tiny(orc):
    h, W, T = wl.make_inputs(wl.TINY, 4)
    hb, Wb, Tn = wl.bf16_bits(h), wl.bf16_bits(W), T.numpy()
    return hb, Wb, Tn, orc.logits(hb, Wb)


def test_greedy_rows_are_library_argmax(orc):
    B, D, V = 6, 64, 3000
    hb, Wb = _rand_bf16((B, D), 1.0, 1), _rand_bf16((V, D), 0.1, 2)
    T = np.array([0.0, -0.0, -1.0, np.nan, 0.0, 0.0], np.float32)
    ids, val, _ = orc.sample(hb, Wb, T, seed=7, step=3)
    ref = _f64(hb) @ _f64(Wb).T
    assert np.array_equal(ids, np.argmax(ref, axis=1))
    assert np.array_equal(val, ref.astype(np.float32).max(axis=1))


def test_small_temperature_limit_is_greedy(orc):
    """With g bounded ([-3.131, 22.874] over all 2^32 words), any
    0 < T < gap / 26.01 yields the greedy id; T = gap / 40 is well inside."""
    B, D, V = 8, 64, 2000
    hb, Wb = _rand_bf16((B, D), 1.0, 3), _rand_bf16((V, D), 0.1, 4)
    z = _f64(hb) @ _f64(Wb).T
    top2 = np.sort(z, axis=1)[:, -2:]
    gap = (top2[:, 1] - top2[:, 0]).astype(np.float32)
    for seed in range(5):
        ids, _, _ = orc.sample(hb, Wb, gap / 40, seed=seed, step=seed)
        assert np.array_equal(ids, np.argmax(z, axis=1))


def test_tie_goes_to_smaller_id(orc):
    """Three identical W rows aligned with h[0] tie for the maximum logit of
    row 0; the greedy sample must return the smallest of the three ids."""
    D, V = 32, 50
    hb = _rand_bf16((2, D), 1.0, 5)
    Wb = _rand_bf16((V, D), 0.1, 6)
    Wb[[44, 9, 31]] = hb[0]
    ids, _, gap = orc.sample(hb, Wb, np.zeros(2, np.float32), seed=0, step=0)
    z = _f64(hb) @ _f64(Wb).T
    assert np.argmax(z[0]) == 9 and z[0, 9] == z[0, 31] == z[0, 44]
    assert ids[0] == 9 and gap[0] == 0.0


@pytest.mark.parametrize("widths", [[1], [7], [128], [256], [1000], "random"])
def test_partition_invariance(orc, tiny, widths):
    """Per-tile maximisers merged across tiles equal the global maximiser,
    bit for bit, for any partition of the vocabulary (tile widths 1, 7, 128,
    256, V and random cuts)."""
    hb, Wb, T, _ = tiny
    V = Wb.shape[0]
    if widths == "random":
        rng = np.random.default_rng(11)
        cuts = np.sort(rng.choice(np.arange(1, V), size=23, replace=False))
    else:
        cuts = np.arange(widths[0], V, widths[0])
    bounds = [0, *cuts.tolist(), V]
    full_ids, full_val, _ = orc.sample(hb, Wb, T, seed=5, step=2)
    pv, pi = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        ids, val, _ = orc.sample(hb, Wb[a:b], T, seed=5, step=2, vocab_offset=a)
        pv.append(val)
        pi.append(ids)
    perm = np.random.default_rng(len(bounds)).permutation(len(pv))  # slot order is free
    m_ids, m_val = orc.merge(np.stack(pv)[perm], np.stack(pi)[perm])
    assert np.array_equal(m_ids, full_ids)
    assert np.array_equal(m_val.view(np.uint32), full_val.view(np.uint32))


def test_shard_invariance(orc):
    """Eight vocabulary shards with global offsets plus a merge equal the
    unsharded run (tensor-parallel flow of the wiki summary, "Method")."""
    B, D, V, P = 5, 48, 8 * 203 + 0, 8
    hb, Wb = _rand_bf16((B, D), 1.0, 8), _rand_bf16((V, D), 0.15, 9)
    T = np.array([1.0, 0.7, 0.0, 1.3, 2.0], np.float32)
    full = orc.sample(hb, Wb, T, seed=99, step=12345678901)
    vs = V // P
    pv, pi = [], []
    for p in range(P):
        ids, val, _ = orc.sample(hb, Wb[p * vs:(p + 1) * vs], T, seed=99,
                                 step=12345678901, vocab_offset=p * vs)
        assert np.all((ids >= p * vs) & (ids < (p + 1) * vs))
        pv.append(val)
        pi.append(ids)
    m_ids, m_val = orc.merge(np.stack(pv), np.stack(pi))
    assert np.array_equal(m_ids, full[0]) and np.array_equal(m_val, full[1])


def test_doubling_w_and_t_is_exact(orc):
    """z -> 2z and T -> 2T leave every score unchanged: doubling is exact in
    bf16 and fp32, and (2z) * fp32(1/(2T)) == z * fp32(1/T) bit for bit."""
    B, D, V = 4, 64, 700
    hb, Wb = _rand_bf16((B, D), 1.0, 10), _rand_bf16((V, D), 0.1, 11)
    W2 = wl.bf16_bits((torch.from_numpy(Wb.view(np.int16)).view(torch.bfloat16) * 2))
    T = np.array([1.0, 0.5, 1.5, 0.3], np.float32)
    a = orc.sample(hb, Wb, T, seed=3, step=4)
    b = orc.sample(hb, W2, 2 * T, seed=3, step=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_zero_hidden_state_samples_uniformly(orc):
    """h = 0 makes every logit 0, so the id is uniform over V whatever D is."""
    V = 40
    for D in (8, 96):
        hb = np.zeros((1, D), np.uint16)
        Wb = _rand_bf16((V, D), 1.0, 12)
        z = orc.logits(hb, Wb)
        assert np.all(z == 0)
        ids, _, _ = orc.sample_logits(z, np.ones(1, np.float32), 0, 0, n_seeds=200_000)
        counts = np.bincount(ids.ravel(), minlength=V)
        assert _chisq(counts, np.full(V, 1.0 / V)) > P_MIN
    # independent of D: identical noise field, identical ids
    i8 = orc.sample(np.zeros((3, 8), np.uint16), _rand_bf16((V, 8), 1, 1),
                    np.ones(3, np.float32), 4, 4)[0]
    i96 = orc.sample(np.zeros((3, 96), np.uint16), _rand_bf16((V, 96), 1, 2),
                     np.ones(3, np.float32), 4, 4)[0]
    assert np.array_equal(i8, i96)


@pytest.mark.parametrize("dz,T", [(0.0, 1.0), (0.7, 1.0), (-1.3, 0.5), (2.0, 3.0)])
def test_two_ids_logistic_law(orc, dz, T):
    """With two ids, P(id = 1) = sigmoid((z1 - z0) / T): binomial test."""
    z = np.array([[0.25, 0.25 + dz]], np.float32)
    n = 400_000
    ids, _, _ = orc.sample_logits(z, np.array([T], np.float32), 1000, 0, n_seeds=n)
    p1 = special.expit((np.float64(z[0, 1]) - np.float64(z[0, 0])) / T)
    k = int((ids == 1).sum())
    assert stats.binomtest(k, n, p1).pvalue > P_MIN


@pytest.mark.parametrize("T", [0.3, 1.0, 2.0])
def test_softmax_law_small_vocab(orc, T):
    z = (np.linspace(-2.0, 2.0, 16) + 0.1 * np.sin(np.arange(16))).astype(np.float32)[None]
    n = 1_000_000
    ids, _, _ = orc.sample_logits(z, np.array([T], np.float32), 0, 0, n_seeds=n)
    counts = np.bincount(ids.ravel(), minlength=16)
    probs = special.softmax(z[0].astype(np.float64) / T)
    assert _chisq(counts, probs) > P_MIN


def test_softmax_law_tiny_workload_1e6_seeds(orc, tiny):
    """10^6 seeds (0 .. 999999, step 0) on a row of the tiny workload:
    sampled ids follow softmax(z / T) (Pearson chi-square, p > 1e-3)."""
    _, _, T, z = tiny
    row = 2
    ids, _, _ = orc.sample_logits(z[row:row + 1], T[row:row + 1], 0, 0, n_seeds=1_000_000,
                                  rows=np.array([row], np.int32))
    counts = np.bincount(ids.ravel(), minlength=z.shape[1])
    probs = special.softmax(z[row].astype(np.float64) / T[row])
    assert _chisq(counts, probs) > P_MIN


def test_max_value_law(orc, tiny):
    """The winning score minus logsumexp(z/T) is standard Gumbel (KS test),
    with mean gamma and variance pi^2/6, and is independent of the id."""
    _, _, T, z = tiny
    row = 1
    n = 200_000
    ids, val, _ = orc.sample_logits(z[row:row + 1], T[row:row + 1], 77, 5, n_seeds=n,
                                    rows=np.array([row], np.int32))
    lse = special.logsumexp(z[row].astype(np.float64) / T[row])
    x = val.ravel().astype(np.float64) - lse
    assert stats.kstest(x, stats.gumbel_r.cdf).pvalue > P_MIN
    assert abs(x.mean() - 0.5772156649) < 5 * math.pi / math.sqrt(6 * n)
    # independence: the score law is the same whether or not the mode won
    mode = np.argmax(z[row])
    won = ids.ravel() == mode
    assert stats.ks_2samp(x[won], x[~won]).pvalue > P_MIN


def test_sample_from_logits_matches_sample(orc, tiny):
    hb, Wb, T, z = tiny
    a = orc.sample(hb, Wb, T, seed=31, step=9)
    b = orc.sample_logits(z, T, 31, 9, n_seeds=1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y[0])


def test_rows_subset_and_row_keying(orc, tiny):
    """A listed subset of rows reproduces those rows of the full call; the
    batch position keys the noise, so identical rows sample independently."""
    hb, Wb, T, _ = tiny
    full = orc.sample(hb, Wb, T, seed=1, step=1)
    sub = orc.sample(hb, Wb, T, seed=1, step=1, rows=[3, 0])
    assert np.array_equal(sub[0], full[0][[3, 0]])
    rep = np.repeat(hb[:1], 64, axis=0)
    ids, _, _ = orc.sample(rep, Wb, np.ones(64, np.float32), seed=1, step=1)
    assert len(set(ids.tolist())) > 20


def test_merge_matches_lexicographic_order(orc):
    """Merge = per row, the largest value, then the smallest id (checked
    against numpy.lexsort), with planted ties and every slot order."""
    rng = np.random.default_rng(21)
    P, B = 9, 400
    val = rng.normal(size=(P, B)).astype(np.float32)
    ids = rng.integers(0, 1 << 30, size=(P, B)).astype(np.int32)
    tie = rng.random(B) < 0.3
    val[4, tie] = 10.0
    val[7, tie] = 10.0
    val[2, tie[:]] = np.where(rng.random(tie.sum()) < 0.5, 10.0, val[2, tie])
    ids[:, 0] = [5, 3, 9, 3, 1, 8, 7, 6, 2]
    val[:, 0] = 1.0
    for trial in range(4):
        perm = rng.permutation(P)
        m_ids, m_val = orc.merge(val[perm], ids[perm])
        for b in range(B):
            order = np.lexsort((ids[:, b], -val[:, b]))
            assert m_ids[b] == ids[order[0], b] and m_val[b] == val[order[0], b]
    assert orc.merge(val, ids)[0][0] == 1
