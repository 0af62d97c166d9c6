"""Distribution of the GPU's samples on the tiny workload: 10^6 draws per
row against softmax(z / T) (closed form), and the winning score against
the Gumbel max law.  The noise is keyed on the batch position, so copies of
one hidden state in many batch rows are independent draws."""
import numpy as np
import pytest
import torch
from scipy import special, stats

from conftest import gpu_available

import oracle
import lm_head_exact_amd as fsl
from lm_head_exact_amd import workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]
DEV = "cuda"


def _chisq(counts, probs):
    n = counts.sum()
    e = probs * n
    order = np.argsort(e)
    c, e = counts[order].astype(np.float64), e[order]
    small = np.cumsum(e) < 5.0
    if small.any():
        k = int(small.sum()) + 1
        c = np.concatenate([[c[:k].sum()], c[k:]])
        e = np.concatenate([[e[:k].sum()], e[k:]])
    return stats.chisquare(c, e * (c.sum() / e.sum())).pvalue


def test_tiny_softmax_law_1e6_draws_per_row():
    h, W, T = wl.make_inputs(wl.TINY, 4)
    z = oracle.logits(wl.bf16_bits(h), wl.bf16_bits(W)).astype(np.float64)
    reps = 2048                                   # copies of each row per call
    hb = h.repeat(reps, 1).to(DEV)                # batch row i holds h[i % 4]
    Tb = T.repeat(reps).to(DEV)
    Wd = W.to(DEV)
    calls = (10**6 + reps - 1) // reps
    counts = np.zeros((4, W.shape[0]), np.int64)
    vals = []
    for s in range(calls):
        ids, val = fsl.sample(hb, Wd, Tb, s, 0)
        ids = ids.view(reps, 4).cpu().numpy()
        for r in range(4):
            counts[r] += np.bincount(ids[:, r], minlength=W.shape[0])
        if s < 50:
            vals.append(val.view(reps, 4).cpu().numpy())
    vals = np.concatenate(vals)
    for r in range(4):
        probs = special.softmax(z[r] / float(T[r]))
        p = _chisq(counts[r], probs)
        print(f"row {r}: chi-square p = {p:.4f} over {counts[r].sum()} draws")
        assert p > 1e-3
        lse = special.logsumexp(z[r] / float(T[r]))
        ks = stats.kstest(vals[:, r].astype(np.float64) - lse, stats.gumbel_r.cdf).pvalue
        print(f"row {r}: max-score KS p = {ks:.4f}")
        assert ks > 1e-3
