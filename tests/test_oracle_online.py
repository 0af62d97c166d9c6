"""Pins for the oracle's online (chunked) sampler with early finalisation.

The pages say the streaming sampler of the online setting may finalise the
sample as soon as later tiles can no longer overtake the running maximum
(wiki summary, "Method"), without a bound.  The oracle's reading: a later
score is at most (|h_b| R (1/T) + g_max)(1 + 2^-8), R the largest later row
norm (Cauchy-Schwarz) and g_max the largest grid Gumbel value.  The pins:
  * the samples equal the plain whole-vocabulary oracle for any chunking,
    whether or not rows stop early (exactness);
  * with all later rows zero the rule must stop after the first chunk;
  * with an exact duplicate of each row's aligned, winning row in a later
    chunk the rule must never stop before that chunk (a missing noise term,
    temperature factor or norm in the bound stops early there, and then the
    duplicate's draw changes about half of the ids);
  * the largest row norm against numpy, g_max against its closed form.
"""
import numpy as np
import pytest
import torch

import oracle
from lm_head_exact_amd import workloads as wl

TEMPS = (1.0, 0.3, 0.0, 1.7, 0.6, -1.0)


def _random(B, D, V, seed):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn(B, D, generator=g).to(torch.bfloat16)
    W = (0.05 * torch.randn(V, D, generator=g)).to(torch.bfloat16)
    T = np.resize(np.asarray(TEMPS, np.float32), B)
    return wl.bf16_bits(h), wl.bf16_bits(W), T


def _aligned(B, D, V, chunk_rows, later, seed, norm=8.0):
    """Row b < B of W is h_b scaled to norm / |h_b|, so z_bb ~= norm; rows
    after the first chunk come from ``later(W_float)``."""
    g = torch.Generator().manual_seed(seed)
    h = torch.randn(B, D, generator=g)
    W = 0.02 * torch.randn(V, D, generator=g)
    W[:B] = h / h.norm(dim=1, keepdim=True) * (norm / h.norm(dim=1, keepdim=True))
    later(W, chunk_rows)
    return wl.bf16_bits(h.to(torch.bfloat16)), wl.bf16_bits(W.to(torch.bfloat16))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_online_equals_plain_sample_for_any_chunking(seed):
    B, D, V = 18, 64, 700
    hb, Wb, T = _random(B, D, V, seed)
    rng = np.random.default_rng(seed)
    o_id, o_val, _ = oracle.sample(hb, Wb, T, 5, 6, vocab_offset=40)
    for n in (1, 2, 7, 64):
        cuts = np.concatenate([[0], np.sort(rng.choice(np.arange(1, V), n - 1, replace=False)), [V]])
        ids, val, used = oracle.sample_online(hb, Wb, T, 5, 6, cuts, vocab_offset=40)
        assert np.array_equal(ids, o_id) and np.array_equal(val.view(np.uint32), o_val.view(np.uint32))
        assert np.all((used >= 1) & (used <= n))


def test_stops_after_first_chunk_when_later_rows_are_zero():
    B, D, V, c0 = 12, 128, 600, 100

    def zero_later(W, c):
        W[c:] = 0.0

    hb, Wb = _aligned(B, D, V, c0, zero_later, seed=7, norm=60.0)
    T = np.resize(np.asarray(TEMPS, np.float32), B)
    cuts = np.array([0, c0, 300, V])
    ids, val, used = oracle.sample_online(hb, Wb, T, 9, 1, cuts)
    assert np.all(used == 1), used
    o_id, o_val, _ = oracle.sample(hb, Wb, T, 9, 1)
    assert np.array_equal(ids, o_id) and np.array_equal(val, o_val)


@pytest.mark.parametrize("where", ["next", "last"])
def test_never_stops_before_a_duplicate_of_the_winner(where):
    B, D, V, c0 = 64, 128, 640, 80
    cuts = np.array([0, c0, 160, 320, V])
    dup0 = c0 if where == "next" else cuts[-2]

    def duplicate(W, c):
        W[dup0:dup0 + B] = W[:B]

    hb, Wb = _aligned(B, D, V, c0, duplicate, seed=11)
    # the duplicate rows are bit-identical after rounding
    assert np.array_equal(Wb[:B], Wb[dup0:dup0 + B])
    T = np.resize(np.asarray((1.0, 0.3, 0.7, 0.0, 2.0), np.float32), B)
    ids, val, used = oracle.sample_online(hb, Wb, T, 21, 3, cuts)
    last_needed = 1 + int(np.searchsorted(cuts, dup0, side="right")) - 1
    assert np.all(used >= last_needed), used
    o_id, o_val, _ = oracle.sample(hb, Wb, T, 21, 3)
    assert np.array_equal(ids, o_id) and np.array_equal(val, o_val)
    # the duplicates do win on some rows: the case has teeth
    assert np.any(o_id >= dup0)


def test_confident_workload_stops_early():
    """The generator of the bench's early-finalisation case, at a small
    shape: every row is final after the first chunk."""
    w = wl.Workload(9, "online-test", D=256, V=2048, batches=(8,), w_std=0.02,
                    h_rmsnorm=True, global_V=2048)
    h = wl.make_h(w, 8)
    W = wl.make_confident_w(w, h, chunk_rows=256, later_std=0.002, gain=6.0)
    T = np.full(8, 1.0, np.float32)
    T[3] = 0.0
    cuts = np.arange(0, 2049, 256)
    hb, Wb = wl.bf16_bits(h), wl.bf16_bits(W)
    ids, val, used = oracle.sample_online(hb, Wb, T, 1, 2, cuts)
    assert np.all(used == 1), used
    assert np.array_equal(ids, np.arange(8))  # each row picks its aligned row
    o_id, _, _ = oracle.sample(hb, Wb, T, 1, 2)
    assert np.array_equal(ids, o_id)


def test_max_row_norm_matches_numpy():
    _, Wb, _ = _random(1, 96, 333, 5)
    W = (Wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert oracle.max_row_norm(Wb) == pytest.approx(np.linalg.norm(W, axis=1).max(), rel=1e-14)


def test_gumbel_max_closed_form():
    assert oracle.gumbel_max() == pytest.approx(-np.log(-np.log1p(-2.0 ** -33)), rel=1e-12)
    # and it is the map's value at the top word
    assert np.float32(oracle.gumbel_max()) == np.float32(oracle.gumbel(0xFFFFFFFF))
