"""fs_merge bit-exact against the oracle's merge, and the vocabulary-shard
flow (one GPU's share of a tensor-parallel step, then the cross-shard
argmax)."""
import numpy as np
import pytest
import torch

from conftest import gpu_available
from parity import check_rows, to_host

import oracle
import lm_head_exact_amd as fsl
from lm_head_exact_amd import workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]
DEV = "cuda"


@pytest.mark.parametrize("P,B", [(1, 1), (2, 5), (8, 256), (9, 1000), (501, 33), (2004, 7),
                                 (64, 4097)])
def test_merge_bit_exact(P, B):
    rng = np.random.default_rng(P * 31 + B)
    val = rng.normal(size=(P, B)).astype(np.float32)
    idx = rng.integers(0, 2**31 - 1, size=(P, B)).astype(np.int32)
    tie = rng.random(B) < 0.25
    if P > 1:
        a, b = rng.integers(0, P, size=2)
        val[a, tie] = 7.5
        val[b, tie] = 7.5
    val[:, : min(B, 3)] = -3.25                       # whole-column ties
    for trial in range(2):
        perm = rng.permutation(P)
        v, i = val[perm], idx[perm]
        g_ids, g_val = fsl.merge(torch.from_numpy(v).to(DEV), torch.from_numpy(i).to(DEV))
        o_ids, o_val = oracle.merge(v, i)
        assert np.array_equal(to_host(g_ids), o_ids)
        assert np.array_equal(to_host(g_val).view(np.uint32), o_val.view(np.uint32))


@pytest.mark.parametrize("B", [1, 64, 256])
def test_tp_shard_partial_plus_synthetic_slots(B):
    """Shard 3 of 8 (D=8192, V_shard=16032, vocab_offset=48096) emitted into
    slot 3 of a P x B buffer whose other slots are seeded synthetic partials,
    then merged on the GPU; the oracle merges the same synthetic slots with
    its own shard-3 result."""
    wlk = wl.TP8_SHARD
    h = wl.make_h(wlk, B, DEV)
    W = wl.make_w(wlk, DEV)
    T = wl.make_temperature(wlk, B, DEV)
    pv, pi = wl.make_shard_partials(B, P=8, V_shard=wlk.V, real_slot=3, seed=500 + B)
    pv_d, pi_d = pv.clone().to(DEV), pi.clone().to(DEV)
    seed, step = wlk.sampler_seed(0)
    fsl.sample_partial(h, W, T, seed, step, wlk.vocab_offset, pv_d[3], pi_d[3])
    g_ids, g_val = fsl.merge(pv_d, pi_d)
    torch.cuda.synchronize()
    hb, Wb, Tn = wl.bf16_bits(h), wl.bf16_bits(W), to_host(T)
    rows = np.arange(B, dtype=np.int32) if B <= 8 else np.unique(
        np.concatenate([np.arange(0, B, B // 6), [5, B - 1]])).astype(np.int32)
    # slot 3 itself against the oracle on the checked rows
    check_rows(hb, Wb, Tn, seed, step, wlk.vocab_offset, to_host(pi_d[3]), to_host(pv_d[3]),
               rows=rows, label=f"shard3 B={B}")
    o_ids, o_val, o_gap = oracle.sample(hb, Wb, Tn, seed, step, wlk.vocab_offset, rows)
    v_ref, i_ref = pv.numpy()[:, rows].copy(), pi.numpy()[:, rows].copy()
    v_ref[3], i_ref[3] = o_val, o_ids
    m_ids, m_val = oracle.merge(v_ref, i_ref)
    gi, gv = to_host(g_ids)[rows], to_host(g_val)[rows]
    assert np.all(np.abs(gv - m_val) <= 1e-3)
    decided = (o_gap > 2e-3) | (i_ref[3] != m_ids)   # shard 3 lost, or won clearly
    assert np.array_equal(gi[decided], m_ids[decided])


def test_eight_shards_merge_to_full_vocabulary():
    """All eight shards of one global W (global V = 128256) through
    fs_sample_partial + fs_merge equal one fs_sample over the whole
    vocabulary, bit for bit, and the oracle on sampled rows."""
    B, D, Vg, P = 24, 256, 128256, 8
    g = torch.Generator(device=DEV).manual_seed(42)
    h = torch.randn(B, D, generator=g, device=DEV).to(torch.bfloat16)
    W = (0.05 * torch.randn(Vg, D, generator=g, device=DEV)).to(torch.bfloat16)
    T = torch.full((B,), 0.9, device=DEV)
    T[::5] = 0.0
    full_ids, full_val = fsl.sample(h, W, T, 11, 12)
    vs = Vg // P
    pv = torch.empty(P, B, device=DEV)
    pi = torch.empty(P, B, dtype=torch.int32, device=DEV)
    for p in range(P):
        fsl.sample_partial(h, W[p * vs:(p + 1) * vs], T, 11, 12, p * vs, pv[p], pi[p])
    m_ids, m_val = fsl.merge(pv, pi)
    assert torch.equal(m_ids, full_ids) and torch.equal(m_val, full_val)
    rows = np.array([0, 1, 7, 13, 23], np.int32)
    check_rows(wl.bf16_bits(h), wl.bf16_bits(W), to_host(T), 11, 12, 0, to_host(full_ids),
               to_host(full_val), rows=rows, label="full-V")
