"""GPU parity of the grouped (hierarchical) sampler against the CPU oracle.

fs_sample_partial_lse emits one vocabulary group's (max, global argmax) --
the same pairs as fs_sample_partial -- plus the group's log-sum-exp of the
scaled logits; fs_merge_lse draws the group with probability proportional to
exp(LSE) and keeps its sample.  Every case runs the library through its C ABI
and compares with oracle.sample_lse / oracle.merge_lse on the same seeded
inputs.

Tolerances (derived from the arithmetic):
  * LSE_TOL: the device log-sum-exp accumulates fp32 exponentials of fp32
    logits with hardware exp2/log2 (relative error a few 1e-7 per term) and
    the device logits differ from the fp64-summed ones by ~1e-6 relative;
    2e-4 absolute plus 2e-6 relative is far below the change one missing
    tile makes (log(1 + its share of the mass)).
  * KEY_TOL: the group key lse + gamma uses the device Gumbel map, within
    1e-5 of the oracle's on the whole grid (checked exhaustively elsewhere);
    the chosen group must match wherever the oracle's top-two key gap
    exceeds 1e-4, and otherwise be within 1e-4 of the best key.
"""
import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from parity import check_rows, sample_rows, to_host

import lm_head_exact_amd as fsl
from lm_head_exact_amd import workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

DEV = "cuda"
LSE_TOL_ABS, LSE_TOL_REL = 2e-4, 2e-6
KEY_TOL = 1e-4


@pytest.fixture(autouse=True)
def _reset_config():
    fsl.force_config(-1)
    yield
    fsl.force_config(-1)


def _rand(B, D, V, seed, w_std=0.05, temps=(1.0, 0.5, 0.0, 1.4, 0.3, 2.0, -1.0, 0.8)):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn(B, D, generator=g).to(torch.bfloat16)
    W = (w_std * torch.randn(V, D, generator=g)).to(torch.bfloat16)
    T = torch.tensor(np.resize(np.asarray(temps, np.float32), B))
    return h, W, T


def _partial_lse(h, W, T, seed, step, off):
    B = h.shape[0]
    val = torch.empty(B, dtype=torch.float32, device=DEV)
    idx = torch.empty(B, dtype=torch.int32, device=DEV)
    lse = torch.empty(B, dtype=torch.float32, device=DEV)
    fsl.sample_partial_lse(h.to(DEV), W.to(DEV), T.to(DEV), seed, step, off, val, idx, lse)
    torch.cuda.synchronize()
    return to_host(idx), to_host(val), to_host(lse)


def _check_lse(g_lse, o_lse, label):
    err = np.abs(g_lse.astype(np.float64) - o_lse.astype(np.float64))
    tol = LSE_TOL_ABS + LSE_TOL_REL * np.abs(o_lse.astype(np.float64))
    bad = np.nonzero(~(err <= tol))[0]
    assert bad.size == 0, f"{label}: lse off on rows {bad[:8]}: gpu {g_lse[bad][:8]} oracle {o_lse[bad][:8]}"


def _num_configs():
    try:
        return fsl.num_configs()
    except Exception:  # library not built: collection must still succeed
        return 35


@pytest.mark.parametrize("cfg", range(_num_configs()))
def test_partial_lse_every_config(cfg):
    """Each configuration's LSE kernel on a tiny, a ragged (unaligned vocab
    offset, B and V off every tile) and a multi-batch-block shape, at the
    smallest D the configuration accepts; (val, idx) also bit-identical to
    fs_sample_partial's on the same configuration."""
    fsl.force_config(cfg)
    cases = [("tiny", 4, 1000, 0), ("ragged", 37, 1531, 6), ("B=300", 300, 2000, 48096)]
    ran = []
    for label, B, V, off in cases:
        for D in (256, 264, 512, 1024, 2048, 4096, 8192):
            h, W, T = _rand(B, D, V, seed=cfg * 7 + B)
            try:
                ids, val, lse = _partial_lse(h, W, T, 3, 5, off)
            except fsl.FlashSampleError as e:
                assert e.status == fsl.binding.FS_ERR_UNSUPPORTED
                continue
            hb, Wb, Tn = wl.bf16_bits(h), wl.bf16_bits(W), T.numpy()
            check_rows(hb, Wb, Tn, 3, 5, off, ids, val, label=f"{label} D={D} cfg {cfg}")
            o = oracle.sample_lse(hb, Wb, Tn, 3, 5, vocab_offset=off)
            _check_lse(lse, o[3], f"{label} D={D} cfg {cfg}")
            pv = torch.empty(B, dtype=torch.float32, device=DEV)
            pi = torch.empty(B, dtype=torch.int32, device=DEV)
            fsl.sample_partial(h.to(DEV), W.to(DEV), T.to(DEV), 3, 5, off, pv, pi)
            assert np.array_equal(to_host(pi), ids)
            assert np.array_equal(to_host(pv).view(np.uint32), val.view(np.uint32))
            ran.append(label)
            break
    assert "tiny" in ran, f"configuration {cfg} accepted none of the D values"


def _synthetic_partials(P, B, seed):
    rng = np.random.default_rng(seed)
    lse = (8.0 + 1.5 * rng.standard_normal((P, B))).astype(np.float32)
    val = (lse + rng.gumbel(size=(P, B))).astype(np.float32)
    ids = (np.arange(P)[:, None] * 1000 + rng.integers(0, 1000, size=(P, B))).astype(np.int32)
    # equal log-sum-exps of two groups on some rows (ties for greedy rows)
    if P >= 2:
        lse[1, ::11] = lse[0, ::11]
    T = np.resize(np.array([1.0, 0.7, 0.0, 1.3, -0.0, 2.0, 0.4], np.float32), B)
    return val, ids, lse, T


@pytest.mark.parametrize("P,B", [(1, 7), (2, 64), (8, 200), (67, 33), (300, 5)])
def test_merge_lse_matches_oracle(P, B):
    val, ids, lse, T = _synthetic_partials(P, B, seed=P * 31 + B)
    seed, step = 2**40 + P, 17 + B
    o_id, o_val, o_lse, o_gap = oracle.merge_lse(val, ids, lse, T, seed, step)
    g_id, g_val, g_lse = [to_host(x) for x in fsl.merge_lse(
        torch.from_numpy(val).to(DEV), torch.from_numpy(ids).to(DEV),
        torch.from_numpy(lse).to(DEV), torch.from_numpy(T).to(DEV), seed, step)]
    _check_lse(g_lse, o_lse, f"merge P={P} B={B}")
    for b in range(B):
        greedy = not (T[b] > 0)
        if g_id[b] == o_id[b] and g_val[b] == o_val[b]:
            continue
        assert not greedy, f"greedy row {b}: gpu {g_id[b]} oracle {o_id[b]}"
        assert o_gap[b] <= KEY_TOL, f"row {b}: gpu {g_id[b]} oracle {o_id[b]} gap {o_gap[b]}"
        p = int(np.nonzero(ids[:, b] == g_id[b])[0][0])
        key = np.float32(lse[p, b]) + np.float32(oracle.group_gumbel(seed, step, b, p))
        best = max(np.float32(lse[q, b]) + np.float32(oracle.group_gumbel(seed, step, b, q))
                   for q in range(P))
        assert best - key <= KEY_TOL


def test_grouped_pipeline_matches_oracle():
    """Five uneven groups with unaligned offsets, each through
    fs_sample_partial_lse into its slot, then fs_merge_lse; the oracle runs
    the same pipeline."""
    B, D, V = 24, 512, 9000
    h, W, T = _rand(B, D, V, seed=5)
    hb, Wb, Tn = wl.bf16_bits(h), wl.bf16_bits(W), T.numpy()
    cuts = [0, 1501, 3003, 5555, 7001, V]
    P = len(cuts) - 1
    pv = torch.empty(P, B, dtype=torch.float32, device=DEV)
    pi = torch.empty(P, B, dtype=torch.int32, device=DEV)
    pl = torch.empty(P, B, dtype=torch.float32, device=DEV)
    Wd, hd, Td = W.to(DEV), h.to(DEV), T.to(DEV)
    o_val, o_ids, o_lse, o_gap = [], [], [], []
    for p, (a, c) in enumerate(zip(cuts[:-1], cuts[1:])):
        fsl.sample_partial_lse(hd, Wd[a:c], Td, 9, 4, a, pv[p], pi[p], pl[p])
        oi, ov, og, ol = oracle.sample_lse(hb, Wb[a:c], Tn, 9, 4, vocab_offset=a)
        o_val.append(ov), o_ids.append(oi), o_lse.append(ol), o_gap.append(og)
    torch.cuda.synchronize()
    o_val, o_ids, o_lse, o_gap = map(np.stack, (o_val, o_ids, o_lse, o_gap))
    for p, (a, c) in enumerate(zip(cuts[:-1], cuts[1:])):
        check_rows(hb, Wb[a:c], Tn, 9, 4, a, to_host(pi[p]), to_host(pv[p]), label=f"group {p}")
    _check_lse(to_host(pl).ravel(), o_lse.ravel(), "group partials")
    g_id, g_val, g_lse = [to_host(x) for x in fsl.merge_lse(pv, pi, pl, Td, 9, 4)]
    m_id, m_val, m_lse, m_gap = oracle.merge_lse(o_val, o_ids, o_lse, Tn, 9, 4)
    _check_lse(g_lse, m_lse, "pipeline total")
    full = oracle.sample_lse(hb, Wb, Tn, 9, 4)
    _check_lse(g_lse, full[3], "pipeline total vs whole vocabulary")
    group_of = lambda gv: int(np.searchsorted(cuts, gv, side="right")) - 1
    for b in range(B):
        if g_id[b] == m_id[b]:
            continue
        # allowed only for a near tie: of the group keys, or of the tokens
        # inside the group both sides chose
        p = group_of(m_id[b])
        near = m_gap[b] <= KEY_TOL or (group_of(g_id[b]) == p and o_gap[p, b] <= 2e-3)
        assert near, f"row {b}: gpu {g_id[b]} oracle {m_id[b]} key gap {m_gap[b]}"


@pytest.mark.parametrize("wlk,B", [(wl.LLAMA3_8B, 32), (wl.LLAMA3_8B, 256), (wl.QWEN3, 128),
                                   (wl.TP8_SHARD, 64)],
                         ids=["llama3-B32", "llama3-B256", "qwen3-B128", "tp8-B64"])
def test_partial_lse_full_workloads_sampled_rows(wlk, B):
    h = wl.make_h(wlk, B, DEV)
    W = wl.make_w(wlk, DEV)
    T = wl.make_temperature(wlk, B, DEV)
    hb, Wb, Tn = wl.bf16_bits(h), wl.bf16_bits(W), to_host(T)
    rows = sample_rows(B, k=4, seed=B)
    if wlk.greedy_every:
        rows = np.unique(np.concatenate([rows, [wlk.greedy_every - 1]])).astype(np.int32)
    seed, step = wlk.sampler_seed(1)
    val = torch.empty(B, dtype=torch.float32, device=DEV)
    idx = torch.empty(B, dtype=torch.int32, device=DEV)
    lse = torch.empty(B, dtype=torch.float32, device=DEV)
    fsl.sample_partial_lse(h, W, T, seed, step, wlk.vocab_offset, val, idx, lse)
    torch.cuda.synchronize()
    check_rows(hb, Wb, Tn, seed, step, wlk.vocab_offset, to_host(idx), to_host(val), rows=rows,
               label=f"{wlk.name} B={B} lse")
    o = oracle.sample_lse(hb, Wb, Tn, seed, step, vocab_offset=wlk.vocab_offset, rows=rows)
    _check_lse(to_host(lse)[rows], o[3], f"{wlk.name} B={B}")
    del h, W
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# All groups in one launch (fs_sample_groups_lse)
# ---------------------------------------------------------------------------
GROUP_CASES = [
    # (B, D, V, vocab_offset, cuts)
    (24, 512, 9000, 0, [0, 1501, 3003, 5555, 7001, 9000]),        # uneven groups
    (37, 256, 1531, 6, [0, 1, 17, 700, 1531]),                      # a one-row group
    (300, 256, 2600, 3, [0, 1300, 2600]),                           # several batch blocks
    (5, 4096, 3000, 1, [0, 1000, 2000, 3000]),                      # D = 4096, small batch
    (29, 4096, 2003, 5, [0, 1, 16, 700, 1300, 2003]),               # two batch tiles, one-row group
    (3, 8192, 1200, 2, [0, 17, 600, 1200]),                         # D = 8192
]


def _lse_exact(name):
    """Batch-tiled configurations cover each group with the same blocks in
    one launch as in a separate call; the persistent ones split a group's
    16-row groups over their blocks differently, so a group's log-sum-exp
    partials are added in another order."""
    return not name.startswith("persist")


def _groups_separately(h, W, T, seed, step, off, cuts):
    """Slot g by one fs_sample_partial_lse call over group g."""
    B, G = h.shape[0], len(cuts) - 1
    pv = torch.empty(G, B, dtype=torch.float32, device=DEV)
    pi = torch.empty(G, B, dtype=torch.int32, device=DEV)
    pl = torch.empty(G, B, dtype=torch.float32, device=DEV)
    hd, Wd, Td = h.to(DEV), W.to(DEV), T.to(DEV)
    for g, (a, c) in enumerate(zip(cuts[:-1], cuts[1:])):
        fsl.sample_partial_lse(hd, Wd[a:c], Td, seed, step, off + a, pv[g], pi[g], pl[g])
    torch.cuda.synchronize()
    return to_host(pv), to_host(pi), to_host(pl)


@pytest.mark.parametrize("cfg", range(_num_configs()))
def test_groups_one_launch_every_config_equals_separate_calls(cfg):
    """In one configuration the one-launch slots hold the separate calls'
    values and ids bit for bit (each logit is summed the same way), and
    their log-sum-exps bit for bit or, on the persistent configurations,
    within rounding."""
    name = fsl.config_name(cfg)
    fsl.force_config(cfg)
    ran = 0
    for B, D, V, off, cuts in GROUP_CASES:
        h, W, T = _rand(B, D, V, seed=B + V)
        try:
            pv, pi, pl = fsl.sample_groups_lse(h.to(DEV), W.to(DEV), T.to(DEV), 13, 5, cuts, off)
        except fsl.FlashSampleError as e:
            assert e.status == fsl.binding.FS_ERR_UNSUPPORTED, (name, str(e))
            continue
        torch.cuda.synchronize()
        sv, si, sl = _groups_separately(h, W, T, 13, 5, off, cuts)
        pv, pi, pl = to_host(pv), to_host(pi), to_host(pl)
        assert np.array_equal(pi, si), (name, B, D, V)
        assert np.array_equal(pv.view(np.uint32), sv.view(np.uint32)), (name, B, D, V)
        if _lse_exact(name):
            assert np.array_equal(pl.view(np.uint32), sl.view(np.uint32)), (name, B, D, V)
        else:
            _check_lse(pl.ravel(), sl.ravel(), f"{name} B={B} D={D} V={V}")
        ran += 1
    if ran == 0:
        pytest.skip("configuration supports none of the test shapes")


@pytest.mark.parametrize("case", range(len(GROUP_CASES)))
def test_groups_one_launch_matches_oracle(case):
    """The automatic choice, every group against oracle.sample_lse over its
    slice on every row; then fs_merge_lse against the oracle merge."""
    B, D, V, off, cuts = GROUP_CASES[case]
    h, W, T = _rand(B, D, V, seed=3 * B + V)
    hb, Wb, Tn = wl.bf16_bits(h), wl.bf16_bits(W), T.numpy()
    pv, pi, pl = fsl.sample_groups_lse(h.to(DEV), W.to(DEV), T.to(DEV), 21, 2, cuts, off)
    torch.cuda.synchronize()
    o_val, o_ids, o_lse = [], [], []
    for g, (a, c) in enumerate(zip(cuts[:-1], cuts[1:])):
        check_rows(hb, Wb[a:c], Tn, 21, 2, off + a, to_host(pi[g]), to_host(pv[g]),
                   label=f"one launch group {g}")
        oi, ov, og, ol = oracle.sample_lse(hb, Wb[a:c], Tn, 21, 2, vocab_offset=off + a)
        o_val.append(ov), o_ids.append(oi), o_lse.append(ol)
    o_val, o_ids, o_lse = map(np.stack, (o_val, o_ids, o_lse))
    _check_lse(to_host(pl).ravel(), o_lse.ravel(), "one-launch group partials")
    g_id, g_val, g_lse = [to_host(x) for x in fsl.merge_lse(pv, pi, pl, T.to(DEV), 21, 2)]
    m_id, m_val, m_lse, m_gap = oracle.merge_lse(o_val, o_ids, o_lse, Tn, 21, 2)
    _check_lse(g_lse, m_lse, "one-launch total")
    full = oracle.sample_lse(hb, Wb, Tn, 21, 2, vocab_offset=off)
    _check_lse(g_lse, full[3], "one-launch total vs whole vocabulary")
    ok = (g_id == m_id) | (m_gap <= KEY_TOL)
    # remaining mismatches: the same group chosen, a near tie of its tokens
    for b in np.nonzero(~ok)[0]:
        p = int(np.searchsorted(cuts, m_id[b] - off, side="right")) - 1
        assert int(np.searchsorted(cuts, g_id[b] - off, side="right")) - 1 == p, b
        a, c = cuts[p], cuts[p + 1]
        _, _, og, _ = oracle.sample_lse(hb, Wb[a:c], Tn, 21, 2, vocab_offset=off + a, rows=[b])
        assert og[0] <= 2e-3, f"row {b}: gpu {g_id[b]} oracle {m_id[b]}"


def test_groups_one_launch_packed_equals_row_major():
    """Fragment-order W (group starts multiples of 16, unaligned offset): the
    slots equal the row-major one-launch call's in the same configuration."""
    B, D, V, off = 40, 512, 5000, 7
    cuts = [0, 1024, 1040, 3200, V]
    h, W, T = _rand(B, D, V, seed=77)
    hd, Wd, Td = h.to(DEV), W.to(DEV), T.to(DEV)
    Wp = fsl.pack_weights(Wd, off)
    pk = fsl.sample_groups_lse(hd, Wp, Td, 4, 9, cuts, off, V=V)
    fsl.force_config(fsl.selected_config(B, D, V, packed=True, grouped=True))
    rm = fsl.sample_groups_lse(hd, Wd, Td, 4, 9, cuts, off)
    torch.cuda.synchronize()
    for a_, b_ in zip(pk, rm):
        assert np.array_equal(to_host(a_).view(np.uint32), to_host(b_).view(np.uint32))
    hb, Wb, Tn = wl.bf16_bits(h), wl.bf16_bits(W), T.numpy()
    for g, (a, c) in enumerate(zip(cuts[:-1], cuts[1:])):
        check_rows(hb, Wb[a:c], Tn, 4, 9, off + a, to_host(pk[1][g]), to_host(pk[0][g]),
                   label=f"packed one launch group {g}")


@pytest.mark.parametrize("B", [32, 256])
def test_groups_one_launch_full_size_eight_groups(B):
    """Llama-3-8B-shaped head in 8 groups of 16032 rows at B = 32 (the
    persistent kernel) and 256 (the DMA-staged loop), as the bench times
    them: sampled rows of every group against the oracle, and the merged
    draw's total log-sum-exp against the oracle's whole-vocabulary one."""
    w = wl.LLAMA3_8B
    h = wl.make_h(w, B, DEV)
    W = wl.make_w(w, DEV)
    T = wl.make_temperature(w, B, DEV)
    cuts = list(range(0, w.V + 1, w.V // 8))
    seed, step = w.sampler_seed(3)
    pv, pi, pl = fsl.sample_groups_lse(h, W, T, seed, step, cuts)
    _, _, lse = fsl.merge_lse(pv, pi, pl, T, seed, step)
    torch.cuda.synchronize()
    hb, Wb, Tn = wl.bf16_bits(h), wl.bf16_bits(W), to_host(T)
    rows = sample_rows(B, k=4, seed=8)
    for g, (a, c) in enumerate(zip(cuts[:-1], cuts[1:])):
        check_rows(hb, Wb[a:c], Tn, seed, step, a, to_host(pi[g]), to_host(pv[g]), rows=rows,
                   label=f"8 groups, group {g}")
    o = oracle.sample_lse(hb, Wb, Tn, seed, step, rows=rows)
    _check_lse(to_host(lse)[rows], o[3], "8 groups total")
    del h, W
    torch.cuda.empty_cache()


@pytest.mark.parametrize("D", [256, 4096])
def test_groups_one_launch_sixty_four_groups(D):
    """The largest group table (64 groups, among them one-row groups and
    groups shorter than a block), row-major at an unaligned offset and in
    fragment order, on a batch-tiled (D = 256) and a persistent (D = 4096)
    configuration: slots equal separate per-group calls (log-sum-exps within
    rounding on the persistent one), every group meets the oracle on every
    row, and fragment order equals row-major bit for bit."""
    B, V, off = 9, 6000, 3
    rng = np.random.default_rng(64)
    inner = np.sort(rng.choice(np.arange(1, V), size=63, replace=False))
    inner[:3] = [1, 2, 3]                                  # three one-row groups
    cuts = [0] + sorted(set(int(x) for x in inner)) + [V]
    assert len(cuts) == 65
    h, W, T = _rand(B, D, V, seed=640)
    hd, Wd, Td = h.to(DEV), W.to(DEV), T.to(DEV)
    pv, pi, pl = fsl.sample_groups_lse(hd, Wd, Td, 8, 1, cuts, off)
    cfg = fsl.selected_config(B, D, V, grouped=True)
    assert fsl.config_name(cfg).startswith("persist") == (D == 4096)
    fsl.force_config(cfg)
    sv, si, sl = _groups_separately(h, W, T, 8, 1, off, cuts)
    fsl.force_config(-1)
    pv, pi, pl = to_host(pv), to_host(pi), to_host(pl)
    assert np.array_equal(pi, si)
    assert np.array_equal(pv.view(np.uint32), sv.view(np.uint32))
    if _lse_exact(fsl.config_name(cfg)):
        assert np.array_equal(pl.view(np.uint32), sl.view(np.uint32))
    else:
        _check_lse(pl.ravel(), sl.ravel(), "64 groups, persistent")
    hb, Wb, Tn = wl.bf16_bits(h), wl.bf16_bits(W), T.numpy()
    for g, (a, c) in enumerate(zip(cuts[:-1], cuts[1:])):
        check_rows(hb, Wb[a:c], Tn, 8, 1, off + a, pi[g], pv[g], label=f"64 groups, group {g}")
    # fragment order: group starts rounded to multiples of 16
    pcuts = sorted(set([0] + [c - c % 16 for c in cuts[1:-1] if c >= 16] + [V]))
    Wp = fsl.pack_weights(Wd, off)
    qv, qi, ql = fsl.sample_groups_lse(hd, Wp, Td, 8, 1, pcuts, off, V=V)
    fsl.force_config(fsl.selected_config(B, D, V, packed=True, grouped=True))
    rv, ri, rl = fsl.sample_groups_lse(hd, Wd, Td, 8, 1, pcuts, off)
    fsl.force_config(-1)
    torch.cuda.synchronize()
    for x, y in ((qv, rv), (qi, ri), (ql, rl)):
        assert np.array_equal(to_host(x).view(np.uint32), to_host(y).view(np.uint32))
