"""GPU parity of the online (chunked) sampler with early finalisation.

fs_online_bounds computes, per chunk, the largest row norm of W over the later
chunks; fs_sample_online runs the fused sampler chunk by chunk and finalises a
row once its running best exceeds (|h_b| R_c (1/T) + g_max)(1 + 2^-8).  Every
case goes through the C ABI and is compared with the oracle on the same seeded
inputs:
  * ids and scores against the plain whole-vocabulary oracle (oracle.sample)
    by the parity rules of parity.py: stopping early never changes the sample;
  * the number of chunks each row used against oracle.sample_online, exactly,
    except on rows whose oracle running best lies within BOUND_TOL (relative)
    of the oracle's bound after some chunk: there the device's fp32 scores
    (about 1e-5 from the oracle's) may fall on the other side;
  * the bounds against oracle.max_row_norm of each suffix of W (fp64 sums in
    another order: 1e-12 relative).
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
BOUND_TOL = 1e-4
MARGIN = 1.0 + 2.0 ** -8
TEMPS = (1.0, 0.3, 0.0, 1.7, 0.6, -1.0, 0.8, 2.0)


@pytest.fixture(autouse=True)
def _reset_config():
    fsl.force_config(-1)
    yield
    fsl.force_config(-1)


def _f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _aligned(B, D, V, chunk_rows, seed, norm, later_std=0.02, dup_at=None):
    """h ~ N(0,1); row b < B of W parallel to h_b with |W_b| = norm / |h_b|
    (z_bb ~= norm), other rows N(0, 0.02^2), rows after the first chunk
    N(0, later_std^2); optionally an exact copy of rows [0, B) at dup_at."""
    g = torch.Generator().manual_seed(seed)
    h = torch.randn(B, D, generator=g)
    W = 0.02 * torch.randn(V, D, generator=g)
    W[chunk_rows:] *= later_std / 0.02
    W[:B] = h / h.norm(dim=1, keepdim=True) * (norm / h.norm(dim=1, keepdim=True))
    if dup_at is not None:
        W[dup_at:dup_at + B] = W[:B]
    return h.to(torch.bfloat16), W.to(torch.bfloat16)


def _run(h, W, T, seed, step, cuts, off=0):
    hd, Wd, Td = h.to(DEV), W.to(DEV), torch.as_tensor(T).to(DEV)
    later = fsl.online_bounds(Wd, cuts)
    ids, val, used = fsl.sample_online(hd, Wd, Td, seed, step, cuts, later, vocab_offset=off)
    torch.cuda.synchronize()
    return to_host(ids), to_host(val), to_host(used), to_host(later)


def _ambiguous_rows(hb, Wb, T, seed, step, cuts, off, rows):
    """Rows whose oracle running best is within BOUND_TOL of the oracle's
    bound after some chunk before the last."""
    hn = np.linalg.norm(_f32(hb[rows]), axis=1)
    norms = np.linalg.norm(_f32(Wb), axis=1)
    g_max = oracle.gumbel_max()
    amb = np.zeros(len(rows), bool)
    for c in range(len(cuts) - 2):
        R = norms[cuts[c + 1]:].max()
        _, best, _ = oracle.sample(hb, Wb[:cuts[c + 1]], T, seed, step, off, rows)
        Tr = T[rows]
        greedy = ~(Tr > 0)
        inv_t = np.where(greedy, 1.0, (np.float32(1.0) / np.where(greedy, 1.0, Tr)).astype(np.float32))
        bound = np.where(greedy, hn * R, hn * R * inv_t + g_max) * MARGIN
        amb |= np.abs(best.astype(np.float64) - bound) <= BOUND_TOL * np.maximum(1.0, np.abs(bound))
    return amb


def _check(hb, Wb, T, seed, step, cuts, off, ids, val, used, rows=None, label=""):
    B = hb.shape[0]
    rows = np.arange(B, dtype=np.int32) if rows is None else np.asarray(rows, np.int32)
    check_rows(hb, Wb, T, seed, step, off, ids, val, rows=rows, label=label)
    _, _, o_used = oracle.sample_online(hb, Wb, T, seed, step, cuts, vocab_offset=off, rows=rows)
    amb = _ambiguous_rows(hb, Wb, T, seed, step, cuts, off, rows)
    bad = np.nonzero(~amb & (used[rows] != o_used))[0]
    assert bad.size == 0, (f"{label}: chunks used differ on rows {rows[bad][:8]}: gpu "
                           f"{used[rows][bad][:8]} oracle {o_used[bad][:8]}")
    assert np.all((used[rows] >= 1) & (used[rows] <= len(cuts) - 1))
    return o_used


def test_bounds_match_oracle():
    g = torch.Generator().manual_seed(3)
    V, D = 1531, 264
    W = (0.05 * torch.randn(V, D, generator=g)).to(torch.bfloat16)
    W[700:710] *= 3  # the largest rows sit in the middle chunk
    cuts = np.array([0, 17, 500, 701, 705, 1200, V])
    later = to_host(fsl.online_bounds(W.to(DEV), cuts))
    Wb = wl.bf16_bits(W)
    for c in range(len(cuts) - 1):
        ref = oracle.max_row_norm(Wb[cuts[c + 1]:]) if cuts[c + 1] < V else 0.0
        assert later[c] == pytest.approx(ref, rel=1e-12, abs=0.0), c
    assert later[-1] == 0.0


@pytest.mark.parametrize("seed", [1, 2])
@pytest.mark.parametrize("n", [1, 2, 7])
def test_random_inputs_match_whole_vocabulary(seed, n):
    B, D, V, off = 37, 256, 1531, 3
    g = torch.Generator().manual_seed(seed)
    h = torch.randn(B, D, generator=g).to(torch.bfloat16)
    W = (0.05 * torch.randn(V, D, generator=g)).to(torch.bfloat16)
    T = np.resize(np.asarray(TEMPS, np.float32), B)
    rng = np.random.default_rng(seed)
    cuts = np.concatenate([[0], np.sort(rng.choice(np.arange(1, V), n - 1, replace=False)), [V]])
    ids, val, used, _ = _run(h, W, T, 10 + seed, 4, cuts, off)
    _check(wl.bf16_bits(h), wl.bf16_bits(W), T, 10 + seed, 4, cuts, off, ids, val, used,
           label=f"random n={n}")


@pytest.mark.parametrize("norm", [8.0, 60.0])
@pytest.mark.parametrize("B", [5, 40, 300])
def test_aligned_rows_stop_early(norm, B):
    """norm 60: every row is final after the first chunk; norm 8: a mix of
    rows that stop after the first chunk and rows that run to the end."""
    D, V, c0 = 128, 2400, 320
    h, W = _aligned(B, D, V, c0, seed=B, norm=norm)
    T = np.resize(np.asarray(TEMPS, np.float32), B)
    cuts = np.array([0, c0, 900, 1301, V])
    ids, val, used, _ = _run(h, W, T, 77, 5, cuts, off=1)
    hb, Wb = wl.bf16_bits(h), wl.bf16_bits(W)
    o_used = _check(hb, Wb, T, 77, 5, cuts, 1, ids, val, used, label=f"aligned norm={norm}")
    if norm == 60.0:
        assert np.all(o_used == 1)
    else:
        assert np.any(o_used == 1) and np.any(o_used > 1), o_used


def test_never_stops_before_a_duplicate_of_the_winner():
    B, D, V, c0 = 64, 128, 640, 80
    cuts = np.array([0, c0, 160, 320, V])
    h, W = _aligned(B, D, V, c0, seed=11, norm=8.0, dup_at=480)
    T = np.resize(np.asarray((1.0, 0.3, 0.7, 0.0, 2.0), np.float32), B)
    ids, val, used, _ = _run(h, W, T, 21, 3, cuts)
    hb, Wb = wl.bf16_bits(h), wl.bf16_bits(W)
    _check(hb, Wb, T, 21, 3, cuts, 0, ids, val, used, label="duplicate")
    assert np.all(used == 4)


def test_zero_later_rows_stop_after_first_chunk():
    """With every later row zero the bound is g_max (1 + 2^-8) ~ 22.96; the
    aligned logits (~60) scaled by 1/T >= 1/2 exceed it on every row."""
    B, D, V, c0 = 16, 256, 1000, 128
    h, W = _aligned(B, D, V, c0, seed=5, norm=60.0, later_std=0.0)
    T = np.resize(np.asarray(TEMPS, np.float32), B)
    cuts = np.array([0, c0, 500, V])
    ids, val, used, later = _run(h, W, T, 1, 1, cuts)
    assert later[0] == 0.0
    assert np.all(used == 1)
    _check(wl.bf16_bits(h), wl.bf16_bits(W), T, 1, 1, cuts, 0, ids, val, used, label="zero")


def test_repeated_calls_reset_state():
    """A second call on the same buffers starts from a clean running state."""
    B, D, V, c0 = 40, 128, 2400, 320
    cuts = np.array([0, c0, 900, V])
    h1, W1 = _aligned(B, D, V, c0, seed=1, norm=60.0)
    h2, W2 = _aligned(B, D, V, c0, seed=2, norm=8.0)
    T = np.resize(np.asarray(TEMPS, np.float32), B)
    Td = torch.as_tensor(T).to(DEV)
    ws = fsl.alloc_workspace(fsl.online_workspace_bytes(B, D, V, 3), DEV)
    out = (torch.empty(B, dtype=torch.int32, device=DEV),
           torch.empty(B, dtype=torch.float32, device=DEV),
           torch.empty(B, dtype=torch.int32, device=DEV))
    for h, W in ((h1, W1), (h2, W2)):
        Wd = W.to(DEV)
        later = fsl.online_bounds(Wd, cuts)
        fsl.sample_online(h.to(DEV), Wd, Td, 8, 9, cuts, later, out=out, workspace=ws)
        torch.cuda.synchronize()
        ids, val, used = (to_host(t) for t in out)
        _check(wl.bf16_bits(h), wl.bf16_bits(W), T, 8, 9, cuts, 0, ids, val, used,
               label="repeat")


@pytest.mark.parametrize("B", [32, 256])
def test_full_size_confident_and_random(B):
    """Llama-3-8B-shaped head (D = 4096, V = 128256) in 8 chunks of 16032 rows,
    in the configuration the bench times: the confident weights stop every
    row after the first chunk, random weights use every chunk; sampled rows
    against the oracle."""
    w = wl.LLAMA3_8B
    h = wl.make_h(w, B, DEV)
    T = wl.make_temperature(w, B, DEV)
    cuts = np.arange(0, w.V + 1, w.V // 8)
    rows = sample_rows(B, k=6, seed=B)
    hb, Tb = wl.bf16_bits(h), to_host(T)
    for kind in ("confident", "random"):
        if kind == "confident":
            W = wl.make_confident_w(w, h, chunk_rows=w.V // 8, later_std=0.002, device=DEV)
        else:
            W = wl.make_w(w, DEV)
        seed, step = w.sampler_seed(3)
        later = fsl.online_bounds(W, cuts)
        ids, val, used = fsl.sample_online(h, W, T, seed, step, cuts, later)
        torch.cuda.synchronize()
        ids, val, used = to_host(ids), to_host(val), to_host(used)
        Wb = wl.bf16_bits(W)
        del W
        if kind == "confident":
            assert np.all(used == 1), used
            _, _, o_used = oracle.sample_online(hb, Wb, Tb, seed, step, cuts, rows=rows)
            assert np.all(o_used == 1)
        else:
            assert np.all(used == 8), used
        check_rows(hb, Wb, Tb, seed, step, 0, ids, val, rows=rows, label=f"{kind} B={B}")


def test_captured_graph_replays_match_eager():
    """The online step (init, 2 launches per chunk) captured once and replayed
    several times, with other device work between the replays, gives the
    eager result every time (it records no memset nodes)."""
    B, D, V, c0 = 40, 128, 2400, 320
    h, W = _aligned(B, D, V, c0, seed=4, norm=8.0)
    T = torch.as_tensor(np.resize(np.asarray(TEMPS, np.float32), B)).to(DEV)
    hd, Wd = h.to(DEV), W.to(DEV)
    cuts = [0, c0, 900, 1301, V]
    later = fsl.online_bounds(Wd, cuts)
    ws = fsl.alloc_workspace(fsl.online_workspace_bytes(B, D, V, 4), DEV)
    out = (torch.empty(B, dtype=torch.int32, device=DEV),
           torch.empty(B, dtype=torch.float32, device=DEV),
           torch.empty(B, dtype=torch.int32, device=DEV))
    ref = [t.clone() for t in fsl.sample_online(hd, Wd, T, 5, 6, cuts, later)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fsl.sample_online(hd, Wd, T, 5, 6, cuts, later, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fsl.sample_online(hd, Wd, T, 5, 6, cuts, later, out=out, workspace=ws)
    for r in range(4):
        for t in out:
            t.fill_(-7)
        junk = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert junk.isfinite()
        for a, b in zip(out, ref):
            assert torch.equal(a, b), f"replay {r}"
    assert (ref[2] == 1).any() and (ref[2] > 1).any()


# ---- fragment-order (packed) weights ----
def _run_packed(h, W, T, seed, step, cuts, off=0):
    hd, Wd, Td = h.to(DEV), W.to(DEV), torch.as_tensor(T).to(DEV)
    later = fsl.online_bounds(Wd, cuts)
    Wp = fsl.pack_weights(Wd, off)
    ids, val, used = fsl.sample_online(hd, Wp, Td, seed, step, cuts, later, vocab_offset=off,
                                       V=W.shape[0])
    torch.cuda.synchronize()
    return to_host(ids), to_host(val), to_host(used)


@pytest.mark.parametrize("norm", [8.0, 60.0])
@pytest.mark.parametrize("B,off", [(5, 0), (40, 3), (300, 6)])
def test_packed_aligned_rows_stop_early(norm, B, off):
    D, V, c0 = 128, 2400, 320
    h, W = _aligned(B, D, V, c0, seed=B + 1, norm=norm)
    T = np.resize(np.asarray(TEMPS, np.float32), B)
    cuts = np.array([0, c0, 896, 1296, V])
    ids, val, used = _run_packed(h, W, T, 31, 7, cuts, off)
    o_used = _check(wl.bf16_bits(h), wl.bf16_bits(W), T, 31, 7, cuts, off, ids, val, used,
                    label=f"packed aligned norm={norm} B={B}")
    if norm == 60.0:
        assert np.all(o_used == 1)


@pytest.mark.parametrize("B", [32, 256])
def test_packed_full_size_confident_and_random(B):
    """Llama-3-8B-shaped head in 8 chunks of 16032 rows (multiples of 16) on
    fragment-order W, bounds computed from the packed copy: confident weights
    stop after the first chunk, random weights use all 8; sampled rows against
    the oracle."""
    w = wl.LLAMA3_8B
    h = wl.make_h(w, B, DEV)
    T = wl.make_temperature(w, B, DEV)
    cuts = np.arange(0, w.V + 1, w.V // 8)
    rows = sample_rows(B, k=4, seed=B + 1)
    hb, Tb = wl.bf16_bits(h), to_host(T)
    for kind in ("confident", "random"):
        W = (wl.make_confident_w(w, h, chunk_rows=w.V // 8, later_std=0.002, device=DEV)
             if kind == "confident" else wl.make_w(w, DEV))
        seed, step = w.sampler_seed(4)
        Wp = fsl.pack_weights(W)
        later = fsl.online_bounds(Wp, cuts, V=w.V, D=w.D)  # from the packed copy alone
        ids, val, used = fsl.sample_online(h, Wp, T, seed, step, cuts, later, V=w.V)
        torch.cuda.synchronize()
        del Wp
        ids, val, used = to_host(ids), to_host(val), to_host(used)
        Wb = wl.bf16_bits(W)
        del W
        assert np.all(used == (1 if kind == "confident" else 8)), used
        check_rows(hb, Wb, Tb, seed, step, 0, ids, val, rows=rows, label=f"packed {kind} B={B}")


def test_poisoned_workspace():
    """Workspace contents on entry are ignored: a 0xFF-filled workspace (as
    partials, norms, flags and live counts) gives the same result as a fresh
    one, on row-major and on packed W."""
    B, D, V, c0 = 40, 128, 2400, 320
    h, W = _aligned(B, D, V, c0, seed=6, norm=8.0)
    T = torch.as_tensor(np.resize(np.asarray(TEMPS, np.float32), B)).to(DEV)
    hd, Wd = h.to(DEV), W.to(DEV)
    cuts = [0, c0, 896, V]
    later = fsl.online_bounds(Wd, cuts)
    Wp = fsl.pack_weights(Wd)
    for Wx, kw in ((Wd, {}), (Wp, {"V": V})):
        ref = [t.clone() for t in fsl.sample_online(hd, Wx, T, 2, 3, cuts, later, **kw)]
        ws = fsl.alloc_workspace(fsl.online_workspace_bytes(B, D, V, 3), DEV)
        ws.fill_(0xFF)
        got = fsl.sample_online(hd, Wx, T, 2, 3, cuts, later, workspace=ws, **kw)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
        assert (ref[2] == 1).any() and (ref[2] > 1).any()


@pytest.mark.parametrize("off", [0, 3, 6])
def test_packed_bounds_match_row_major_and_oracle(off):
    """fs_online_bounds_packed (row norms read from fragment-order W, padding
    rows skipped) against the row-major bounds and the oracle's suffix norms."""
    g = torch.Generator().manual_seed(8 + off)
    V, D = 1531, 256
    W = (0.05 * torch.randn(V, D, generator=g)).to(torch.bfloat16)
    W[700:710] *= 3
    cuts = np.array([0, 16, 496, 704, 1200, V])
    Wd = W.to(DEV)
    rm = to_host(fsl.online_bounds(Wd, cuts))
    pk = to_host(fsl.online_bounds(fsl.pack_weights(Wd, off), cuts, V=V, D=D, vocab_offset=off))
    Wb = wl.bf16_bits(W)
    for c in range(len(cuts) - 1):
        ref = oracle.max_row_norm(Wb[cuts[c + 1]:]) if cuts[c + 1] < V else 0.0
        assert pk[c] == pytest.approx(ref, rel=1e-12, abs=0.0), c
        assert pk[c] == pytest.approx(rm[c], rel=1e-12, abs=0.0), c
    assert pk[-1] == 0.0
