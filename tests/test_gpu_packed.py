"""GPU tests of the fragment-order (packed) weight path.

fs_pack_weights re-tiles W; fs_sample_packed runs the same main loops on it,
so in one configuration its ids and scores must equal fs_sample's on the
row-major W bit for bit (same fragments, same summation order), and meet the
oracle's parity rules.  The layout itself is checked element by element against its
definition, written out here with NumPy.
"""
import numpy as np
import pytest
import torch

from conftest import gpu_available
from parity import check_rows, sample_rows, to_host

import lm_head_exact_amd as fsl
from lm_head_exact_amd import workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

DEV = "cuda"
TEMPS = (1.0, 0.5, 0.0, 1.4, 0.3, 2.0, -1.0, 0.8)


@pytest.fixture(autouse=True)
def _reset_config():
    fsl.force_config(-1)
    yield
    fsl.force_config(-1)


def _num_configs():
    try:
        return fsl.num_configs()
    except Exception:  # library not built: collection must still succeed
        return 48


def _packed_capable(cfg):
    name = fsl.config_name(cfg)
    return name.startswith(("persist", "dma", "lds"))


def _rand(B, D, V, seed, w_std=0.05):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn(B, D, generator=g).to(torch.bfloat16)
    W = (w_std * torch.randn(V, D, generator=g)).to(torch.bfloat16)
    T = torch.tensor(np.resize(np.asarray(TEMPS, np.float32), B))
    return h, W, T


@pytest.mark.parametrize("V,D,off", [(1000, 256, 0), (1531, 64, 3), (17, 96, 6), (48, 32, 1)])
def test_layout_matches_definition(V, D, off):
    _, W, _ = _rand(1, D, V, V)
    Wp = to_host(fsl.pack_weights(W.to(DEV), off).view(torch.int16)).view(np.uint16)
    Wb = wl.bf16_bits(W)
    shift = off % 4
    groups = (V + shift + 15) // 16
    assert Wp.size == groups * 16 * D
    # element ((g * D/32 + s) * 64 + l) * 8 + j = W[16g + l%16 - shift][32s + 8(l//16) + j]
    ref = np.zeros((groups, D // 32, 64, 8), np.uint16)
    for g in range(groups):
        for l in range(64):
            v = 16 * g + l % 16 - shift
            if 0 <= v < V:
                for s in range(D // 32):
                    k = 32 * s + 8 * (l // 16)
                    ref[g, s, l] = Wb[v, k:k + 8]
    assert np.array_equal(Wp.reshape(ref.shape), ref)


@pytest.mark.parametrize("cfg", range(_num_configs()))
def test_every_packed_config_equals_row_major(cfg):
    if not _packed_capable(cfg):
        pytest.skip("configuration without a packed-W kernel")
    # the last three fit the persistent kernels (D = 32 * waves * k-steps,
    # B <= 16 or 32), at offsets that do and do not start on a Philox block
    shapes = [(37, 256, 1531, 5), (4, 256, 1000, 0), (300, 128, 700, 2),
              (29, 4096, 1531, 5), (4, 4096, 1000, 0), (16, 8192, 1000, 6)]
    ran = 0
    fsl.force_config(cfg)
    for B, D, V, off in shapes:
        h, W, T = _rand(B, D, V, seed=B + V)
        try:
            Wp = fsl.pack_weights(W.to(DEV), off)
            ids_p, val_p = fsl.sample_packed(h.to(DEV), Wp, V, T.to(DEV), 11, 4, off)
        except fsl.FlashSampleError as e:
            if e.status == fsl.binding.FS_ERR_UNSUPPORTED:
                continue
            raise
        ids, val = fsl.sample(h.to(DEV), W.to(DEV), T.to(DEV), 11, 4, off)
        torch.cuda.synchronize()
        ids_p, val_p, ids, val = (to_host(t) for t in (ids_p, val_p, ids, val))
        assert np.array_equal(ids_p, ids), fsl.config_name(cfg)
        assert np.array_equal(val_p.view(np.uint32), val.view(np.uint32)), fsl.config_name(cfg)
        check_rows(wl.bf16_bits(h), wl.bf16_bits(W), to_host(T), 11, 4, off, ids_p, val_p,
                   label=f"packed {fsl.config_name(cfg)} B={B}")
        ran += 1
    if ran == 0:
        pytest.skip("configuration supports none of the test shapes")


@pytest.mark.parametrize("B", [1, 32, 64, 256])
def test_full_size_equals_row_major(B):
    """Llama-3-8B-shaped head in the configuration the bench times: every row
    bit-identical to fs_sample (both choices sum each logit in k order in one
    wave), sampled rows against the oracle."""
    w = wl.LLAMA3_8B
    h = wl.make_h(w, B, DEV)
    W = wl.make_w(w, DEV)
    T = wl.make_temperature(w, B, DEV)
    Wp = fsl.pack_weights(W)
    seed, step = w.sampler_seed(5)
    ids_p, val_p = fsl.sample_packed(h, Wp, w.V, T, seed, step)
    ids, val = fsl.sample(h, W, T, seed, step)
    torch.cuda.synchronize()
    del Wp
    assert torch.equal(ids_p, ids) and torch.equal(val_p.view(torch.int32), val.view(torch.int32))
    rows = sample_rows(B, k=6, seed=B)
    check_rows(wl.bf16_bits(h), wl.bf16_bits(W), to_host(T), seed, step, 0, to_host(ids_p),
               to_host(val_p), rows=rows, label=f"packed full B={B}")


@pytest.mark.parametrize("wk,B", [(wl.QWEN3, 1), (wl.QWEN3, 128), (wl.TP8_SHARD, 64),
                                  (wl.LARGE_BATCH, 512)])
def test_other_workloads_equal_row_major(wk, B):
    """The packed path's automatic configuration, on the row-major W too (the
    row-major choice may sum in another order: Qwen3 head at B = 1 takes the
    K-split loop there), bit for bit; sampled rows against the oracle."""
    h = wl.make_h(wk, B, DEV)
    W = wl.make_w(wk, DEV)
    T = wl.make_temperature(wk, B, DEV)
    Wp = fsl.pack_weights(W, wk.vocab_offset)
    seed, step = wk.sampler_seed(2)
    ids_p, val_p = fsl.sample_packed(h, Wp, wk.V, T, seed, step, wk.vocab_offset)
    fsl.force_config(fsl.selected_config(B, wk.D, wk.V, packed=True))
    ids, val = fsl.sample(h, W, T, seed, step, wk.vocab_offset)
    torch.cuda.synchronize()
    del Wp
    assert torch.equal(ids_p, ids) and torch.equal(val_p.view(torch.int32), val.view(torch.int32))
    rows = sample_rows(B, k=4, seed=B)
    check_rows(wl.bf16_bits(h), wl.bf16_bits(W), to_host(T), seed, step, wk.vocab_offset,
               to_host(ids_p), to_host(val_p), rows=rows, label=f"packed {wk.name} B={B}")


def test_unsupported_configuration_is_an_error():
    """A shape whose configuration has no packed-W kernel is refused."""
    B, D, V = 8, 256, 1000
    stream = [i for i in range(fsl.num_configs()) if fsl.config_name(i).startswith("stream")][0]
    fsl.force_config(stream)
    h, W, T = _rand(B, D, V, 1)
    Wp = fsl.pack_weights(W.to(DEV))
    with pytest.raises(fsl.FlashSampleError) as e:
        fsl.sample_packed(h.to(DEV), Wp, V, T.to(DEV), 1, 1)
    assert e.value.status == fsl.binding.FS_ERR_UNSUPPORTED


@pytest.mark.parametrize("cfg", range(_num_configs()))
def test_every_packed_config_partial_lse_equals_row_major(cfg):
    """The grouped sampler's per-group kernel on fragment-order W: (val, idx,
    lse) bit-identical to the row-major call in the same configuration."""
    if not _packed_capable(cfg):
        pytest.skip("configuration without a packed-W kernel")
    fsl.force_config(cfg)
    ran = 0
    for B, D, V, off in [(37, 256, 1531, 6), (4, 256, 1000, 0), (300, 128, 700, 48097),
                         (29, 4096, 1531, 7), (4, 4096, 1000, 0), (16, 8192, 1000, 6)]:
        h, W, T = _rand(B, D, V, seed=2 * B + V)
        outs = []
        try:
            for Wx, kw in ((W.to(DEV), {}), (fsl.pack_weights(W.to(DEV), off), {"V": V})):
                o = (torch.empty(B, dtype=torch.float32, device=DEV),
                     torch.empty(B, dtype=torch.int32, device=DEV),
                     torch.empty(B, dtype=torch.float32, device=DEV))
                fsl.sample_partial_lse(h.to(DEV), Wx, T.to(DEV), 7, 2, off, *o, **kw)
                outs.append([to_host(t) for t in o])
        except fsl.FlashSampleError as e:
            if e.status == fsl.binding.FS_ERR_UNSUPPORTED:
                continue
            raise
        torch.cuda.synchronize()
        (v0, i0, l0), (v1, i1, l1) = outs
        assert np.array_equal(i0, i1), fsl.config_name(cfg)
        assert np.array_equal(v0.view(np.uint32), v1.view(np.uint32)), fsl.config_name(cfg)
        assert np.array_equal(l0.view(np.uint32), l1.view(np.uint32)), fsl.config_name(cfg)
        check_rows(wl.bf16_bits(h), wl.bf16_bits(W), to_host(T), 7, 2, off, i1, v1,
                   label=f"packed lse {fsl.config_name(cfg)} B={B} D={D}")
        ran += 1
    if ran == 0:
        pytest.skip("configuration supports none of the test shapes")


def test_captured_graph_replays_match_eager():
    """fs_sample_packed captured once and replayed several times, with other
    device work between the replays, gives the eager result every time."""
    B, D, V = 64, 256, 1531
    h, W, T = _rand(B, D, V, seed=9)
    hd, Td = h.to(DEV), T.to(DEV)
    Wp = fsl.pack_weights(W.to(DEV), 2)
    ws = fsl.alloc_workspace(fsl.workspace_bytes(B, D, V), DEV)
    out = (torch.empty(B, dtype=torch.int32, device=DEV),
           torch.empty(B, dtype=torch.float32, device=DEV))
    ref = [t.clone() for t in fsl.sample_packed(hd, Wp, V, Td, 3, 4, 2)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fsl.sample_packed(hd, Wp, V, Td, 3, 4, 2, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fsl.sample_packed(hd, Wp, V, Td, 3, 4, 2, out=out, workspace=ws)
    for r in range(4):
        for t in out:
            t.fill_(-3)
        junk = torch.randn(1 << 20, device=DEV).sum()
        graph.replay()
        torch.cuda.synchronize()
        assert junk.isfinite()
        for a, b in zip(out, ref):
            assert torch.equal(a, b), f"replay {r}"


@pytest.mark.parametrize("B,D,V,off", [
    (4096, 256, 600, 0),                 # sixteen 256-row batch tiles
    (3, 256, 2000, 2**31 - 1 - 2000),    # the vocabulary ends at id 2^31 - 2
    (1, 256, 1, 2**31 - 2),              # one id (one padded group), near the top of the ids
])
def test_maximum_sizes(B, D, V, off):
    """Extremes of the argument ranges on fragment-order W: against the
    oracle, and bit-identical to the row-major call in the same configuration."""
    h, W, T = _rand(B, D, V, seed=B + V)
    hd, Wd, Td = h.to(DEV), W.to(DEV), T.to(DEV)
    Wp = fsl.pack_weights(Wd, off)
    assert Wp.numel() == ((V + off % 4 + 15) // 16) * 16 * D
    ids_p, val_p = fsl.sample_packed(hd, Wp, V, Td, 123, 456, off)
    fsl.force_config(fsl.selected_config(B, D, V, packed=True))
    ids, val = fsl.sample(hd, Wd, Td, 123, 456, off)
    torch.cuda.synchronize()
    assert torch.equal(ids_p, ids) and torch.equal(val_p.view(torch.int32), val.view(torch.int32))
    rows = None if B <= 64 else sample_rows(B, k=24, seed=1)
    check_rows(wl.bf16_bits(h), wl.bf16_bits(W), T.numpy(), 123, 456, off, to_host(ids_p),
               to_host(val_p), rows=rows, label=f"packed max B{B} V{V} off{off}")


def test_poisoned_workspace():
    """A 0xFF-filled workspace gives the same result as a fresh one."""
    B, D, V = 300, 256, 1531
    h, W, T = _rand(B, D, V, seed=12)
    hd, Td = h.to(DEV), T.to(DEV)
    Wp = fsl.pack_weights(W.to(DEV), 1)
    ref = [t.clone() for t in fsl.sample_packed(hd, Wp, V, Td, 5, 5, 1)]
    ws = fsl.alloc_workspace(fsl.workspace_bytes(B, D, V), DEV)
    ws.fill_(0xFF)
    got = fsl.sample_packed(hd, Wp, V, Td, 5, 5, 1, workspace=ws)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
