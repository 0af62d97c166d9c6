"""The library's calls inside a captured HIP graph (torch.cuda.graph).

The sampler allocates nothing and records only kernel launches (no memset or
copy nodes), so a decode step can be captured once and replayed.  Each test
replays several times, with the program's own eager work and
synchronisations between replays, and checks every replay bit for bit
against the eager call on the same inputs.
"""
import numpy as np
import pytest
import torch

from conftest import gpu_available
from parity import to_host

import lm_head_exact_amd as fsl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

DEV = "cuda"


@pytest.fixture(autouse=True)
def _reset_config():
    fsl.force_config(-1)
    yield
    fsl.force_config(-1)


def _inputs(B, D, V, seed):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn(B, D, generator=g).to(torch.bfloat16).to(DEV)
    W = (0.05 * torch.randn(V, D, generator=g)).to(torch.bfloat16).to(DEV)
    T = torch.tensor(np.resize(np.array([1.0, 0.6, 0.0, 1.7], np.float32), B)).to(DEV)
    return h, W, T


def _replay_and_check(graph, outs, refs):
    for r in range(3):
        for o in outs:
            o.fill_(-7)
        noise = torch.randn(1 << 16, device=DEV).abs().sum()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert float(noise) > 0
        for o, ref in zip(outs, refs):
            assert np.array_equal(to_host(o).view(np.uint32), ref.view(np.uint32)), f"replay {r}"


@pytest.mark.parametrize("B,D,V,config", [(20, 512, 3000, None), (40, 512, 5000, "dma_mr2_nt16_nw8_kc64_p4_s4_br4_g2"),
                                          (8, 4096, 4000, "persist_nt1_nw8_ks16_p8")])
def test_sample_graph_replays_match_eager(B, D, V, config):
    if config is not None:
        names = [fsl.config_name(i) for i in range(fsl.num_configs())]
        fsl.force_config(names.index(config))
    h, W, T = _inputs(B, D, V, seed=B + V)
    ref = [to_host(x) for x in fsl.sample(h, W, T, 11, 12, vocab_offset=5)]
    out = (torch.empty(B, dtype=torch.int32, device=DEV), torch.empty(B, device=DEV))
    ws = fsl.alloc_workspace(fsl.workspace_bytes(B, D, V), DEV)
    fsl.sample(h, W, T, 11, 12, vocab_offset=5, out=out, workspace=ws)  # one-time set-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fsl.sample(h, W, T, 11, 12, vocab_offset=5, out=out, workspace=ws)
    _replay_and_check(graph, out, ref)


def test_grouped_step_graph_replays_match_eager():
    B, D, V, G = 16, 256, 4000, 4
    h, W, T = _inputs(B, D, V, seed=3)
    Vg = V // G
    pv = torch.empty(G, B, device=DEV)
    pi = torch.empty(G, B, dtype=torch.int32, device=DEV)
    pl = torch.empty(G, B, device=DEV)
    ws = fsl.alloc_workspace(fsl.workspace_bytes(B, D, Vg), DEV)
    outs = (torch.empty(B, dtype=torch.int32, device=DEV), torch.empty(B, device=DEV),
            torch.empty(B, device=DEV))

    def step():
        for p in range(G):
            fsl.sample_partial_lse(h, W[p * Vg:(p + 1) * Vg], T, 21, 22, p * Vg, pv[p], pi[p],
                                   pl[p], workspace=ws)
        fsl.merge_lse(pv, pi, pl, T, 21, 22, out=outs)

    step()
    torch.cuda.synchronize()
    refs = [to_host(o).copy() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    _replay_and_check(graph, outs, refs)


@pytest.mark.parametrize("B,D,V", [(16, 4096, 4000), (70, 256, 4000)])
def test_grouped_one_launch_graph_replays_match_eager(B, D, V):
    """fs_sample_groups_lse then fs_merge_lse in one captured graph, on the
    persistent kernel (D = 4096, small batch) and on a batch-tiled one."""
    cuts = [0, 999, 1000, 2600, V]
    G = len(cuts) - 1
    h, W, T = _inputs(B, D, V, seed=B + 5)
    pv = torch.empty(G, B, device=DEV)
    pi = torch.empty(G, B, dtype=torch.int32, device=DEV)
    pl = torch.empty(G, B, device=DEV)
    ws = fsl.alloc_workspace(fsl.groups_workspace_bytes(B, D, V, G), DEV)
    outs = (torch.empty(B, dtype=torch.int32, device=DEV), torch.empty(B, device=DEV),
            torch.empty(B, device=DEV))

    def step():
        fsl.sample_groups_lse(h, W, T, 31, 32, cuts, vocab_offset=3, out=(pv, pi, pl), workspace=ws)
        fsl.merge_lse(pv, pi, pl, T, 31, 32, out=outs)

    step()
    torch.cuda.synchronize()
    refs = [to_host(o).copy() for o in (*outs, pv, pi, pl)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    _replay_and_check(graph, (*outs, pv, pi, pl), refs)
