"""Seeded random shapes through the automatic configuration choice.

Each case draws a batch size, row length (a multiple of 8), vocabulary size,
vocab_offset, weight scale, temperature mix (greedy, negative and NaN rows
among them) and group cuts from a fixed seed, so every run checks the same
cases, and runs fs_sample, fs_sample_packed (D % 32 == 0) and
fs_sample_groups_lse, each against the oracle on every row (the parity rules
of tests/parity.py).  Sizes keep B * V * D below 4e8 so that the oracle takes
a fraction of a second per case.
"""
import numpy as np
import pytest
import torch

from conftest import gpu_available
from parity import check_rows, to_host

import lm_head_exact_amd as fsl
from lm_head_exact_amd import workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

DEV = "cuda"
BATCHES = [1, 2, 3, 5, 8, 13, 16, 17, 24, 31, 32, 33, 47, 64, 65, 100, 128, 129, 200, 256, 300]
ROWS = [8, 24, 64, 136, 256, 512, 1024, 2048, 4096]


def _case(k):
    rng = np.random.default_rng(7000 + k)
    B = int(rng.choice(BATCHES))
    D = int(rng.choice(ROWS))
    if k >= 20:  # the persistent kernels' row lengths and batch sizes
        D = 4096 if k % 2 == 0 else 8192
        B = int(rng.choice([1, 3, 8, 16, 17, 29, 32] if D == 4096 else [1, 5, 12, 16]))
    V = int(rng.integers(1, 6000))
    while B * V * D > 4e8:
        V = max(1, V // 2)
    off = int(rng.integers(0, 50000))
    w_std = float(rng.choice([0.02, 0.05, 0.2]))
    g = torch.Generator().manual_seed(100 + k)
    h = torch.randn(B, D, generator=g).to(torch.bfloat16)
    W = (w_std * torch.randn(V, D, generator=g)).to(torch.bfloat16)
    T = (0.3 + 1.7 * torch.rand(B, generator=g)).float()
    special = rng.random(B)
    T[torch.from_numpy(special < 0.10)] = 0.0
    T[torch.from_numpy((special >= 0.10) & (special < 0.13))] = -1.0
    T[torch.from_numpy((special >= 0.13) & (special < 0.15))] = float("nan")
    G = int(rng.integers(1, min(8, V) + 1))
    cuts = [0] + sorted(int(x) for x in rng.choice(np.arange(1, V), size=G - 1, replace=False)) + [V] \
        if G > 1 else [0, V]
    seed, step = int(rng.integers(0, 2**63)), int(rng.integers(0, 2**40))
    return B, D, V, off, h, W, T, cuts, seed, step


@pytest.fixture(autouse=True)
def _reset_config():
    fsl.force_config(-1)
    yield
    fsl.force_config(-1)


@pytest.mark.parametrize("k", range(26))
def test_random_shape(k):
    B, D, V, off, h, W, T, cuts, seed, step = _case(k)
    label = f"case {k}: B={B} D={D} V={V} off={off} groups={len(cuts) - 1}"
    print(label, fsl.config_name(fsl.selected_config(B, D, V)), flush=True)
    hd, Wd, Td = h.to(DEV), W.to(DEV), T.to(DEV)
    hb, Wb, Tn = wl.bf16_bits(h), wl.bf16_bits(W), T.numpy()

    ids, val = fsl.sample(hd, Wd, Td, seed, step, vocab_offset=off)
    torch.cuda.synchronize()
    check_rows(hb, Wb, Tn, seed, step, off, to_host(ids), to_host(val), label=label + " fs_sample")

    if D % 32 == 0:
        Wp = fsl.pack_weights(Wd, off)
        try:
            pids, pval = fsl.sample_packed(hd, Wp, V, Td, seed, step, vocab_offset=off)
        except fsl.FlashSampleError as e:  # no fragment-order kernel for this shape's choice
            assert e.status == fsl.binding.FS_ERR_UNSUPPORTED, str(e)
        else:
            torch.cuda.synchronize()
            check_rows(hb, Wb, Tn, seed, step, off, to_host(pids), to_host(pval),
                       label=label + " fs_sample_packed")

    pv, pi, _ = fsl.sample_groups_lse(hd, Wd, Td, seed, step, cuts, off)
    torch.cuda.synchronize()
    for gi, (a, c) in enumerate(zip(cuts[:-1], cuts[1:])):
        check_rows(hb, Wb[a:c], Tn, seed, step, off + a, to_host(pi[gi]), to_host(pv[gi]),
                   label=label + f" group {gi}")
