"""The unfused baseline (logits and probabilities in device memory) samples
the same ids as the oracle under the same rules as the fused path."""
import numpy as np
import pytest
import torch

from conftest import gpu_available
from parity import check_rows, inputs_host_and_device, to_host

import lm_head_exact_amd as fsl
from lm_head_exact_amd import workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]
DEV = "cuda"


@pytest.mark.parametrize("B,D,V,off", [(4, 256, 1000, 0), (37, 264, 5000, 3), (1, 64, 1, 0),
                                       (130, 128, 9001, 48096)])
def test_unfused_small(B, D, V, off):
    g = torch.Generator().manual_seed(V + B)
    h = torch.randn(B, D, generator=g).to(torch.bfloat16)
    W = (0.05 * torch.randn(V, D, generator=g)).to(torch.bfloat16)
    T = (0.3 + 1.2 * torch.rand(B, generator=g)).float()
    T[::7] = 0.0
    ids, val = fsl.sample_unfused(h.to(DEV), W.to(DEV), T.to(DEV), 9, 10, vocab_offset=off)
    check_rows(wl.bf16_bits(h), wl.bf16_bits(W), T.numpy(), 9, 10, off, to_host(ids),
               to_host(val), label=f"unfused B{B}")


@pytest.mark.parametrize("wlk,B", [(wl.LLAMA3_8B, 8), (wl.QWEN3, 64)])
def test_unfused_full_size_sampled_rows(wlk, B):
    h, W, T, hb, Wb, Tn = inputs_host_and_device(wlk, B)
    seed, step = wlk.sampler_seed(0)
    ids, val = fsl.sample_unfused(h, W, T, seed, step)
    f_ids, f_val = fsl.sample(h, W, T, seed, step)
    rows = np.array([0, 3, 7] if B == 8 else [0, 7, 15, 33, 63], np.int32)
    check_rows(hb, Wb, Tn, seed, step, 0, to_host(ids), to_host(val), rows=rows,
               label=f"unfused {wlk.name}")
    assert np.mean(to_host(ids) == to_host(f_ids)) > 0.9
