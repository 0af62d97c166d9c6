"""Pin of the oracle's logits against a library matmul (CPU only).

The LM head computes logits = h W^T (wiki summary, "Method", step 1 of the
decode step).  The oracle sums each dot product in fp64 in increasing d and
rounds once to fp32; NumPy's fp64 matmul (a BLAS routine with its own
summation order) must agree to within one fp32 ulp.
"""
import numpy as np
import pytest
import torch

from lm_head_exact_amd import workloads as wl


def _f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("B,D,V", [(4, 256, 1000), (3, 520, 77), (1, 8, 5)])
def test_logits_match_fp64_matmul(orc, B, D, V):
    g = torch.Generator().manual_seed(B * 1000 + D)
    h = torch.randn(B, D, generator=g).to(torch.bfloat16)
    W = (0.05 * torch.randn(V, D, generator=g)).to(torch.bfloat16)
    hb, Wb = wl.bf16_bits(h), wl.bf16_bits(W)
    z = orc.logits(hb, Wb)
    ref = _f64(hb) @ _f64(Wb).T
    ref32 = ref.astype(np.float32)
    ulp = np.spacing(np.abs(ref32))
    assert np.all(np.abs(z.astype(np.float64) - ref) <= ulp)
    # single-element entry point agrees with the batched one
    assert orc.logit(hb[B - 1], Wb[V - 1]) == z[B - 1, V - 1]


def test_logits_tiny_workload(orc):
    h, W, _ = wl.make_inputs(wl.TINY, 4)
    hb, Wb = wl.bf16_bits(h), wl.bf16_bits(W)
    z = orc.logits(hb, Wb)
    ref = _f64(hb) @ _f64(Wb).T
    assert np.all(np.abs(z - ref) <= np.spacing(np.abs(ref.astype(np.float32))))
    # N(0,1) against N(0, 0.05^2) over D = 256: z has std ~ 0.05 * 16 = 0.8
    assert 0.6 < z.std() < 1.0
