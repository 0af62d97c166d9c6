"""The allocation-free entry point (fs_sample_packed_noalloc) against the
entry point it varies (fs_sample_packed): the same kernels over the same
fragments, so ids and scores must agree bit for bit -- on two calls in a row,
the second with a smaller input, since every call shares the library's
scratch array and the second must not see the first's partials."""
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


def _inputs(B, D, V, seed, off):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn(B, D, generator=g).to(torch.bfloat16)
    W = (0.05 * torch.randn(V, D, generator=g)).to(torch.bfloat16)
    T = torch.tensor(np.resize(np.asarray([1.0, 0.5, 0.0, 1.3], np.float32), B))
    return h, W, T


@pytest.mark.parametrize("shapes", [
    [(300, 256, 3001, 5), (7, 256, 1531, 5)],     # batch-tiled kernel, then a small one
    [(32, 4096, 5000, 0), (3, 4096, 2000, 2)],    # persistent kernels
])
def test_noalloc_equals_workspace_call(shapes):
    for B, D, V, off in shapes:
        print(f"noalloc B={B} D={D} V={V} off={off}", flush=True)
        h, W, T = _inputs(B, D, V, seed=B + V, off=off)
        hd, Td = h.to(DEV), T.to(DEV)
        Wp = fsl.pack_weights(W.to(DEV), off)
        ids0, val0 = fsl.sample_packed(hd, Wp, V, Td, 21, 4, off)
        out = (torch.empty(B, dtype=torch.int32, device=DEV),
               torch.empty(B, dtype=torch.float32, device=DEV))
        ids1, val1 = fsl.sample_packed_noalloc(hd, Wp, V, Td, 21, 4, off, out=out)
        torch.cuda.synchronize()
        ids0, val0, ids1, val1 = (to_host(t) for t in (ids0, val0, ids1, val1))
        assert np.array_equal(ids1, ids0)
        assert np.array_equal(val1.view(np.uint32), val0.view(np.uint32))
        check_rows(wl.bf16_bits(h), wl.bf16_bits(W), T.numpy(), 21, 4, off, ids1, val1,
                   label=f"noalloc B={B}")


def test_noalloc_refuses_shapes_beyond_the_scratch_array():
    """Partials beyond the 8 MiB array: refused before any launch."""
    B, D, V = 2048, 256, 200000
    h = torch.zeros(B, D, dtype=torch.bfloat16, device=DEV)
    T = torch.ones(B, device=DEV)
    Wp = torch.zeros(fsl.packed_weights_bytes(V, D, 0) // 2, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fsl.FlashSampleError) as e:
        fsl.sample_packed_noalloc(h, Wp, V, T, 1, 1)
    assert e.value.status == fsl.binding.FS_ERR_WORKSPACE
