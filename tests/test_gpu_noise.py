"""GPU noise field against the oracle: raw Philox words bit-exact, Gumbel
values exhaustively over the whole 2^23-point uniform grid."""
import numpy as np
import pytest
import torch

from conftest import gpu_available

import oracle
import lm_head_exact_amd as fsl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

G_TOL = 1e-5  # absolute, fp32 device evaluation vs fp64-rounded oracle


@pytest.mark.parametrize("seed,step,row,gv0,n", [
    (0, 0, 0, 0, 1 << 20),
    (2**64 - 1, 2**64 - 1, 2**32 - 1, 2**32 - (1 << 16), 1 << 16),
    (0x0123456789ABCDEF, 0xFEDCBA9876543210, 77, 48096, 16032),
    (5000, 3, 255, 128256 - 1000, 1000),
    (1, 1, 1, 3, 4097),
])
def test_noise_words_bit_exact(seed, step, row, gv0, n):
    bits, g = fsl.debug_noise(seed, step, row, gv0, n)
    gpu_bits = bits.cpu().numpy().view(np.uint32)
    ref = oracle.noise_bits_range(seed, step, row, gv0, n)
    assert np.array_equal(gpu_bits, ref)
    ref_g = oracle.gumbel_array(ref)
    assert np.max(np.abs(g.cpu().numpy().astype(np.float64) - ref_g)) <= G_TOL


def test_gumbel_exhaustive_grid():
    k = np.arange(1 << 23, dtype=np.uint64)
    words = (k << np.uint64(9)).astype(np.uint32)
    # also set the ignored low bits on half of the grid
    words[1::2] |= np.uint32(0x1FF)
    bits = torch.from_numpy(words.view(np.int32)).to("cuda")
    g = fsl.debug_gumbel(bits).cpu().numpy().astype(np.float64)
    ref = oracle.gumbel_array(words).astype(np.float64)
    err = np.abs(g - ref)
    worst = int(np.argmax(err))
    print(f"max |g_gpu - g_oracle| = {err[worst]:.3e} at k = {worst}")
    assert np.all(np.isfinite(g))
    assert err[worst] <= G_TOL
    assert np.all(np.diff(g) >= 0)
