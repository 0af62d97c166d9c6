"""GPU noise field against the oracle: raw Philox words bit-exact; Gumbel
values on every one of the top 2^24 and bottom 2^20 words (the tail, where a
large vocabulary's winners draw their noise) and on a stratified grid of
2^24 words over the rest (one word per cell of 256)."""
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


WORD_SETS = {
    "top_2^24": ((1 << 32) - (1 << 24) + np.arange(1 << 24, dtype=np.uint64)).astype(np.uint32),
    "bottom_2^20": np.arange(1 << 20, dtype=np.uint32),
    "stratified": (np.arange(1 << 24, dtype=np.uint64) * np.uint64(256)
                   + np.uint64(97)).astype(np.uint32),
}


@pytest.mark.parametrize("name", list(WORD_SETS))
def test_gumbel_against_oracle(name):
    words = WORD_SETS[name]
    print(f"gumbel map on {name}: {words.size} words", flush=True)
    bits = torch.from_numpy(words.view(np.int32)).to("cuda")
    g = fsl.debug_gumbel(bits).cpu().numpy().astype(np.float64)
    ref = oracle.gumbel_array(words).astype(np.float64)
    err = np.abs(g - ref)
    worst = int(np.argmax(err))
    print(f"max |g_gpu - g_oracle| = {err[worst]:.3e} at x = {int(words[worst])}")
    assert np.all(np.isfinite(g))
    assert err[worst] <= G_TOL
    if name == "top_2^24":
        # the series branch: non-decreasing in the word, as the exact map is
        assert np.all(np.diff(g) >= 0)
