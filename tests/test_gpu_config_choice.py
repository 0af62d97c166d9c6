"""Every configuration the library ships is one the automatic choice can take.

The choice depends on the device's CU count (how well a grid fills it), so
this runs on the GPU.  It only queries the choice; nothing is launched.
"""
import itertools

import pytest

from conftest import gpu_available

import lm_head_exact_amd as fsl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

# the last batch makes h too large for the DMA loop's 32-bit buffer offsets
BATCHES = (1, 4, 8, 16, 17, 32, 33, 64, 65, 128, 129, 200, 256, 257, 384, 512, 1 << 18)
DIMS = (256, 264, 512, 1024, 4096, 5120, 8192)
# 70000 and 100000: vocabularies whose tallest DMA blocks leave CUs idle
VOCABS = (1000, 16032, 32000, 40000, 70000, 100000, 128256, 151936)


def test_every_shipped_configuration_is_reachable():
    fsl.force_config(-1)
    reached = set()
    for B, D, V in itertools.product(BATCHES, DIMS, VOCABS):
        reached.add(fsl.selected_config(B, D, V))
        if D % 32 == 0:
            reached.add(fsl.selected_config(B, D, V, packed=True))
    shipped = {fsl.config_name(i) for i in range(fsl.num_configs())}
    missing = shipped - {fsl.config_name(i) for i in reached if i >= 0}
    assert not missing, f"never chosen: {sorted(missing)}"
