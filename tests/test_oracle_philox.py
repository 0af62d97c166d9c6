"""Pins of the oracle's counter-based generator (CPU only).

The FlashSampling pages say each element of a tile receives its own Gumbel
draw from the tile's RNG state (wiki summary, "Method") but do not name the
generator; this build uses Philox-4x32-10 (Salmon et al., SC'11), which the
oracle implements from that paper.  The pin is the published known-answer
list (tests/golden/philox4x32_10_kat.txt), which an implementation with a
wrong multiplier, Weyl constant, word permutation or key schedule cannot
reproduce.
"""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        w = [int(x, 16) for x in line.split()]
        assert len(w) == 10
        rows.append((w[0:4], w[4:6], w[6:10]))
    assert len(rows) == 3
    return rows


@pytest.mark.parametrize("ctr,key,expect", _kat())
def test_philox_known_answers(orc, ctr, key, expect):
    assert orc.philox4x32_10(ctr, key) == expect


def test_noise_word_layout(orc):
    """Element gv takes word gv mod 4 of the block at counter gv / 4: four
    consecutive ids share one block, and the block is keyed as documented."""
    seed, step, row = 0x0123456789ABCDEF, 0xFEDCBA9876543210, 77
    for gv in (0, 1, 2, 3, 4, 1001, 48096, 128255, 2**31 - 2):
        blk = orc.philox4x32_10([gv >> 2, row, step & 0xFFFFFFFF, step >> 32],
                                [seed & 0xFFFFFFFF, seed >> 32])
        assert orc.noise_bits(seed, step, row, gv) == blk[gv & 3]
    bulk = orc.noise_bits_range(seed, step, row, 48096, 4000)
    one = np.array([orc.noise_bits(seed, step, row, 48096 + i) for i in range(4000)],
                   np.uint32)
    assert np.array_equal(bulk, one)


def test_noise_depends_on_every_key_part(orc):
    base = orc.noise_bits_range(5, 9, 3, 0, 4096)
    for args in ((6, 9, 3), (5, 10, 3), (5, 9, 4), (5 + (1 << 32), 9, 3), (5, 9 + (1 << 32), 3)):
        other = orc.noise_bits_range(*args, 0, 4096)
        assert np.mean(base == other) < 0.01


def test_noise_bit_frequencies(orc):
    """Every output bit is 1 with frequency 1/2 (4-sigma band) and
    successive words are uncorrelated."""
    n = 1 << 20
    x = orc.noise_bits_range(123, 0, 0, 0, n)
    bits = ((x[:, None] >> np.arange(32, dtype=np.uint32)) & 1).astype(np.float64)
    freq = bits.mean(axis=0)
    assert np.all(np.abs(freq - 0.5) < 4 * 0.5 / np.sqrt(n))
    u = x.astype(np.float64)
    u = (u - u.mean()) / u.std()
    corr = np.mean(u[:-1] * u[1:])
    assert abs(corr) < 5 / np.sqrt(n)
