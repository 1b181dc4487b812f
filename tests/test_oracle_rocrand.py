"""The oracle's Philox4x32-10 and packed planes against rocRAND's open-source Philox engine
(Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11, section 4), an
implementation written independently of this repository.  Counters cover the high words
(block index above 2^32, large probe and step) and 64-bit seeds."""
import numpy as np
import pytest

import oracle
import rocrand_ref

pytestmark = pytest.mark.skipif(not rocrand_ref.available(),
                                reason="rocRAND header not installed")

CASES = [
    (0, 0, 0, 0),
    (0x243F6A8885A308D3, 7, 159, 12345),
    (0xFFFFFFFFFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, (1 << 40) + 3),
    (42, 3, 17, (1 << 32) - 2),          # crosses the low-word boundary of the block index
]


@pytest.mark.parametrize("seed,step,probe,blk0", CASES)
def test_words_match_rocrand(seed, step, probe, blk0):
    ref = rocrand_ref.philox_words(seed, step, probe, blk0, 64)
    k = (seed & 0xFFFFFFFF, seed >> 32)
    for i in range(64):
        b = blk0 + i
        got = oracle.philox4x32_10((b & 0xFFFFFFFF, (b >> 32) & 0xFFFFFFFF, probe, step), k)
        assert tuple(int(x) for x in ref[i]) == tuple(int(x) for x in got), (seed, step, probe, b)


@pytest.mark.parametrize("n", [1, 127, 128, 4096, 100_003])
def test_planes_match_rocrand(n):
    for seed, step, probe, offset in [(0, 0, 0, 0), (99, 4, 31, 128 * 977),
                                      (2**63 + 5, 2**31, 511, 128 * ((1 << 33) + 1))]:
        ref = rocrand_ref.plane(seed, step, probe, offset, n)
        got = oracle.gen_plane(seed, step, probe, offset, n)
        assert np.array_equal(ref, got), (seed, step, probe, offset, n)
