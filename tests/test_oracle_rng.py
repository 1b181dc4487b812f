"""Pins of the oracle's probe generator (Philox4x32-10 and the packed sign planes).

Independent anchors: the published Philox4x32-10 known-answer vectors, and statistical
properties every Rademacher stream must have ("Stanford's 1.5-SPSA Trains OPT-30B Without
Backpropagation", section "How 1.5-SPSA Works": probe entries are independent +/-1).
"""
import numpy as np
import pytest
from scipy import stats

import oracle
from conftest import read_golden


def test_philox_known_answers():
    rows = read_golden("philox4x32_10_kat.txt")
    assert len(rows) == 3
    for r in rows:
        v = [int(x, 16) for x in r]
        out = oracle.philox4x32_10(v[0:4], v[4:6])
        assert [int(x) for x in out] == v[6:10]


def test_plane_byte_order_from_known_answer():
    # seed 0, step 0, probe 0, block 0 is Philox of the all-zero counter and key: the
    # first known-answer vector.  Its words stored little-endian are the plane's bytes.
    rows = read_golden("philox4x32_10_kat.txt")
    words = [int(x, 16) for x in rows[0][6:10]]
    expect = b"".join(w.to_bytes(4, "little") for w in words)
    plane = oracle.gen_plane(0, 0, 0, 0, 128)
    assert plane.tobytes() == expect
    # bit j of the block <-> param j, bit 1 <-> +1
    for j in range(128):
        bit = (words[j // 32] >> (j % 32)) & 1
        assert oracle.sign(0, 0, 0, j) == (1 if bit else -1)


def test_plane_field_layout():
    # The documented layout: counter = (blk_lo, blk_hi, probe, step), key = seed.
    seed, step, probe = 0x0123456789ABCDEF, 7, 11
    for blk in (0, 5, (1 << 32) + 3):
        ref = oracle.philox4x32_10([blk & 0xFFFFFFFF, blk >> 32, probe, step],
                                   [seed & 0xFFFFFFFF, seed >> 32])
        plane = oracle.gen_plane(seed, step, probe, blk * 128, 128)
        assert plane.view("<u4").tolist() == [int(x) for x in ref]


def test_plane_offset_and_tail():
    seed, step, probe = 3, 1, 2
    full = oracle.gen_plane(seed, step, probe, 0, 128 * 9)
    part = oracle.gen_plane(seed, step, probe, 128 * 4, 300)   # 3 blocks, ragged tail
    assert part.size == 48
    assert np.array_equal(part, full[64:112])
    # per-element signs agree with the packed plane
    z = oracle.signs_from_plane(part, 300)
    for e in (0, 1, 127, 128, 255, 299):
        assert z[e] == oracle.sign(seed, step, probe, 128 * 4 + e)


def test_sign_statistics():
    n = 1 << 20
    planes = oracle.gen_planes(0, 0, 0, 4, 0, n)
    z = np.stack([oracle.signs_from_plane(p, n) for p in planes])
    # values in {-1, +1}, mean ~ 0
    assert set(np.unique(z)) == {-1.0, 1.0}
    assert abs(z[0].mean()) <= 5.0 / np.sqrt(n)
    # every bit position inside a byte is balanced
    bits = np.unpackbits(planes[0], bitorder="little").reshape(-1, 8)
    for b in range(8):
        assert abs(bits[:, b].mean() - 0.5) <= 2.5 / np.sqrt(bits.shape[0])
    # bytes uniform over 256 values (chi-square, 255 dof)
    counts = np.bincount(planes[0], minlength=256)
    chi2 = ((counts - counts.mean()) ** 2 / counts.mean()).sum()
    p = stats.chi2.sf(chi2, 255)
    assert 1e-4 < p < 1 - 1e-4
    # probes are uncorrelated
    for a, b in ((0, 1), (1, 2), (0, 3)):
        assert abs((z[a] * z[b]).mean()) <= 5.0 / np.sqrt(n)


def test_streams_are_distinct():
    n = 4096
    base = oracle.gen_plane(0, 0, 0, 0, n)
    for other in (oracle.gen_plane(1, 0, 0, 0, n), oracle.gen_plane(0, 1, 0, 0, n),
                  oracle.gen_plane(0, 0, 1, 0, n), oracle.gen_plane(1 << 32, 0, 0, 0, n)):
        za = oracle.signs_from_plane(base, n)
        zb = oracle.signs_from_plane(other, n)
        assert abs((za * zb).mean()) <= 5.0 / np.sqrt(n)
