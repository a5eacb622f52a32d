"""Pins for the oracle's Philox4x32-10 generator and Gaussian sketch."""

import os

import numpy as np

from conftest import GOLDEN
from oracle import philox


def _kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if line:
                w = [int(x, 16) for x in line.split()]
                rows.append((tuple(w[0:4]), tuple(w[4:6]), tuple(w[6:10])))
    return rows


def test_published_known_answers():
    rows = _kat()
    assert len(rows) == 3
    for ctr, key, out in rows:
        assert philox.philox4x32_10(ctr, key) == out


def test_vectorised_blocks_match_scalar():
    seed = 0x1234_5678_9ABC_DEF1
    blocks = philox.philox_blocks(257, seed)
    for c in (0, 1, 2, 100, 256):
        ref = philox.philox4x32_10((c, 0, 0, 0), (seed & 0xFFFFFFFF, seed >> 32))
        assert tuple(int(v) for v in blocks[c]) == ref


def test_sketch_layout_and_box_muller():
    d, l, seed = 5, 7, 42
    om = philox.gaussian_sketch(d, l, seed)
    assert om.shape == (d, l)
    for i in range(d):
        for j in range(l):
            n = i * l + j
            w = philox.philox4x32_10((n // 4, 0, 0, 0), (seed, 0))
            pair = (w[0], w[1]) if (n % 4) < 2 else (w[2], w[3])
            u1 = (pair[0] + 1.0) * 2.0 ** -32
            u2 = pair[1] * 2.0 ** -32
            r = np.sqrt(-2.0 * np.log(u1))
            z = r * np.cos(2 * np.pi * u2) if n % 2 == 0 else r * np.sin(2 * np.pi * u2)
            assert om[i, j] == z


def test_sketch_moments():
    z = philox.gaussian_sketch(1024, 256, 3).ravel()
    n = z.size
    assert abs(z.mean()) < 5 / np.sqrt(n)
    assert abs(z.var() - 1) < 5 * np.sqrt(2 / n)
    kurt = np.mean(z ** 4)
    assert abs(kurt - 3) < 5 * np.sqrt(96 / n)
    # different seeds differ, same seed repeats
    assert np.array_equal(philox.gaussian_sketch(16, 8, 9), philox.gaussian_sketch(16, 8, 9))
    assert not np.array_equal(philox.gaussian_sketch(16, 8, 9), philox.gaussian_sketch(16, 8, 10))
