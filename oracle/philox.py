"""Philox4x32-10 and the Gaussian sketch (oracle; test infrastructure only).

The GIFT review does not say how the rank-32 factor is computed (the paper's
Algorithm 1 is only named, in the referee report's major comment 2).  This
implementation reads the eigensolve as randomized subspace iteration started
from a seeded Gaussian sketch; the sketch is drawn with a counter-based
generator so that the device and the oracle can each draw it from the same
published definition:

* Philox4x32-10 (Salmon et al., SC'11, section 4): a 4x32-bit counter and a
  2x32-bit key, ten rounds of two 32x32->64 multiplies with the multipliers
  0xD2511F53 and 0xCD9E8D57, the key bumped between rounds by the Weyl
  constants 0x9E3779B9 and 0xBB67AE85.
* Box-Muller: two uniforms u1 in (0, 1], u2 in [0, 1) give
  r = sqrt(-2 ln u1), z0 = r cos(2 pi u2), z1 = r sin(2 pi u2).

Sketch element (i, j) of the d x l matrix, flat index n = i*l + j, is
normal number n of the stream for key (seed lo, seed hi): counter
(n // 4, 0, 0, 0) yields four words w0..w3; (w0, w1) make one Box-Muller
pair and (w2, w3) the next, so the four numbers n = 4c .. 4c+3 come from
counter c as (z0(w0,w1), z1(w0,w1), z0(w2,w3), z1(w2,w3)).  Uniforms:
u1 = (w + 1) * 2^-32, u2 = w * 2^-32.
"""

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """One block: counter = 4 ints, key = 2 ints -> 4 ints (pure Python)."""
    c0, c1, c2, c3 = (int(v) & MASK for v in counter)
    k0, k1 = (int(v) & MASK for v in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + W0) & MASK
            k1 = (k1 + W1) & MASK
        p0 = M0 * c0
        p1 = M1 * c2
        hi0, lo0 = p0 >> 32, p0 & MASK
        hi1, lo1 = p1 >> 32, p1 & MASK
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def philox_blocks(n_blocks, seed):
    """Vectorised Philox over counters (c, 0, 0, 0), c = 0..n_blocks-1.

    Returns a (n_blocks, 4) uint32 array.  Same arithmetic as
    ``philox4x32_10`` on uint64 numpy lanes.
    """
    c0 = np.arange(n_blocks, dtype=np.uint64)
    c1 = np.zeros(n_blocks, dtype=np.uint64)
    c2 = np.zeros(n_blocks, dtype=np.uint64)
    c3 = np.zeros(n_blocks, dtype=np.uint64)
    k0 = np.uint64(seed & MASK)
    k1 = np.uint64((seed >> 32) & MASK)
    m = np.uint64(MASK)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + np.uint64(W0)) & m
            k1 = (k1 + np.uint64(W1)) & m
        p0 = np.uint64(M0) * c0          # < 2^64: exact in uint64
        p1 = np.uint64(M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & m
        hi1, lo1 = p1 >> np.uint64(32), p1 & m
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=1).astype(np.uint32)


def box_muller(w_a, w_b):
    """Two uint32 words -> (z0, z1), fp64."""
    u1 = (w_a.astype(np.float64) + 1.0) * 2.0 ** -32
    u2 = w_b.astype(np.float64) * 2.0 ** -32
    r = np.sqrt(-2.0 * np.log(u1))
    t = 2.0 * np.pi * u2
    return r * np.cos(t), r * np.sin(t)


def gaussian_sketch(d, width, seed):
    """d x width standard-normal sketch (fp64), element n = i*width + j."""
    total = d * width
    n_blocks = (total + 3) // 4
    w = philox_blocks(n_blocks, seed)
    z0, z1 = box_muller(w[:, 0], w[:, 1])
    z2, z3 = box_muller(w[:, 2], w[:, 3])
    flat = np.stack([z0, z1, z2, z3], axis=1).reshape(-1)[:total]
    return flat.reshape(d, width)
