"""Pins for the oracle's block-diagonal factor (block-A-b).

Each check ties the oracle to something other than its own eigh call: the
defining equations of the inverse square root and square root (matrix
products only), the closed-form square root of a 2 x 2 SPD matrix, the
reduction to full-rank whitening when the blocks cover all of A or A is
block-diagonal, isotropy, and the bit-exact equality with the Euclidean
round trip for an isotropic factor with a power-of-two scale.
"""

import numpy as np
import pytest

import synth
from oracle import gift as og


@pytest.fixture(scope="module")
def layer():
    w = synth.single_layer()
    inp = synth.draw_input(w.inputs[0], seed=11)
    G = synth.draw_gradient(256, inp["Q"], inp["ev"], seed=12).numpy()
    return dict(G=G, A=og.covariance(inp["X"].numpy()))


@pytest.mark.parametrize("b", [32, 64])
def test_defining_equations(layer, b):
    A = layer["A"]
    bf = og.block_factor(A, b)
    lam = 1e-3 * np.trace(A) / A.shape[0]
    assert abs(bf.lambda_iso - lam) <= 1e-15 * lam
    for i in range(A.shape[0] // b):
        sl = slice(i * b, (i + 1) * b)
        M = A[sl, sl] + lam * np.eye(b)
        S, Si = bf.S[sl], bf.S_inv[sl]
        assert np.allclose(S, S.T, atol=1e-12 * np.abs(S).max())
        assert np.linalg.norm(S @ S @ M - np.eye(b)) < 1e-8
        assert np.linalg.norm(Si @ Si - M) < 1e-10 * np.linalg.norm(M)
        assert np.linalg.norm(S @ Si - np.eye(b)) < 1e-9
        assert np.all(np.diff(bf.theta[sl]) <= 0)
        assert abs(bf.theta[sl].sum() - np.trace(A[sl, sl])) < 1e-10 * np.trace(A[sl, sl])


def test_two_by_two_closed_form():
    """b = 2: the square root of an SPD 2 x 2 matrix M is
    (M + sqrt(det M) I) / sqrt(tr M + 2 sqrt(det M))."""
    rng = np.random.default_rng(4)
    X = rng.standard_normal((50, 6))
    A = X.T @ X / 50
    bf = og.block_factor(A, 2)
    lam = 1e-3 * np.trace(A) / 6
    for i in range(3):
        M = A[2 * i:2 * i + 2, 2 * i:2 * i + 2] + lam * np.eye(2)
        sd = np.sqrt(np.linalg.det(M))
        R = (M + sd * np.eye(2)) / np.sqrt(np.trace(M) + 2 * sd)
        assert np.allclose(bf.S_inv[2 * i:2 * i + 2], R, rtol=1e-12, atol=0)
        Rinv = np.array([[R[1, 1], -R[0, 1]], [-R[1, 0], R[0, 0]]]) / np.linalg.det(R)
        assert np.allclose(bf.S[2 * i:2 * i + 2], Rinv, rtol=1e-11, atol=0)


def test_whole_matrix_block_is_full_rank_whitening(layer):
    """b = d_in: block-A is exact full-rank damped whitening: W W^T-free check
    through the defining equation (W (A + lam I) W^T = G G^T for the rows)."""
    A, G = layer["A"], layer["G"].astype(np.float64)
    d = A.shape[0]
    bf = og.block_factor(A, d)
    lam = 1e-3 * np.trace(A) / d
    W = og.block_whiten(G, bf)
    assert np.allclose(W @ (A + lam * np.eye(d)) @ W.T, G @ G.T, rtol=1e-8,
                       atol=1e-9 * np.abs(G @ G.T).max())
    assert np.linalg.norm(og.block_unwhiten(W, bf) - G) < 1e-10 * np.linalg.norm(G)


def test_block_diagonal_matrix_gives_the_full_factor():
    """A exactly block-diagonal in 32-blocks: block-A-32 = block-A-64 = full."""
    rng = np.random.default_rng(7)
    d = 128
    A = np.zeros((d, d))
    for i in range(d // 32):
        X = rng.standard_normal((200, 32)) * rng.uniform(0.1, 3.0, 32)
        A[32 * i:32 * i + 32, 32 * i:32 * i + 32] = X.T @ X / 200
    G = rng.standard_normal((10, d))
    full = og.block_whiten(G, og.block_factor(A, d))
    for b in (32, 64):
        assert np.linalg.norm(og.block_whiten(G, og.block_factor(A, b)) - full) \
            < 1e-10 * np.linalg.norm(full)


def test_isotropic_block_factor_equals_euclid_bit_exactly(layer):
    """A = c I with c + lambda = 4^-3: S = 8 I, so the block-A codes are the
    Euclidean codes of 8 G, and G^ is identical."""
    d = 512
    c = 4.0 ** -3 / (1 + 1e-3)   # lambda = 1e-3 c, so c + lambda = 4^-3
    bf = og.block_factor(c * np.eye(d), 32)
    assert np.allclose(bf.S[:32], 8 * np.eye(32), rtol=1e-12)
    bf.S[:] = np.tile(8 * np.eye(32), (d // 32, 1))
    bf.S_inv[:] = np.tile(np.eye(32) / 8, (d // 32, 1))
    G = layer["G"]
    for blk in (False, True):
        codes, inv, _, gh, _ = og.block_roundtrip(G, bf, blk)
        ce, ie, ge, _ = og.euclid_roundtrip(G, blk)
        assert np.array_equal(codes, ce)
        assert np.array_equal(gh.astype(np.float32), ge)


@pytest.mark.parametrize("b", [32, 64])
def test_unwhiten_inverts_whiten(layer, b):
    bf = og.block_factor(layer["A"], b)
    G = layer["G"]
    assert np.linalg.norm(og.block_unwhiten(og.block_whiten(G, bf), bf) - G) \
        < 1e-11 * np.linalg.norm(G)


def test_full_rank_block_is_the_best_whitening(layer):
    """One block covering all of A (exact damped whitening) has a smaller
    error in the K-FAC metric than the rank-32 factor, which beats Euclid;
    with a randomly rotated eigenbasis the 32- and 64-blocks hold little of
    A's anisotropy and stay near Euclid (within 10%)."""
    A, G = layer["A"], layer["G"]
    S = og.metric_sqrt_inv(A, 1e-3 * np.trace(A) / A.shape[0])
    e_eu = og.rel_error_kfac(G, og.euclid_roundtrip(G)[2], S)
    e_full = og.rel_error_kfac(G, og.block_roundtrip(G, og.block_factor(A, 512))[3], S)
    omega = synth.gaussian_sketch(512, og.SKETCH_WIDTH, seed=13).numpy()
    f = og.refresh_factor(None, omega, A=A)
    e_r32 = og.rel_error_kfac(G, og.gift_roundtrip(G, f)[3], S)
    assert e_full < e_r32 < e_eu
    for b in (32, 64):
        e = og.rel_error_kfac(G, og.block_roundtrip(G, og.block_factor(A, b))[3], S)
        assert abs(e / e_eu - 1) < 0.1
