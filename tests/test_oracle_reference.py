"""Pins for the oracle's full-rank and two-sided references.

The symmetric and Cholesky forms are both whitenings of the damped A: for
either W, W W^T = G (A + lam I)^-1 G^T, checked with a linear solve (no
eigendecomposition or Cholesky on the checking side); the two-sided form
factors satisfy their defining equations and left-whitening by the output
side leaves row second-moment eigenvalues w / (w + mu); every transform's
inverse undoes it; the references order as the review's claim says on the
power-law input.
"""

import numpy as np
import pytest

import synth
from oracle import gift as og


@pytest.fixture(scope="module")
def layer():
    w = synth.single_layer()
    inp = synth.draw_input(w.inputs[0], seed=11)
    G = synth.draw_gradient(256, inp["Q"], inp["ev"], seed=12).numpy().astype(np.float64)
    return dict(G=G, A=og.covariance(inp["X"].numpy()))


def test_both_input_forms_whiten(layer):
    G, A = layer["G"], layer["A"]
    d = A.shape[0]
    Ad = A + 1e-3 * np.trace(A) / d * np.eye(d)
    ref = G @ np.linalg.solve(Ad, G.T)
    tr = og.reference_transforms(G, A)
    for name in ("input_full", "input_cholesky"):
        W = og._lr(G, *tr[name][:2])
        assert np.allclose(W @ W.T, ref, rtol=1e-8, atol=1e-9 * np.abs(ref).max()), name


def test_cholesky_factor_is_lower_triangular_and_exact(layer):
    A = layer["A"]
    d = A.shape[0]
    Lt_inv, Lt = og.cholesky_pair(A)
    L = Lt.T
    assert np.all(np.triu(L, 1) == 0)
    assert np.linalg.norm(L @ L.T - (A + 1e-3 * np.trace(A) / d * np.eye(d))) < 1e-12 * np.linalg.norm(A)
    assert np.linalg.norm(Lt_inv @ Lt - np.eye(d)) < 1e-9


def test_two_sided_factors():
    """The output-side pair satisfies its defining equations (matrix products
    only), and left-whitening by it gives the row second moment the
    eigenvalues w / (w + mu) of the damped output factor; the two-sided
    transform is the composition of the two sides."""
    rng = np.random.default_rng(2)
    d_out, d_in = 40, 24
    X = rng.standard_normal((300, d_in)) * np.linspace(3, 0.2, d_in)
    A = X.T @ X / 300
    G = rng.standard_normal((d_out, d_in)) * np.exp(rng.standard_normal((d_out, 1)))
    B = og.output_factor(G)
    assert np.allclose(B, sum(np.outer(G[:, j], G[:, j]) for j in range(d_in)) / d_in)
    mu = 1e-3 * np.trace(B) / d_out
    SB, SBi = og.sym_pair(B)
    Bd = B + mu * np.eye(d_out)
    assert np.linalg.norm(SB @ SB @ Bd - np.eye(d_out)) < 1e-8
    assert np.linalg.norm(SBi @ SBi - Bd) < 1e-10 * np.linalg.norm(Bd)
    M = SB @ G
    wB = np.maximum(np.linalg.eigvalsh(B), 0)
    assert np.allclose(np.sort(np.linalg.eigvalsh(M @ M.T / d_in)), np.sort(wB / (wB + mu)),
                       atol=1e-9)
    S, _ = og.sym_pair(A)
    l, r, _, _ = og.reference_transforms(G, A)["two_sided"]
    assert np.linalg.norm(og._lr(G, l, r) - SB @ G @ S) < 1e-12 * np.linalg.norm(SB @ G @ S)


def test_inverses_undo_the_transforms(layer):
    G, A = layer["G"], layer["A"]
    for name, (l, r, li, ri) in og.reference_transforms(G, A).items():
        back = og._lr(og._lr(G, l, r), li, ri)
        assert np.linalg.norm(back - G) < 1e-9 * np.linalg.norm(G), name


def test_references_order_on_the_power_law_input(layer):
    """Full-rank input-side whitening beats the rank-32 factor, which beats
    Euclid, in the input-side K-FAC metric."""
    G, A = layer["G"], layer["A"]
    Sm = og.metric_sqrt_inv(A, 1e-3 * np.trace(A) / A.shape[0])
    e_eu = og.rel_error_kfac(G, og.euclid_roundtrip(G)[2], Sm)
    tr = og.reference_transforms(G, A)
    e_full = og.rel_error_kfac(G, og.reference_roundtrip(G, tr["input_full"])[3], Sm)
    omega = synth.gaussian_sketch(512, og.SKETCH_WIDTH, seed=13).numpy()
    f = og.refresh_factor(None, omega, A=A)
    e_r32 = og.rel_error_kfac(G, og.gift_roundtrip(G, f)[3], Sm)
    assert e_full < e_r32 < e_eu
    e_ch = og.rel_error_kfac(G, og.reference_roundtrip(G, tr["input_cholesky"])[3], Sm)
    e_two = og.rel_error_kfac(G, og.reference_roundtrip(G, tr["two_sided"])[3], Sm)
    assert e_ch < e_eu and e_two < e_eu
