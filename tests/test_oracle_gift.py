"""Pins for the oracle's factor refresh, whitening, quantization and metrics.

Each check ties the oracle to something other than itself: brute force,
a dense eigendecomposition of the matrix the formula claims to represent,
closed forms (isotropy, identity, scale invariance), the FP8 error bound.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import e4m3
from oracle import gift as og


@pytest.fixture(scope="module")
def layer():
    """The single-layer workload: d_in 512, d_out 256, 4096 fp32 tokens."""
    w = synth.single_layer()
    inp = synth.draw_input(w.inputs[0], seed=11)
    G = synth.draw_gradient(256, inp["Q"], inp["ev"], seed=12).numpy()
    X = inp["X"].numpy()
    omega = synth.gaussian_sketch(512, og.SKETCH_WIDTH, seed=13).numpy()
    A = og.covariance(X)
    return dict(X=X, G=G, A=A, omega=omega, f=og.refresh_factor(X, omega, A=A))


# ---------------------------------------------------------------- covariance

def test_covariance_brute_force():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((7, 5)).astype(np.float32)
    A = og.covariance(X)
    for i in range(5):
        for j in range(5):
            s = 0.0
            for n in range(7):
                s += float(X[n, i]) * float(X[n, j])
            assert abs(A[i, j] - s / 7) < 1e-14
    t, lf = og.trace_floor(A, 1e-3)
    assert abs(t - sum(A[i, i] for i in range(5))) < 1e-14
    assert abs(lf - 1e-3 * t / 5) < 1e-18


# ---------------------------------------------------------------- eigensolve

def test_subspace_iteration_exact_low_rank():
    """A of exact rank 20 < 32: subspace iteration + Rayleigh-Ritz recovers its
    eigenvalues and eigenprojector to rounding."""
    rng = np.random.default_rng(1)
    d, k = 128, 20
    V, _ = np.linalg.qr(rng.standard_normal((d, k)))
    ev = np.linspace(5.0, 0.5, k)
    A = (V * ev) @ V.T
    omega = rng.standard_normal((d, og.SKETCH_WIDTH))
    Q = og.subspace_iteration(A, omega)
    theta, U = og.rayleigh_ritz(A, Q, og.RANK)
    assert np.allclose(theta[:k], ev, rtol=1e-10, atol=0)
    assert np.all(np.abs(theta[k:]) < 1e-12)
    P = U[:, :k] @ U[:, :k].T
    assert np.linalg.norm(P - V @ V.T) < 1e-10
    assert np.linalg.norm(U.T @ U - np.eye(og.RANK)) < 1e-12


def test_subspace_iteration_matches_eigh_on_power_law(layer):
    A, f = layer["A"], layer["f"]
    w, V = np.linalg.eigh(A)
    w, V = w[::-1], V[:, ::-1]
    r = og.RANK
    assert np.allclose(f.theta, w[:r], rtol=1e-4, atol=0)
    # principal cosines between span(U) and the top-r eigenvectors
    cos = np.linalg.svd(V[:, :r].T @ f.U, compute_uv=False)
    assert cos.min() > 0.999
    # Eckart-Young: the rank-r part is (near) the best rank-r approximation
    best = np.sqrt(np.sum(w[r:] ** 2))
    got = np.linalg.norm(A - (f.U * f.theta) @ f.U.T)
    assert got <= best * (1 + 1e-3)
    # tail variance = mean of the discarded eigenvalues
    assert abs(f.sigma2_tail - np.mean(w[r:])) < 1e-4 * np.mean(w[r:])
    assert abs(f.trace - np.sum(w)) < 1e-10 * np.sum(w)


@pytest.mark.parametrize("r", [8, 16])
def test_lower_rank_factor_matches_eigh(layer, r):
    """rank r < 32 (the rank sweep): the top r Ritz pairs of the same subspace
    are the top r eigenpairs of A, the tail variance is the mean of the d - r
    discarded eigenvalues, and the rank-r part is (near) the best rank-r
    approximation (Eckart-Young)."""
    A = layer["A"]
    f = og.refresh_factor(layer["X"], layer["omega"], rank=r, A=A)
    w, V = np.linalg.eigh(A)
    w, V = w[::-1], V[:, ::-1]
    assert f.U.shape == (512, r) and f.theta.shape == (r,)
    assert np.allclose(f.theta, w[:r], rtol=1e-6, atol=0)
    assert np.linalg.svd(V[:, :r].T @ f.U, compute_uv=False).min() > 0.9999
    assert abs(f.sigma2_tail - np.mean(w[r:])) < 1e-6 * np.mean(w[r:])
    assert abs(f.lambda_iso - (1e-3 * np.sum(w) / 512 + np.mean(w[r:]))) < 1e-6 * f.lambda_iso
    best = np.sqrt(np.sum(w[r:] ** 2))
    assert np.linalg.norm(A - (f.U * f.theta) @ f.U.T) <= best * (1 + 1e-4)
    # the rank-32 factor's top r pairs are the rank-r factor's
    f32 = layer["f"]
    assert np.allclose(f32.theta[:r], f.theta, rtol=1e-12, atol=0)


def test_damping_readings():
    theta = np.array([4.0, 2.0])
    lam, lf, tail = og.damping(10.0, theta, 6, 1e-3, og.DAMPING_FLOOR_PLUS_TAIL)
    assert lf == 1e-3 * 10 / 6 and tail == (10 - 6) / 4 and lam == lf + tail
    lam1, lf1, _ = og.damping(10.0, theta, 6, 1e-3, og.DAMPING_FLOOR)
    assert lam1 == lf1
    # all-zero input: damping is held at its floor, coefficients stay finite
    lam0, _, _ = og.damping(0.0, np.zeros(2), 6, 1e-3, og.DAMPING_FLOOR_PLUS_TAIL)
    assert lam0 == og.LAMBDA_MIN
    assert all(np.all(np.isfinite(c)) for c in og.coefficients(np.zeros(2), lam0))


# ---------------------------------------------------------------- whitening

def _dense_power(M, p):
    w, V = np.linalg.eigh(M)
    return (V * w ** p) @ V.T


def test_coefficients_match_dense_matrix_functions(layer):
    f = layer["f"]
    Ar = f.dense()
    inv_sqrt = f.alpha * np.eye(f.d_in) + (f.U * f.d_w) @ f.U.T
    sqrt = f.beta * np.eye(f.d_in) + (f.U * f.d_u) @ f.U.T
    ref_is = _dense_power(Ar, -0.5)
    ref_s = _dense_power(Ar, 0.5)
    assert np.linalg.norm(inv_sqrt - ref_is) < 1e-9 * np.linalg.norm(ref_is)
    assert np.linalg.norm(sqrt - ref_s) < 1e-9 * np.linalg.norm(ref_s)
    assert np.linalg.norm(sqrt @ inv_sqrt - np.eye(f.d_in)) < 1e-9


def test_whiten_isotropy_closed_form(layer):
    """G = Z A_r^{1/2}  =>  whiten(G) = Z."""
    f = layer["f"]
    Z = np.random.default_rng(3).standard_normal((64, f.d_in))
    G = Z @ _dense_power(f.dense(), 0.5)
    W = og.whiten(G, f)
    assert np.linalg.norm(W - Z) < 1e-10 * np.linalg.norm(Z)


def test_whiten_full_rank_gives_identity_covariance():
    """With every eigenpair kept, whitened rows of G = Z A^{1/2} have the
    sample covariance of Z (the identity, up to sampling)."""
    rng = np.random.default_rng(4)
    d = 48
    M = rng.standard_normal((d, d))
    A = M @ M.T / d + 0.1 * np.eye(d)
    w, V = np.linalg.eigh(A)
    lam = 1e-6
    f = og.factor_from_parts(V[:, ::-1], w[::-1] - lam, lam)
    Z = rng.standard_normal((4000, d))
    G = Z @ _dense_power(A, 0.5)
    W = og.whiten(G, f)
    assert np.linalg.norm(W - Z) < 1e-8 * np.linalg.norm(Z)


def test_unwhiten_inverts_whiten(layer):
    f, G = layer["f"], layer["G"]
    back = og.unwhiten(og.whiten(G, f), f)
    assert np.linalg.norm(back - G) < 1e-12 * np.linalg.norm(G)


def test_isotropic_factor_equals_euclid_bit_exactly(layer):
    """Theta = 0 and lambda_iso = 4^-3: whitening is multiplication by 2^3, so
    GIFT codes equal Euclidean codes and G^ is identical."""
    G = layer["G"]
    d = G.shape[1]
    U = np.linalg.qr(np.random.default_rng(5).standard_normal((d, og.RANK)))[0]
    f = og.factor_from_parts(U, np.zeros(og.RANK), 4.0 ** -3)
    assert f.alpha == 8.0 and np.all(f.d_w == 0) and np.all(f.d_u == 0)
    codes, inv, W32, Gh, flags = og.gift_roundtrip(G, f)
    ce, inve, Ghe, fle = og.euclid_roundtrip(G)
    assert np.array_equal(codes, ce)
    assert inv == np.float32(8.0) * inve
    assert np.array_equal(Gh.astype(np.float32), Ghe)


# ---------------------------------------------------------------- quantization

def test_power_of_two_scaling_commutes(layer):
    G = layer["G"].astype(np.float32)
    c0, i0, g0, _ = og.euclid_roundtrip(G)
    for k in (-20, -3, 5, 30):
        ck, ik, gk, _ = og.euclid_roundtrip(G * np.float32(2.0 ** k))
        assert np.array_equal(ck, c0)
        assert ik == i0 * np.float32(2.0 ** k)
        assert np.array_equal(gk, g0 * np.float32(2.0 ** k))


def test_amax_element_gets_the_max_code(layer):
    G = layer["G"].astype(np.float32)
    codes, inv, _ = og.quantize_tensor(G)
    i = np.argmax(np.abs(G))
    assert codes.ravel()[i] & 0x7F == 0x7E
    assert np.all(codes & 0x7F <= 0x7E)
    assert inv == np.float32(np.abs(G).max()) / np.float32(448)


def test_constant_tensor_reconstructs_exactly():
    w = np.full((3, 5), 3.5, dtype=np.float32)
    w[1] = -3.5
    codes, inv, _ = og.quantize_tensor(w)
    assert np.all(codes[0] == 0x7E) and np.all(codes[1] == 0xFE)
    assert np.array_equal(og.dequantize_tensor(codes, inv), w)


def test_fp8_error_bound(layer):
    """|w^ - w| <= (2^-4 |y| + 2^-10) * inv per element (RNE half-step in the
    normal / subnormal range), plus fp32 rounding of the two products."""
    W = og.whiten(layer["G"], layer["f"]).astype(np.float32)
    codes, inv, _ = og.quantize_tensor(W)
    What = og.dequantize_tensor(codes, inv)
    y = np.abs(W.astype(np.float64)) / float(inv)
    bound = (2.0 ** -4 * y + 2.0 ** -10) * float(inv) * (1 + 1e-6) + 4 * 2.0 ** -24 * np.abs(W)
    assert np.all(np.abs(What.astype(np.float64) - W) <= bound)


def test_zero_and_nonfinite_tensors():
    z = np.zeros((4, 8), dtype=np.float32)
    z[0, 0] = -0.0
    codes, inv, flags = og.quantize_tensor(z)
    assert inv == 1.0 and flags == og.FLAG_ZERO_AMAX
    assert codes[0, 0] == 0x80 and np.all(codes.ravel()[1:] == 0)
    x = np.ones((4, 8), dtype=np.float32)
    x[2, 3] = np.nan
    codes, inv, flags = og.quantize_tensor(x)
    assert flags & og.FLAG_NONFINITE and np.isnan(inv)
    x[2, 3] = np.inf
    codes, inv, flags = og.quantize_tensor(x)
    assert flags & og.FLAG_NONFINITE and np.isinf(inv)
    assert codes[2, 3] == 0x7F and np.all(codes[0] == 0)  # inf*0 = NaN; 1*0 = 0


def test_block128_is_per_segment_tensor_quantization(layer):
    G = layer["G"][:8].astype(np.float32)
    codes, inv, _ = og.quantize_block128(G)
    assert inv.shape == (8, G.shape[1] // 128)
    for i in range(8):
        for b in range(G.shape[1] // 128):
            seg = G[i, 128 * b:128 * (b + 1)]
            c, s, _ = og.quantize_tensor(seg)
            assert np.array_equal(codes[i, 128 * b:128 * (b + 1)], c) and inv[i, b] == s
            assert np.max(codes[i, 128 * b:128 * (b + 1)] & 0x7F) == 0x7E
    with pytest.raises(ValueError):
        og.quantize_block128(np.ones((2, 100), dtype=np.float32))


# ---------------------------------------------------------------- metrics

def test_metrics_closed_forms(layer):
    G = layer["G"].astype(np.float64)
    assert og.rel_frobenius(G, G) == 0.0
    assert abs(og.rel_frobenius(G, 1.01 * G) - 0.01) < 1e-12
    S = og.metric_sqrt_inv(np.eye(G.shape[1]), 0.0)
    Gh = G + np.random.default_rng(6).standard_normal(G.shape) * 1e-2
    assert abs(og.rel_error_kfac(G, Gh, S) - og.rel_frobenius(G, Gh)) < 1e-12
    e, g = og.error_sums(G, Gh)
    assert abs(e - np.sum((Gh - G) ** 2)) < 1e-9 * e


def test_gift_beats_euclid_in_the_kfac_metric(layer):
    """Regression on the generator: the floor+tail factor cuts the K-FAC
    metric error well below Euclidean FP8 and keeps the plain error near it;
    the floor-only reading does not keep the plain error near it."""
    G, A, f = layer["G"], layer["A"], layer["f"]
    S = og.metric_sqrt_inv(A, og.trace_floor(A)[1])
    Gh = og.gift_roundtrip(G, f)[3]
    Ghe = og.euclid_roundtrip(G)[2]
    assert og.rel_error_kfac(G, Gh, S) < 0.5 * og.rel_error_kfac(G, Ghe, S)
    assert og.rel_frobenius(G, Gh) < 1.2 * og.rel_frobenius(G, Ghe)
    f1 = og.refresh_factor(layer["X"], layer["omega"], mode=og.DAMPING_FLOOR, A=A)
    assert og.rel_frobenius(G, og.gift_roundtrip(G, f1)[3]) > 3 * og.rel_frobenius(G, Ghe)


def test_torch_cast_agrees_with_oracle_on_whitened_tensor(layer):
    """Independent cross-check of encode on a real whitened tensor."""
    W = og.whiten(layer["G"], layer["f"]).astype(np.float32)
    codes, inv, _ = og.quantize_tensor(W)
    scale = np.float32(448) / og.amax(W)
    y = (W * scale).astype(np.float32)
    assert np.abs(y).max() < 464
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    assert np.array_equal(e4m3.encode(y), ref)


# --------------------------------------------------------------------------- reduction

def test_reduce_payloads_adds_in_fp32_in_order():
    """Decoded values 2^24, 1, -2^24 (E4M3 code 0x38 = 1.0 with inverse
    scales 2^24, 1, and code 0xB8 = -1.0 with 2^24): fp32 additions in rank
    order give fl32(fl32(2^24 + 1) - 2^24) = 0, not the exact sum 1."""
    one, mone = np.full((1, 4), 0x38, np.uint8), np.full((1, 4), 0xB8, np.uint8)
    p = [("tensor", one, np.float32(2.0 ** 24)), ("tensor", one, np.float32(1.0)),
         ("tensor", mone, np.float32(2.0 ** 24))]
    assert np.all(og.reduce_payloads(p) == 0.0)
    # another order keeps the 1
    assert np.all(og.reduce_payloads([p[0], p[2], p[1]]) == 1.0)
    # one payload is its dequantization
    codes, inv, _ = og.quantize_tensor(np.linspace(-3, 3, 64, dtype=np.float32).reshape(2, 32))
    assert np.array_equal(og.reduce_payloads([("tensor", codes, inv)]),
                          og.dequantize_tensor(codes, inv))


def test_unwhitened_sum_of_whitened_gradients_is_the_sum_of_gradients():
    """Linearity that the reduction relies on: sum_r W_r A^{1/2} = sum_r G_r
    when W_r = G_r A^{-1/2} with one shared factor (fp64, no quantization)."""
    rng = np.random.default_rng(3)
    X = rng.standard_normal((512, 96))
    omega = rng.standard_normal((96, og.SKETCH_WIDTH))
    f = og.refresh_factor(X, omega)
    Gs = [rng.standard_normal((7, 96)) for _ in range(4)]
    S = sum(og.whiten(G, f) for G in Gs)
    assert np.allclose(og.unwhiten(S, f), sum(Gs), rtol=1e-10, atol=1e-10)


# --------------------------------------------------------------------------- pins added for
# the block-scaled dequantization, the K-FAC metric and the tiny-amax scale

def test_dequantize_block128_uses_each_segments_own_scale():
    """Hand-built codes: row i, segment b holds code 0x38 (1.0) except one
    0x3C (1.5) at column 5 of the segment; the inverse scales are distinct
    powers of two per (row, segment), so a segment-to-scale mix-up (tiling
    the scales along the row instead of repeating them, or transposing them)
    changes the result."""
    d_out, nseg = 3, 4
    codes = np.full((d_out, nseg * 128), 0x38, dtype=np.uint8)
    inv = np.empty((d_out, nseg), dtype=np.float32)
    for i in range(d_out):
        for b in range(nseg):
            codes[i, 128 * b + 5] = 0x3C
            inv[i, b] = np.float32(2.0 ** (4 * i + b - 6))
    W = og.dequantize_block128(codes, inv)
    assert W.dtype == np.float32 and W.shape == codes.shape
    for i in range(d_out):
        for b in range(nseg):
            s = 2.0 ** (4 * i + b - 6)
            seg = W[i, 128 * b:128 * (b + 1)]
            assert seg[5] == 1.5 * s
            assert np.all(np.delete(seg, 5) == s)
    # round trip of per-segment quantization: every segment's largest element
    # comes back as +-448 times its own segment's inverse scale, within one
    # ulp of the element (segments differ in scale by up to 1e5)
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((2, 256)) * np.array([[1.0], [1e3]])).astype(np.float32)
    w[:, 128:] *= np.float32(1e-2)
    c, s, _ = og.quantize_block128(w)
    back = og.dequantize_block128(c, s)
    for i in range(2):
        for b in range(2):
            seg = w[i, 128 * b:128 * (b + 1)]
            k = np.argmax(np.abs(seg))
            assert back[i, 128 * b + k] == np.float32(np.sign(seg[k]) * 448) * s[i, b]
            assert abs(back[i, 128 * b + k] - seg[k]) <= np.spacing(np.abs(seg[k]))


def test_metric_sqrt_inv_closed_form():
    """(A + lam I)^{-1/2} of matrices with known eigenpairs: diag(4, 1/4) gives
    diag(1/2, 2) (an exponent of the wrong sign gives diag(2, 1/2)); a rotated
    copy gives the rotated result; damping adds lam before the root."""
    S = og.metric_sqrt_inv(np.diag([4.0, 0.25]), 0.0)
    assert np.allclose(S, np.diag([0.5, 2.0]), rtol=0, atol=1e-14)
    c, s = np.cos(0.3), np.sin(0.3)
    R = np.array([[c, -s, 0.0], [s, c, 0.0], [0.0, 0.0, 1.0]])
    A = R @ np.diag([4.0, 0.25, 9.0]) @ R.T
    S = og.metric_sqrt_inv(A, 0.0)
    assert np.allclose(S, R @ np.diag([0.5, 2.0, 1.0 / 3.0]) @ R.T, rtol=0, atol=1e-13)
    assert np.allclose(S @ A @ S, np.eye(3), rtol=0, atol=1e-13)
    S = og.metric_sqrt_inv(np.diag([3.0, 15.0]), 1.0)
    assert np.allclose(S, np.diag([0.5, 0.25]), rtol=0, atol=1e-14)


def test_rel_error_kfac_closed_form():
    """M2 of an error along one eigenvector of A and a gradient along another:
    A = diag(4, 1/4), G rows along e1 (metric weight 1/2), error along e2
    (metric weight 2): M2 = (0.1 * 2) / (1 * 1/2) = 0.4 while M1 = 0.1; the
    error moved to e1 gives M2 = M1.  G has three rows so a product taken on
    the wrong side (S E instead of E S) does not even have a valid shape."""
    S = og.metric_sqrt_inv(np.diag([4.0, 0.25]), 0.0)
    G = np.array([[1.0, 0.0], [0.0, 0.0], [0.0, 0.0]])
    Gh = G + np.array([[0.0, 0.1], [0.0, 0.0], [0.0, 0.0]])
    assert abs(og.rel_frobenius(G, Gh) - 0.1) < 1e-15
    assert abs(og.rel_error_kfac(G, Gh, S) - 0.4) < 1e-14
    Gh1 = G + np.array([[0.1, 0.0], [0.0, 0.0], [0.0, 0.0]])
    assert abs(og.rel_error_kfac(G, Gh1, S) - 0.1) < 1e-14
    # a gradient along e2 with error along e1: weights swap, M2 = 0.1 * (1/2) / 2
    G2 = np.array([[0.0, 1.0], [0.0, 0.0], [0.0, 0.0]])
    Gh2 = G2 + np.array([[0.1, 0.0], [0.0, 0.0], [0.0, 0.0]])
    assert abs(og.rel_error_kfac(G2, Gh2, S) - 0.025) < 1e-14


def test_tiny_amax_gets_the_largest_finite_scale():
    """An amax below 448 / FLT_MAX (about 1.3e-36): 448 / amax overflows, the
    scale is FLT_MAX, zeros stay code 0 (no NaN from 0 * inf), the largest
    element gets E4M3(fl32(amax * FLT_MAX)) and no flag is raised.  Just above
    the threshold the division is finite and used as is."""
    fmax = np.finfo(np.float32).max
    w = np.zeros((2, 128), dtype=np.float32)
    w[0, 3] = np.float32(1e-38)
    w[1, 7] = np.float32(-5e-39)
    scale, inv, flags = og.scale_from_amax(og.amax(w))
    assert scale == fmax and flags == 0
    assert inv == np.float32(1e-38) / np.float32(448)
    codes, inv2, flags2 = og.quantize_tensor(w)
    assert flags2 == 0 and inv2 == inv
    assert np.count_nonzero(codes) == 2 and not np.any((codes & 0x7F) == 0x7F)
    assert codes[0, 3] == e4m3.encode(np.array([np.float32(1e-38) * fmax], np.float32))[0]
    assert codes[0, 3] == 0x46          # 3.403 is above the 3.375 midpoint: 3.5 (0x46)
    assert codes[1, 7] == e4m3.encode(np.array([np.float32(-5e-39) * fmax], np.float32))[0]
    a = np.float32(1e-35)               # above the threshold: the plain quotient
    s_ok, _, _ = og.scale_from_amax(a)
    assert s_ok == np.float32(448) / a and np.isfinite(s_ok)
    # per-segment scaling takes the same rule
    c128, inv128, _ = og.quantize_block128(w)
    assert np.array_equal(c128, codes) and inv128[0, 0] == inv


def test_rank_64_factor_with_width_96_matches_eigh(layer):
    """The rank sweep's largest rank: 64 Ritz pairs from a 96-wide sketch (the
    same 32 columns of oversampling as rank 32 from 64): the top 48 Ritz
    values within 1e-4 of eigh, all 64 within 2e-3, the subspace close to the
    top-64 eigenvectors, the rank-64 part within 1e-3 of the best rank-64
    approximation (Eckart-Young), and the tail the mean of the 448 discarded
    eigenvalues; its coefficients represent the dense matrix functions."""
    A, X = layer["A"], layer["X"]
    omega = synth.gaussian_sketch(512, 96, seed=14).numpy()
    f = og.refresh_factor(X, omega, rank=64, A=A)
    w, V = np.linalg.eigh(A)
    w, V = w[::-1], V[:, ::-1]
    assert f.U.shape == (512, 64) and f.theta.shape == (64,)
    rel = np.abs(f.theta - w[:64]) / w[:64]
    assert rel[:48].max() < 1e-4 and rel.max() < 2e-3
    assert np.linalg.svd(V[:, :64].T @ f.U, compute_uv=False).min() > 0.99
    best = np.sqrt(np.sum(w[64:] ** 2))
    assert np.linalg.norm(A - (f.U * f.theta) @ f.U.T) <= best * (1 + 1e-3)
    assert abs(f.sigma2_tail - np.mean(w[64:])) < 1e-3 * np.mean(w[64:])
    inv_sqrt = f.alpha * np.eye(512) + (f.U * f.d_w) @ f.U.T
    assert np.linalg.norm(inv_sqrt - _dense_power(f.dense(), -0.5)) < 1e-9 * np.linalg.norm(inv_sqrt)
