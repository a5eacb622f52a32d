"""Device parity of the factor refresh against the oracle.

* sketch: the device's Philox4x32-10 + Box-Muller draw against the oracle's
  own implementation of the same published definition;
* covariance A = X^T X / N within 1e-5 relative Frobenius, exactly symmetric;
* factor, with the same sketch passed to both sides: Ritz values within 1e-4
  relative, the whitening and un-whitening operators A_r^{-1/2} P and
  A_r^{1/2} P within 1e-4 on a probe P, coefficients within 1e-5;
* exact low rank (rank 20 < 32): the dependent sketch directions are dropped
  and the 20 eigenpairs still come out exact.
"""

import numpy as np
import pytest
import torch

import synth
import fac_whitening_gift_amd as fg
from oracle import gift as og
from oracle import philox
from gpu_util import DEV, host, rel_fro, say

pytestmark = pytest.mark.gpu


def _run_refresh(X_dev, d, sketch=None, mode=fg.DAMP_FLOOR_PLUS_TAIL, width=64, steps=4,
                 seed=0, eps=1e-3, rank=32):
    f = fg.Factor(d, rank=rank)
    A = torch.empty(d, d, dtype=torch.float32, device=DEV)
    fg.gift_refresh_factor(X_dev, f, damp_eps=eps, damping_mode=mode, sketch_width=width,
                           power_steps=steps, seed=seed, sketch=sketch, A_out=A)
    torch.cuda.synchronize()
    return f, A


def _check_factor(f_dev, f_orc, P, tol_op=1e-4, tol_theta=1e-4, n_theta=32):
    U = host(f_dev.U).astype(np.float64)
    th = host(f_dev.theta).astype(np.float64)
    c = host(f_dev.coef).astype(np.float64)
    assert np.allclose(th[:n_theta], f_orc.theta[:n_theta], rtol=tol_theta,
                       atol=1e-7 * f_orc.theta[0])
    for k, ref in ((fg.COEF_LAMBDA_ISO, f_orc.lambda_iso), (fg.COEF_ALPHA, f_orc.alpha),
                   (fg.COEF_BETA, f_orc.beta), (fg.COEF_TRACE, f_orc.trace),
                   (fg.COEF_LAMBDA_FLOOR, f_orc.lambda_floor)):
        assert abs(c[k] - ref) <= 1e-5 * abs(ref), k
    dw = c[fg.COEF_DW:fg.COEF_DW + 32]
    du = c[fg.COEF_DU:fg.COEF_DU + 32]
    W_dev = og.whiten_with(P, U, c[fg.COEF_ALPHA], dw)
    W_orc = og.whiten(P, f_orc)
    assert rel_fro(W_dev, W_orc) <= tol_op
    assert rel_fro(og.unwhiten_with(P, U, c[fg.COEF_BETA], du), og.unwhiten(P, f_orc)) <= tol_op
    # U has orthonormal columns (to fp32 rounding)
    assert np.linalg.norm(U.T @ U - np.eye(32)) < 1e-5


def test_sketch_matches_oracle_philox():
    say("sketch d=1000 w=64 seed=0x123456789")
    seed = 0x1_2345_6789
    out = host(fg.gift_draw_sketch(1000, 64, seed))
    ref = philox.gaussian_sketch(1000, 64, seed).astype(np.float32)
    diff_ulp = np.abs(out.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert diff_ulp.max() <= 1
    assert np.count_nonzero(diff_ulp) <= 4
    # ragged total (not a multiple of 4) and another seed
    out2 = host(fg.gift_draw_sketch(33, 3, 7))
    ref2 = philox.gaussian_sketch(33, 3, 7).astype(np.float32)
    assert np.max(np.abs(out2 - ref2) / np.maximum(np.abs(ref2), 1e-30)) <= 2 ** -23


@pytest.mark.parametrize("n,d,bf16", [(4096, 512, False), (8192, 1024, True), (1000, 192, True),
                                      (17, 64, False), (3000, 1040, True)])
def test_covariance(n, d, bf16):
    say("covariance n=%d d=%d bf16=%s" % (n, d, bf16))
    spec = synth.InputSpec("x", d, n, 1.5, bf16=bf16)
    inp = synth.draw_input(spec, seed=n + d, as_bf16=bf16)
    X = inp["X"]
    Xh = X.float().numpy()
    f, A = _run_refresh(X.to(DEV), d, steps=1)
    Ad = host(A)
    assert np.array_equal(Ad, Ad.T)
    assert rel_fro(Ad, og.covariance(Xh)) <= 1e-5
    tr = float(host(f.coef)[fg.COEF_TRACE])
    assert abs(tr - np.trace(og.covariance(Xh))) <= 1e-5 * abs(tr)


@pytest.mark.parametrize("mode", [fg.DAMP_FLOOR_PLUS_TAIL, fg.DAMP_FLOOR])
def test_factor_single_layer(mode):
    """d_in 512, 4096 fp32 tokens, the same sketch on both sides."""
    say("factor single layer mode=%d" % mode)
    spec = synth.InputSpec("x", 512, 4096, 1.5, bf16=False)
    inp = synth.draw_input(spec, seed=41)
    omega = synth.gaussian_sketch(512, 64, seed=42)
    f_dev, _ = _run_refresh(inp["X"].to(DEV), 512, sketch=omega.to(DEV), mode=mode)
    omode = og.DAMPING_FLOOR_PLUS_TAIL if mode == fg.DAMP_FLOOR_PLUS_TAIL else og.DAMPING_FLOOR
    f_orc = og.refresh_factor(inp["X"].numpy(), omega.numpy().astype(np.float64), mode=omode)
    P = np.random.default_rng(3).standard_normal((64, 512))
    _check_factor(f_dev, f_orc, P)


def test_factor_with_device_sketch_is_close():
    """Without a sketch the device draws its own (Philox); the oracle draws
    the same definition in fp64: the operators agree."""
    say("factor device sketch")
    spec = synth.InputSpec("x", 512, 4096, 1.5, bf16=False)
    inp = synth.draw_input(spec, seed=43)
    f_dev, _ = _run_refresh(inp["X"].to(DEV), 512, seed=99)
    f_orc = og.refresh_factor(inp["X"].numpy(), philox.gaussian_sketch(512, 64, 99))
    P = np.random.default_rng(4).standard_normal((64, 512))
    _check_factor(f_dev, f_orc, P)


def test_exact_low_rank_drops_dependent_directions():
    say("factor exact rank 20")
    rng = np.random.default_rng(8)
    d, k, n = 256, 20, 2048
    B = np.linalg.qr(rng.standard_normal((d, k)))[0] * np.linspace(3, 0.5, k)
    X = (rng.standard_normal((n, k)) @ B.T).astype(np.float32)
    omega = synth.gaussian_sketch(d, 64, seed=5)
    f_dev, _ = _run_refresh(torch.from_numpy(X).to(DEV), d, sketch=omega.to(DEV))
    A = og.covariance(X)
    w, V = np.linalg.eigh(A)
    w, V = w[::-1], V[:, ::-1]
    th = host(f_dev.theta).astype(np.float64)
    U = host(f_dev.U).astype(np.float64)
    assert np.allclose(th[:k], w[:k], rtol=1e-4)
    assert np.all(th[k:] <= 1e-5 * w[0])
    Pk = U[:, :k] @ U[:, :k].T
    assert np.linalg.norm(Pk - V[:, :k] @ V[:, :k].T) < 1e-4
    assert np.all(np.isfinite(host(f_dev.coef)))


@pytest.mark.parametrize("width,steps", [(32, 4), (48, 2), (64, 0)])
def test_width_and_power_steps(width, steps):
    say("factor width=%d steps=%d" % (width, steps))
    spec = synth.InputSpec("x", 256, 2048, 2.0, bf16=True)
    inp = synth.draw_input(spec, seed=44, as_bf16=True)
    omega = synth.gaussian_sketch(256, width, seed=45)
    f_dev, _ = _run_refresh(inp["X"].to(DEV), 256, sketch=omega.to(DEV), width=width, steps=steps)
    f_orc = og.refresh_factor(inp["X"].float().numpy(), omega.numpy().astype(np.float64),
                              power_steps=steps)
    P = np.random.default_rng(5).standard_normal((32, 256))
    # same subspace iteration on both sides: only the well-separated head of
    # the spectrum is compared when the iteration is short or narrow
    _check_factor(f_dev, f_orc, P, tol_op=1e-3 if steps < 4 or width < 64 else 1e-4,
                  tol_theta=1e-3, n_theta=16)


def test_refresh_is_deterministic():
    say("refresh determinism")
    spec = synth.InputSpec("x", 1024, 8192, 1.5, bf16=True)
    inp = synth.draw_input(spec, seed=46, as_bf16=True)
    X = inp["X"].to(DEV)
    f1, A1 = _run_refresh(X, 1024, seed=3)
    f2, A2 = _run_refresh(X, 1024, seed=3)
    assert torch.equal(A1, A2) and torch.equal(f1.U, f2.U) and torch.equal(f1.coef, f2.coef)


@pytest.fixture(scope="module")
def block_inputs():
    w = synth.llama_block()
    out = []
    for k, spec in enumerate(w.inputs):
        inp = synth.draw_input(spec, seed=800 + k, as_bf16=True)
        out.append((spec, inp))
    return out


def test_full_block_factors(block_inputs):
    """The four inputs of a hidden-1024 block (8192 bf16 tokens, d_in 1024 and
    2816), refreshed as the benchmark does, against the oracle."""
    for k, (spec, inp) in enumerate(block_inputs):
        say("factor %s d=%d" % (spec.name, spec.d_in))
        omega = synth.gaussian_sketch(spec.d_in, 64, seed=900 + k)
        f_dev, A = _run_refresh(inp["X"].to(DEV), spec.d_in, sketch=omega.to(DEV))
        Xh = inp["X"].float().numpy()
        A_orc = og.covariance(Xh)
        assert rel_fro(host(A), A_orc) <= 1e-5
        f_orc = og.refresh_factor(Xh, omega.numpy().astype(np.float64), A=A_orc)
        P = np.random.default_rng(k).standard_normal((32, spec.d_in))
        _check_factor(f_dev, f_orc, P)


def test_grouped_refresh_matches_oracle_and_writes_packs(block_inputs):
    """All four block inputs plus one fp32 input in one grouped call; each
    factor against the oracle, and the operand packs the refresh writes equal
    gift_prepare_factor's."""
    say("grouped refresh 5 inputs")
    items, ref = [], []
    for k, (spec, inp) in enumerate(block_inputs):
        omega = synth.gaussian_sketch(spec.d_in, 64, seed=950 + k)
        f = fg.Factor(spec.d_in)
        items.append(dict(X=inp["X"].to(DEV), factor=f, sketch=omega.to(DEV)))
        ref.append((inp["X"].float().numpy(), omega.numpy().astype(np.float64)))
    spec32 = synth.InputSpec("x32", 512, 4096, 1.5, bf16=False)
    inp32 = synth.draw_input(spec32, seed=961)
    om32 = synth.gaussian_sketch(512, 64, seed=962)
    items.append(dict(X=inp32["X"].to(DEV), factor=fg.Factor(512), sketch=om32.to(DEV)))
    ref.append((inp32["X"].numpy(), om32.numpy().astype(np.float64)))
    fg.gift_refresh_factors(items)
    torch.cuda.synchronize()
    for k, (it, (Xh, om)) in enumerate(zip(items, ref)):
        f_orc = og.refresh_factor(Xh, om)
        P = np.random.default_rng(20 + k).standard_normal((16, Xh.shape[1]))
        _check_factor(it["factor"], f_orc, P)
        packs = it["factor"].packs.clone()
        fg.gift_prepare_factor(it["factor"])
        assert torch.equal(packs, it["factor"].packs)


def test_selection_from_device_factors():
    """rho from the device factors matches the oracle's (relative 1e-4), and so
    does the top-k choice, on inputs with clearly different spectra."""
    from fac_whitening_gift_amd.select import anisotropy, select_layers
    say("selection by theta_1 / tr(A)")
    exps = [1.0, 2.0, 1.4, 1.8, 1.2]
    facs, rho_o = [], []
    for k, e in enumerate(exps):
        spec = synth.InputSpec("x%d" % k, 256, 2048, e, bf16=True)
        inp = synth.draw_input(spec, seed=60 + k, as_bf16=True)
        om = synth.gaussian_sketch(256, 64, seed=70 + k)
        f = fg.Factor(256)
        fg.gift_refresh_factor(inp["X"].to(DEV), f, sketch=om.to(DEV))
        facs.append(f)
        rho_o.append(og.anisotropy(og.refresh_factor(inp["X"].float().numpy(),
                                                     om.numpy().astype(np.float64))))
    rho_d = [anisotropy(f) for f in facs]
    assert np.allclose(rho_d, rho_o, rtol=1e-4)
    layer_factors = [facs[0], None, facs[1], facs[1], facs[2], facs[3], facs[4], None]
    rhos_o = [None if f is None else rho_o[facs.index(f)] for f in layer_factors]
    for k in (1, 2, 4, 10):
        assert select_layers(layer_factors, k) == og.select_top_k(rhos_o, k)


@pytest.mark.parametrize("rank", [8, 16, 1])
def test_factor_lower_rank(rank):
    """Effective rank r < 32: the top r Ritz pairs of the same subspace,
    damping with the d_in - r discarded eigenvalues, zero columns from r on;
    the round trip through the kernels with that factor matches the oracle's
    rank-r whitening, codes and reconstruction."""
    say("factor rank %d d_in 512" % rank)
    spec = synth.InputSpec("x", 512, 4096, 1.5, bf16=False)
    inp = synth.draw_input(spec, seed=41)
    omega = synth.gaussian_sketch(512, 64, seed=42)
    f_dev, _ = _run_refresh(inp["X"].to(DEV), 512, sketch=omega.to(DEV), rank=rank)
    f_orc = og.refresh_factor(inp["X"].numpy(), omega.numpy().astype(np.float64), rank=rank)
    U = host(f_dev.U).astype(np.float64)
    th = host(f_dev.theta).astype(np.float64)
    c = host(f_dev.coef).astype(np.float64)
    dw = c[fg.COEF_DW:fg.COEF_DW + 32]
    du = c[fg.COEF_DU:fg.COEF_DU + 32]
    assert np.all(U[:, rank:] == 0) and np.all(th[rank:] == 0)
    assert np.all(dw[rank:] == 0) and np.all(du[rank:] == 0)
    assert np.allclose(th[:rank], f_orc.theta, rtol=1e-4, atol=1e-7 * f_orc.theta[0])
    for k, ref in ((fg.COEF_LAMBDA_ISO, f_orc.lambda_iso), (fg.COEF_ALPHA, f_orc.alpha),
                   (fg.COEF_SIGMA2_TAIL, f_orc.sigma2_tail)):
        assert abs(c[k] - ref) <= 1e-5 * abs(ref), k
    assert np.linalg.norm(U[:, :rank].T @ U[:, :rank] - np.eye(rank)) < 1e-5
    P = np.random.default_rng(3).standard_normal((64, 512))
    assert rel_fro(og.whiten_with(P, U, c[fg.COEF_ALPHA], dw), og.whiten(P, f_orc)) <= 1e-4
    assert rel_fro(og.unwhiten_with(P, U, c[fg.COEF_BETA], du), og.unwhiten(P, f_orc)) <= 1e-4
    # round trip with the rank-r factor (P-a, P-b, P-c against its own values)
    G = (np.random.default_rng(5).standard_normal((96, 512)) *
         np.exp(np.random.default_rng(6).standard_normal((96, 1)))).astype(np.float32)
    Gd = torch.from_numpy(G).to(DEV)
    W = torch.empty_like(Gd)
    L = fg.Layer(Gd, factor=f_dev, W_out=W)
    fg.gift_whiten_quantize([L])
    fg.gift_dequant_unwhiten([L])
    U32, alpha, beta, dw32, du32 = (host(f_dev.U), float(c[fg.COEF_ALPHA]), float(c[fg.COEF_BETA]),
                                    dw.astype(np.float32), du.astype(np.float32))
    Wg = host(W)
    assert rel_fro(Wg, og.whiten_with(G, U32, alpha, dw32)) <= 1e-5
    codes, inv_o, _ = og.quantize(Wg, False)
    assert np.array_equal(host(L.q), codes)
    ref = og.unwhiten_with(og.dequantize(host(L.q), inv_o, False), U32, beta, du32)
    assert rel_fro(host(L.G_hat), ref) <= 1e-5


def test_grouped_covariance_two_batches():
    """Nineteen bf16 inputs of mixed widths (64 .. 1040, partial column tiles)
    and token counts (ragged, fewer than one 64-token step, many steps) in one
    call: the covariance work list spans two groups of inputs with their own
    token splits.  Every A against the oracle, exactly symmetric."""
    dims = [64, 192, 1040, 272, 128, 512, 80, 336, 64, 1024, 208, 96, 144, 400, 64, 256, 176, 960, 112]
    toks = [100, 3000, 777, 1500, 63, 2048, 5, 640, 5000, 999, 130, 64, 2500, 300, 4097, 17, 1234, 700, 65]
    items, ref = [], []
    for k, (d, n) in enumerate(zip(dims, toks)):
        spec = synth.InputSpec("x%d" % k, d, n, 1.5, bf16=True)
        inp = synth.draw_input(spec, seed=3000 + k, as_bf16=True)
        A = torch.empty(d, d, dtype=torch.float32, device=DEV)
        items.append(dict(X=inp["X"].to(DEV), factor=fg.Factor(d), A_out=A, seed=k))
        ref.append(og.covariance(inp["X"].float().numpy()))
    say("grouped covariance: %d inputs" % len(items))
    fg.gift_refresh_factors(items, power_steps=1)
    torch.cuda.synchronize()
    for k, (it, A_orc) in enumerate(zip(items, ref)):
        Ad = host(it["A_out"])
        assert np.array_equal(Ad, Ad.T), k
        assert rel_fro(Ad, A_orc) <= 1e-5, (k, dims[k], toks[k])


def test_grouped_covariance_large_group():
    """Three bf16 inputs in one call: widths 4112 (17 tiles of 256, the last
    with 16 valid columns; 33 of the 128-tile partials, the last also with
    16), 4096 and 1040, ragged token counts.  The group's 304 covariance
    tiles of 256 split the longer token ranges in two, so the partials are
    written in the 128-tile layout and reduced.  Every A against the oracle,
    exactly symmetric."""
    dims, toks = [4112, 4096, 1040], [1000, 777, 300]
    items, ref = [], []
    for k, (d, n) in enumerate(zip(dims, toks)):
        spec = synth.InputSpec("w%d" % k, d, n, 1.5, bf16=True)
        inp = synth.draw_input(spec, seed=3100 + k, as_bf16=True)
        A = torch.empty(d, d, dtype=torch.float32, device=DEV)
        items.append(dict(X=inp["X"].to(DEV), factor=fg.Factor(d), A_out=A, seed=k))
        ref.append(og.covariance(inp["X"].float().numpy()))
    say("grouped covariance, large group: widths %s" % dims)
    fg.gift_refresh_factors(items, power_steps=1)
    torch.cuda.synchronize()
    for k, (it, A_orc) in enumerate(zip(items, ref)):
        Ad = host(it["A_out"])
        assert np.array_equal(Ad, Ad.T), k
        assert rel_fro(Ad, A_orc) <= 1e-5, (k, dims[k])


def test_grouped_covariance_direct_write_ragged():
    """Five bf16 inputs whose 657 covariance tiles of 256 fill the machine
    without a token split, so the covariance kernel writes A and its mirror
    image itself: widths 4112 and 2064 (the last tile column 16 wide, the
    DMA loads of the missing features landing only in rows and columns that
    are never written), token counts 300 .. 65 (ragged last steps read as
    zero past the token range).  Every A against the oracle, exactly
    symmetric."""
    dims, toks = [4112, 4112, 2064, 4112, 4112], [300, 200, 129, 100, 65]
    items, ref = [], []
    for k, (d, n) in enumerate(zip(dims, toks)):
        spec = synth.InputSpec("r%d" % k, d, n, 1.5, bf16=True)
        inp = synth.draw_input(spec, seed=3200 + k, as_bf16=True)
        A = torch.empty(d, d, dtype=torch.float32, device=DEV)
        items.append(dict(X=inp["X"].to(DEV), factor=fg.Factor(d), A_out=A, seed=k))
        ref.append(og.covariance(inp["X"].float().numpy()))
    say("grouped covariance, direct write: widths %s tokens %s" % (dims, toks))
    fg.gift_refresh_factors(items, power_steps=1)
    torch.cuda.synchronize()
    for k, (it, A_orc) in enumerate(zip(items, ref)):
        Ad = host(it["A_out"])
        assert np.array_equal(Ad, Ad.T), k
        assert rel_fro(Ad, A_orc) <= 1e-5, (k, dims[k], toks[k])


def test_chained_refresh_many_inputs():
    """Thirty-seven inputs in one call (three covariance groups, the last
    ragged; bf16 and fp32; widths 128 .. 384; ragged token counts): the chain
    after the covariance runs once over all of them with its descriptors in
    the workspace.  Every factor against the oracle, the operand packs equal
    gift_prepare_factor's, and the first sixteen (one whole covariance group,
    so the same covariance plan) bit-identical to a call of those sixteen
    alone, whose chain takes its descriptors as kernel arguments."""
    dims = [128, 192, 256, 320, 384, 160]
    toks = [700, 1500, 2048, 900, 1333]
    n = 37
    items, ref = [], []
    for k in range(n):
        d, t = dims[k % len(dims)], toks[k % len(toks)]
        bf16 = k % 5 != 3
        spec = synth.InputSpec("c%d" % k, d, t, 1.2 + 0.1 * (k % 6), bf16=bf16)
        inp = synth.draw_input(spec, seed=4000 + k, as_bf16=bf16)
        om = synth.gaussian_sketch(d, 64, seed=4100 + k)
        X = inp["X"].to(DEV)
        items.append(dict(X=X, factor=fg.Factor(d), sketch=om.to(DEV)))
        ref.append((inp["X"].float().numpy(), om.numpy().astype(np.float64)))
    say("chained refresh: %d inputs" % n)
    fg.gift_refresh_factors(items)
    torch.cuda.synchronize()
    for k, (it, (Xh, om)) in enumerate(zip(items, ref)):
        f_orc = og.refresh_factor(Xh, om)
        P = np.random.default_rng(40 + k).standard_normal((16, Xh.shape[1]))
        _check_factor(it["factor"], f_orc, P)
        packs = it["factor"].packs.clone()
        fg.gift_prepare_factor(it["factor"])
        assert torch.equal(packs, it["factor"].packs), k
    say("chained refresh: first 16 inputs alone")
    alone = [dict(X=it["X"], factor=fg.Factor(it["factor"].d_in), sketch=it["sketch"])
             for it in items[:16]]
    fg.gift_refresh_factors(alone)
    torch.cuda.synchronize()
    for k, (a, it) in enumerate(zip(alone, items[:16])):
        fa, fb = a["factor"], it["factor"]
        assert torch.equal(fa.U, fb.U) and torch.equal(fa.theta, fb.theta), k
        assert torch.equal(fa.coef, fb.coef) and torch.equal(fa.packs, fb.packs), k


def test_chained_refresh_wide_inputs():
    """Twenty-four bf16 inputs of width 1536 in one call: Y = A Q runs in its
    wide workgroup shape (inputs of width 1024 and more: 128 rows per
    workgroup, Q's operand packs shared through LDS).  Inputs 0, 11 and 23 against
    the oracle (same sketch); every factor's U orthonormal and theta equal to
    its Rayleigh quotients u^T A u."""
    n, d, t = 24, 1536, 2048
    items, ref = [], []
    for k in range(n):
        spec = synth.InputSpec("w%d" % k, d, t, 1.3 + 0.02 * k, bf16=True)
        inp = synth.draw_input(spec, seed=4200 + k, as_bf16=True)
        om = synth.gaussian_sketch(d, 64, seed=4300 + k)
        items.append(dict(X=inp["X"].to(DEV), factor=fg.Factor(d), sketch=om.to(DEV)))
        ref.append((inp["X"], om))
    say("chained refresh: %d inputs of width %d" % (n, d))
    fg.gift_refresh_factors(items)
    torch.cuda.synchronize()
    for k, it in enumerate(items):
        X = it["X"].double()
        A = X.T @ X / X.shape[0]
        U = it["factor"].U.double()
        th = it["factor"].theta.double()
        assert float(torch.linalg.norm(U.T @ U - torch.eye(32, dtype=U.dtype, device=U.device))) < 1e-5, k
        rq = ((A @ U) * U).sum(0)
        assert float((rq - th).abs().max() / th[0]) < 1e-5, k
    for k in (0, 11, 23):
        Xh, om = ref[k]
        f_orc = og.refresh_factor(Xh.float().numpy(), om.numpy().astype(np.float64))
        P = np.random.default_rng(60 + k).standard_normal((16, d))
        _check_factor(items[k]["factor"], f_orc, P)


def test_refresh_more_inputs_than_one_chain():
    """1025 small inputs in one call: two chains (1024 inputs, then 1), each
    reading its descriptors from the workspace.  Results depend only on an
    input's own covariance group, so the lone last input equals a refresh of
    that input alone and the first sixteen equal a call of those sixteen,
    bit for bit."""
    n, d = 1025, 128
    items = []
    for k in range(n):
        g = torch.Generator().manual_seed(5000 + k)
        X = (torch.randn(96 + k % 7, d, generator=g) * (1.0 + (k % 5))).to(torch.bfloat16)
        items.append(dict(X=X.to(DEV), factor=fg.Factor(d), seed=k))
    say("refresh of %d inputs (two chains)" % n)
    fg.gift_refresh_factors(items, power_steps=2)
    torch.cuda.synchronize()
    alone = [dict(X=items[-1]["X"], factor=fg.Factor(d), seed=n - 1)]
    fg.gift_refresh_factors(alone, power_steps=2)
    first = [dict(X=it["X"], factor=fg.Factor(d), seed=k) for k, it in enumerate(items[:16])]
    fg.gift_refresh_factors(first, power_steps=2)
    torch.cuda.synchronize()
    for a, b in [(alone[0], items[-1])] + list(zip(first, items[:16])):
        fa, fb = a["factor"], b["factor"]
        assert bool(torch.isfinite(fb.U).all()) and bool(torch.isfinite(fb.coef).all())
        assert torch.equal(fa.U, fb.U) and torch.equal(fa.theta, fb.theta)
        assert torch.equal(fa.coef, fb.coef) and torch.equal(fa.packs, fb.packs)
