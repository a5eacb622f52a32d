"""Device parity of rank-64 factors (the rank sweep's largest rank; its
factors store 64 columns as two rank blocks of 32).

* Refresh with a 96-wide sketch (rank + 32 oversampling): Ritz values and
  coefficients within 1e-4 of the oracle's refresh from the same sketch,
  U orthonormal, zero columns after the rank, the whitening and
  un-whitening operators on a probe within 1e-4.
* Round trip with a rank-64 factor (per-tensor, 1x128, MXFP4; a layer large
  enough for the slab whiten still runs the two-block tile kernels): W
  within 1e-5 of the oracle, codes and scales bit-exact against the
  oracle's encoding of the device's W, G^ within 1e-5 of the oracle's
  un-whitening of the device's codes.
* A grouped call over rank-32, rank-64 and Euclidean layers gives every
  layer the results of its own call; gift_unwhiten_f32 with a rank-64
  factor matches the oracle.
"""

import numpy as np
import pytest
import torch

import synth
import fac_whitening_gift_amd as fg
from oracle import gift as og
from oracle import mxfp4 as mx
from gpu_util import DEV, factor_host, host, rel_fro, say, to_dev, upload_factor

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module")
def inp512():
    spec = synth.InputSpec("x", 512, 4096, 1.5, bf16=False)
    inp = synth.draw_input(spec, seed=81)
    omega = synth.gaussian_sketch(512, 96, seed=82)
    f_orc = og.refresh_factor(inp["X"].numpy(), omega.numpy().astype(np.float64), rank=64)
    return inp, omega, f_orc


@pytest.mark.parametrize("rank", [64, 48])
def test_refresh_rank_above_32_matches_oracle(inp512, rank):
    say("refresh rank %d width 96" % rank)
    inp, omega, _ = inp512
    f_orc = og.refresh_factor(inp["X"].numpy(), omega.numpy().astype(np.float64), rank=rank)
    f = fg.Factor(512, device=DEV, rank=rank)
    assert f.cols == 64 and tuple(f.U.shape) == (512, 64)
    fg.gift_refresh_factor(inp["X"].to(DEV), f, sketch=omega.to(DEV), sketch_width=96)
    U = host(f.U).astype(np.float64)
    th = host(f.theta).astype(np.float64)
    c = host(f.coef).astype(np.float64)
    dw, du = c[8:8 + 64], c[8 + 64:8 + 128]
    assert np.all(U[:, rank:] == 0) and np.all(th[rank:] == 0)
    assert np.all(dw[rank:] == 0) and np.all(du[rank:] == 0)
    assert np.allclose(th[:rank], f_orc.theta, rtol=1e-4, atol=1e-7 * f_orc.theta[0])
    for k, ref in ((fg.COEF_LAMBDA_ISO, f_orc.lambda_iso), (fg.COEF_ALPHA, f_orc.alpha),
                   (fg.COEF_SIGMA2_TAIL, f_orc.sigma2_tail)):
        assert abs(c[k] - ref) <= 1e-4 * abs(ref), k
    assert np.linalg.norm(U[:, :rank].T @ U[:, :rank] - np.eye(rank)) < 1e-5
    P = np.random.default_rng(3).standard_normal((64, 512))
    assert rel_fro(og.whiten_with(P, U, c[fg.COEF_ALPHA], dw), og.whiten(P, f_orc)) <= 1e-4
    assert rel_fro(og.unwhiten_with(P, U, c[fg.COEF_BETA], du), og.unwhiten(P, f_orc)) <= 1e-4


def _encode(W, scaling):
    if scaling == fg.SCALE_MXFP4:
        return mx.quantize(W)[:2]
    return og.quantize(W, scaling == fg.SCALE_BLOCK128)[:2]


def _decode(q, sc, scaling):
    if scaling == fg.SCALE_MXFP4:
        return mx.dequantize(q, sc)
    return og.dequantize(q, sc, scaling == fg.SCALE_BLOCK128)


def _parity(G, df, scaling):
    Gd = to_dev(G)
    W = torch.empty_like(Gd)
    L = fg.Layer(Gd, factor=df, W_out=W, block128=scaling == fg.SCALE_BLOCK128,
                 mxfp4=scaling == fg.SCALE_MXFP4)
    fg.gift_whiten_quantize([L], scaling=scaling)
    fg.gift_dequant_unwhiten([L], scaling=scaling)
    U, alpha, beta, dw, du = factor_host(df)
    Wg, q, sc, gh = host(W), host(L.q), host(L.inv_scale), host(L.G_hat)
    assert rel_fro(Wg, og.whiten_with(G, U, alpha, dw)) <= TOL
    codes, scales = _encode(Wg, scaling)
    assert np.array_equal(q, codes)
    sc = sc.reshape(np.shape(scales))
    assert np.array_equal(sc, scales)
    ref = og.unwhiten_with(_decode(q, sc, scaling), U, beta, du)
    assert rel_fro(gh, ref) <= TOL
    return q, gh


@pytest.mark.parametrize("scaling", [fg.SCALE_TENSOR, fg.SCALE_BLOCK128, fg.SCALE_MXFP4])
@pytest.mark.parametrize("d_out", [300, 37, 4100])
def test_roundtrip_rank64_parity(inp512, scaling, d_out):
    say("round trip rank 64 %dx512 scaling=%d" % (d_out, scaling))
    inp, _, f_orc = inp512
    G = synth.draw_gradient(d_out, inp["Q"], inp["ev"], seed=90 + d_out).numpy()
    _parity(G, upload_factor(f_orc), scaling)


def test_roundtrip_rank64_large_layer_runs_tiles():
    """A 4096 x 1024 layer (2^22 elements) with a rank-64 factor: per-tensor
    scaling, which would take the slab whiten at rank 32."""
    say("round trip rank 64 4096x1024")
    rng = np.random.default_rng(7)
    U = np.linalg.qr(rng.standard_normal((1024, 64)))[0]
    theta = 80.0 * np.arange(1, 65, dtype=np.float64) ** -1.5
    f = og.factor_from_parts(U, theta, 1e-2)
    G = (np.exp(rng.standard_normal((4096, 1)))
         * (rng.standard_normal((4096, 1024)) + 10.0 * rng.standard_normal((4096, 64)) @ U.T)).astype(np.float32)
    _parity(G, upload_factor(f), fg.SCALE_TENSOR)


def test_grouped_rank32_rank64_euclid_match_their_own_calls(inp512):
    say("grouped rank 32 / 64 / Euclid")
    inp, omega, f64 = inp512
    f32 = og.refresh_factor(inp["X"].numpy(), omega.numpy()[:, :64].astype(np.float64), rank=32)
    d32, d64 = upload_factor(f32), upload_factor(f64)
    rng = np.random.default_rng(11)
    specs = [(synth.draw_gradient(200, inp["Q"], inp["ev"], seed=1).numpy(), d64),
             (synth.draw_gradient(90, inp["Q"], inp["ev"], seed=2).numpy(), d32),
             (rng.standard_normal((50, 512)).astype(np.float32), None),
             (synth.draw_gradient(131, inp["Q"], inp["ev"], seed=3).numpy(), d64)]
    for scaling in (fg.SCALE_TENSOR, fg.SCALE_BLOCK128):
        group = [fg.Layer(to_dev(G), factor=f, block128=scaling == fg.SCALE_BLOCK128)
                 for G, f in specs]
        fg.gift_whiten_quantize(group, scaling=scaling)
        fg.gift_dequant_unwhiten(group, scaling=scaling)
        for i, (G, f) in enumerate(specs):
            one = fg.Layer(to_dev(G), factor=f, block128=scaling == fg.SCALE_BLOCK128)
            fg.gift_whiten_quantize([one], scaling=scaling)
            fg.gift_dequant_unwhiten([one], scaling=scaling)
            assert np.array_equal(host(group[i].q), host(one.q)), i
            assert np.array_equal(host(group[i].G_hat).view(np.uint32), host(one.G_hat).view(np.uint32)), i


def test_unwhiten_f32_rank64(inp512):
    say("unwhiten_f32 rank 64")
    inp, _, f64 = inp512
    df = upload_factor(f64)
    S = np.random.default_rng(12).standard_normal((77, 512)).astype(np.float32)
    Gh = to_dev(S)
    L = fg.Layer(None, factor=df, q=torch.empty(77, 512, dtype=torch.uint8, device=DEV),
                 inv_scale=torch.empty(1, device=DEV), G_hat=Gh, d_out=77, d_in=512, allocate=False)
    fg.gift_unwhiten_f32([L])
    U, _, beta, _, du = factor_host(df)
    assert rel_fro(host(Gh), og.unwhiten_with(S, U, beta, du)) <= TOL
