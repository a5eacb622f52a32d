"""Device parity on the edge cases of the whitened paths and the refresh.

* Non-finite and all-zero gradients through gift_whiten_quantize /
  gift_dequant_unwhiten with a rank-32 factor (per-tensor, 1x128 and MXFP4)
  and with a block-A-32 factor (per-tensor, 1x128): codes, scales and flags
  bit-exact against the oracle's encoding of the device's own whitened
  tensor; the whitened tensor within 1e-5 of the oracle on its finite rows
  and non-finite in the same places; the reconstruction within 1e-5 of the
  oracle's un-whitening of the device's codes on its finite rows, with the
  same non-finite pattern.
* A tensor whose amax is below 448 / FLT_MAX (the scale clamp): Euclidean
  per-tensor and 1x128 round trips bit-exact, and the whitened path's codes
  and scales bit-exact on the device's whitened tensor.
* The refresh flag: a NaN, an infinity, or a bf16 value whose square
  overflows fp32 in X raises GIFT_FLAG_NONFINITE (the condition is forced
  from the host; every kernel still runs to completion); clean X does not.
* The measurement harness's K-FAC metric error (bench.py: kfac_metric,
  m2_parts) against oracle.metric_sqrt_inv and oracle.rel_error_kfac, and
  the reference study's per-layer round trips (bench.reference_outputs)
  against oracle.reference_roundtrip's steps.
"""

import numpy as np
import pytest
import torch

import bench
import synth
import fac_whitening_gift_amd as fg
from oracle import gift as og
from oracle import mxfp4 as mx
from gpu_util import DEV, factor_host, host, rel_fro, say, to_dev, upload_factor

pytestmark = pytest.mark.gpu

TOL = 1e-5
D_OUT, D_IN = 48, 256


def _rank_factor():
    rng = np.random.default_rng(3)
    U = np.linalg.qr(rng.standard_normal((D_IN, 32)))[0]
    theta = 40.0 * np.arange(1, 33, dtype=np.float64) ** -1.5
    return upload_factor(og.factor_from_parts(U, theta, 1e-2))


def _block_factor():
    spec = synth.InputSpec("x", D_IN, 2048, 1.5, bf16=False)
    inp = synth.draw_input(spec, seed=77)
    f = fg.Factor(D_IN, block=32)
    fg.gift_refresh_factor(inp["X"].to(DEV), f)
    torch.cuda.synchronize()
    return f


def _gradient(case):
    rng = np.random.default_rng(11)
    G = (rng.standard_normal((D_OUT, D_IN)) * np.exp(rng.standard_normal((D_OUT, 1)))).astype(np.float32)
    if case == "nan":
        G[5, 17] = np.nan
    elif case == "inf":
        G[7, 100] = np.inf
        G[30, 200] = -np.inf
    elif case == "zero":
        G[:] = 0.0
        G[3, 9] = -0.0
    elif case == "tiny":
        G = (G * np.float32(1e-39)).astype(np.float32)
    return G


def _same_nonfinite(a, b):
    return np.array_equal(np.isfinite(a), np.isfinite(b))


def _finite_rows(a):
    return np.flatnonzero(np.all(np.isfinite(a), axis=1))


def _close_on_finite_rows(dev, ref):
    """Within TOL relative Frobenius on the rows finite in the reference
    (exactly equal where those rows are all zero)."""
    rows = _finite_rows(ref)
    if rows.size == 0:
        return
    if np.any(ref[rows]):
        assert rel_fro(dev[rows], ref[rows]) <= TOL
    else:
        assert np.array_equal(dev[rows], ref[rows].astype(np.float32))


def _bits_equal(a, b):
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    # NaN payloads are not part of the reading: compare NaN as NaN
    both_nan = np.isnan(a) & np.isnan(b)
    return np.array_equal(np.where(both_nan, 0, a.view(np.uint32)), np.where(both_nan, 0, b.view(np.uint32)))


def _encode(W, scaling):
    if scaling == fg.SCALE_MXFP4:
        return mx.quantize(W)
    return og.quantize(W, scaling == fg.SCALE_BLOCK128)


def _decode(codes, scales, scaling):
    if scaling == fg.SCALE_MXFP4:
        return mx.dequantize(codes, scales)
    return og.dequantize(codes, scales, scaling == fg.SCALE_BLOCK128)


@pytest.mark.parametrize("kind", ["rank32", "block32"])
@pytest.mark.parametrize("scaling", [fg.SCALE_TENSOR, fg.SCALE_BLOCK128, fg.SCALE_MXFP4])
@pytest.mark.parametrize("case", ["nan", "inf", "zero", "tiny"])
def test_whitened_edge_cases(kind, scaling, case):
    if kind == "block32" and scaling == fg.SCALE_MXFP4:
        pytest.skip("block factors take no MXFP4 payload")
    say("edge %s scaling=%d case=%s" % (kind, scaling, case))
    f = _rank_factor() if kind == "rank32" else _block_factor()
    G = _gradient(case)
    Gd = to_dev(G)
    W = torch.empty_like(Gd)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    L = fg.Layer(Gd, factor=f, W_out=W, block128=scaling == fg.SCALE_BLOCK128,
                 mxfp4=scaling == fg.SCALE_MXFP4)
    fg.gift_whiten_quantize([L], scaling=scaling, flags=flags)
    fg.gift_dequant_unwhiten([L], scaling=scaling)
    Wg, q, sc, gh = host(W), host(L.q), host(L.inv_scale), host(L.G_hat)
    # the codes, scales and flags of the device's own whitened tensor
    codes, scales, fl = _encode(Wg, scaling)
    assert np.array_equal(q, codes)
    if scaling == fg.SCALE_MXFP4:
        assert np.array_equal(sc, scales)
    else:
        assert _bits_equal(sc.reshape(np.shape(scales)), scales)
    assert int(host(flags)[0]) == fl
    if kind == "rank32":
        U, alpha, beta, dw, du = factor_host(f)
        w_ref = og.whiten_with(G, U, alpha, dw)
        g_ref = og.unwhiten_with(_decode(q, sc.reshape(np.shape(scales)), scaling), U, beta, du)
    else:
        S, Si = host(f.S), host(f.S_inv)
        w_ref = og.block_apply(G, S)
        g_ref = og.block_apply(_decode(q, sc.reshape(np.shape(scales)), scaling), Si)
    if case == "tiny":
        # products of values near the bottom of the fp32 range: the whitened
        # tensor and its reconstruction are subnormal, where the matrix cores
        # may flush; the clamp of the scale (no NaN code from a finite
        # tensor) is what this case checks
        if scaling != fg.SCALE_MXFP4:
            assert not np.any((q & 0x7F) == 0x7F)
        assert not fl & og.FLAG_NONFINITE
        return
    assert _same_nonfinite(Wg, w_ref)
    _close_on_finite_rows(Wg, w_ref)
    assert _same_nonfinite(gh, g_ref)
    _close_on_finite_rows(gh, g_ref)
    if case == "zero":
        assert fl == og.FLAG_ZERO_AMAX and not np.any(q) and np.all(gh == 0)
    else:
        assert fl & og.FLAG_NONFINITE


@pytest.mark.parametrize("block", [False, True])
def test_euclid_tiny_amax_scale_clamp(block):
    """Segments and a tensor whose amax is 1e-38: the scale is FLT_MAX, zeros
    code 0 (not NaN), bit-exact with the oracle; other segments as usual."""
    say("euclid tiny amax block=%s" % block)
    rng = np.random.default_rng(5)
    G = np.zeros((4, 256), dtype=np.float32)
    G[0, :128] = (rng.standard_normal(128) * 1e-38).astype(np.float32)
    G[0, 3] = np.float32(1e-38)
    G[0, 7] = 0.0
    if block:
        G[1:, :] = rng.standard_normal((3, 256)).astype(np.float32)   # ordinary segments
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    L = fg.Layer(to_dev(G), block128=block)
    sc = fg.SCALE_BLOCK128 if block else fg.SCALE_TENSOR
    fg.gift_euclid_fp8_roundtrip([L], scaling=sc, flags=flags)
    codes, inv, gh, fl = og.euclid_roundtrip(G, block128=block)
    assert np.array_equal(host(L.q), codes)
    assert np.array_equal(host(L.inv_scale).reshape(np.shape(inv)), inv)
    assert np.array_equal(host(L.G_hat), gh)
    assert int(host(flags)[0]) == fl
    assert not np.any((codes & 0x7F) == 0x7F)
    assert codes[0, 7] == 0


@pytest.mark.parametrize("poison", ["none", "nan", "inf", "overflow"])
def test_refresh_flags_nonfinite_activations(poison):
    say("refresh flag poison=%s" % poison)
    spec = synth.InputSpec("x", 256, 2048, 1.5, bf16=True)
    inp = synth.draw_input(spec, seed=41, as_bf16=True)
    X = inp["X"].clone()
    if poison == "nan":
        X[5, 7] = float("nan")
    elif poison == "inf":
        X[9, 3] = float("-inf")
    elif poison == "overflow":
        X[11, 200] = 1e20          # finite in bf16, its square is not in fp32
    f = fg.Factor(256, device=DEV)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    fg.gift_refresh_factor(X.to(DEV), f, flags=flags)
    # grouped form, with a clean input beside the poisoned one
    f2, f3 = fg.Factor(256, device=DEV), fg.Factor(256, device=DEV)
    flags2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    fg.gift_refresh_factors([dict(X=inp["X"].to(DEV), factor=f2), dict(X=X.to(DEV), factor=f3)],
                            flags=flags2)
    want = 0 if poison == "none" else og.FLAG_NONFINITE
    assert int(host(flags)[0]) == want
    assert int(host(flags2)[0]) == want


def test_harness_kfac_metric_matches_oracle():
    """M2 as bench.py computes it (fp64 torch on the device) equals the
    oracle's metric_sqrt_inv + rel_error_kfac on the same tensors."""
    say("harness M2 vs oracle")
    spec = synth.InputSpec("x", 256, 4096, 1.5, bf16=True)
    inp = synth.draw_input(spec, seed=51, as_bf16=True)
    G = synth.draw_gradient(96, inp["Q"], inp["ev"], seed=52)
    f = fg.Factor(256, device=DEV)
    fg.gift_refresh_factor(inp["X"].to(DEV), f)
    L = fg.Layer(G.to(DEV), factor=f)
    fg.gift_whiten_quantize([L])
    fg.gift_dequant_unwhiten([L])
    S = bench.kfac_metric(inp["X"].to(DEV))
    e2, g2 = bench.m2_parts(L.G, L.G_hat, S)
    X = inp["X"].float().numpy()
    A = og.covariance(X)
    S_o = og.metric_sqrt_inv(A, og.trace_floor(A)[1])
    assert rel_fro(host(S), S_o) <= 1e-10
    m2_o = og.rel_error_kfac(G.numpy(), host(L.G_hat), S_o)
    assert abs(np.sqrt(e2 / g2) - m2_o) <= 1e-9 * m2_o


def test_reference_study_layer_matches_oracle():
    """The reference study's round trips of one gradient: the harness's
    whitened tensors within 1e-6 of the oracle's transforms of the same A;
    codes and scales bit-exact against the oracle's encoding of the device's
    whitened tensors; reconstructions equal to the oracle's inverse
    transforms of the device's codes (fp64)."""
    say("reference study layer vs oracle")
    spec = synth.InputSpec("x", 256, 4096, 1.5, bf16=True)
    inp = synth.draw_input(spec, seed=61, as_bf16=True, device=DEV)
    G = synth.draw_gradient(96, inp["Q"], inp["ev"], seed=62, device=DEV)
    f = fg.Factor(256, device=DEV)
    fg.gift_refresh_factor(inp["X"], f)
    X = inp["X"].double()
    A_dev = X.T @ X / X.shape[0]
    outs = bench.reference_outputs(G, bench.reference_factors(A_dev, torch.device(DEV)), f)
    Gh = host(G).astype(np.float64)
    A = host(A_dev)
    tr = og.reference_transforms(Gh, A)
    for name in ("input_full", "input_cholesky", "two_sided"):
        left, right, left_inv, right_inv = tr[name]
        W32, q, inv, gh = outs[name]
        Wd = host(W32)
        assert rel_fro(Wd, og._lr(Gh, left, right)) <= 1e-6, name
        codes, inv_o, _ = og.quantize(Wd, False)
        assert np.array_equal(host(q), codes), name
        assert host(inv)[0] == inv_o, name
        ref = og._lr(og.dequantize(codes, inv_o, False), left_inv, right_inv)
        assert rel_fro(host(gh), ref) <= 1e-8, name
    # the library paths of the study are the round trips tested elsewhere;
    # here their M2 terms against the oracle's metric
    S_o = og.metric_sqrt_inv(A, og.trace_floor(A)[1])
    for name in ("euclid", "gift_rank32"):
        gh = host(outs[name][3])
        e2, g2 = bench.m2_parts(G, outs[name][3], bench.reference_factors(A_dev, torch.device(DEV))["S"])
        assert abs(np.sqrt(e2 / g2) - og.rel_error_kfac(Gh, gh, S_o)) <= 1e-8 * np.sqrt(e2 / g2), name
