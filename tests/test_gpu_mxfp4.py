"""Device parity of the MXFP4 payload (OCP MX: E2M1 elements, one E8M0 scale
per 32 elements of a row) through the C ABI against oracle/mxfp4.py.

Protocol as for E4M3: codes and scale bytes bit-exact against the oracle's
MXFP4 encoding of the same fp32 tensor (G for the Euclidean baseline, the
device's own whitened W for GIFT); the Euclidean reconstruction bit-exact;
the whitened tensor and the GIFT reconstruction within 1e-5 relative
Frobenius of the oracle's fp64 whitening and un-whitening.
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


def _euclid(G, flags=None):
    L = fg.Layer(to_dev(G), mxfp4=True)
    fg.gift_euclid_fp8_roundtrip([L], scaling=fg.SCALE_MXFP4, flags=flags)
    return L


def _same_floats(a, b):
    a, b = np.asarray(a, dtype=np.float32), np.asarray(b, dtype=np.float32)
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(
        np.where(np.isnan(a), 0, a).view(np.uint32), np.where(np.isnan(b), 0, b).view(np.uint32))


def _codec_rows():
    """Blocks that hit every E2M1 code, every midpoint and its neighbours,
    saturation, signed zeros, and scale codes from 0 to 254."""
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    vals = np.concatenate([mags, mids, np.nextafter(mids, np.float32(9)),
                           np.nextafter(mids, np.float32(-9)), [6.5, 7.0, 7.99, 5.5]])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    rows = []
    for e in (-127, -126, -100, -3, 0, 1, 20, 100, 124, 125):
        # amax in [4, 8) * 2^e sets the scale to 2^e (code e + 127)
        for k in range(0, vals.size, 31):
            blk = np.zeros(32, dtype=np.float64)
            chunk = vals[k:k + 31]
            blk[:chunk.size] = chunk
            blk[31] = 7.5  # amax of the block
            rows.append((blk * 2.0 ** e).astype(np.float32))
    rows.append(np.zeros(32, dtype=np.float32))
    z = np.zeros(32, dtype=np.float32)
    z[3] = -0.0
    rows.append(z)
    tiny = np.full(32, np.float32(2.0 ** -140))   # subnormal amax: scale clamped to 2^-127
    tiny[::2] *= -1
    rows.append(tiny)
    W = np.stack(rows).astype(np.float32)
    pad = (-W.shape[0]) % 4
    return np.concatenate([W, np.zeros((pad, 32), np.float32)]).reshape(-1, 128)


def test_mx_hardware_codec_matches_oracle():
    say("mxfp4 codec sweep")
    G = _codec_rows()
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    L = _euclid(G, flags)
    codes, scales, fl = mx.quantize(G)
    q, s = host(L.q), host(L.inv_scale)
    assert set(np.unique(scales).tolist()) >= {0, 1, 27, 124, 127, 128, 147, 227, 251, 252}
    bad = np.argwhere(q != codes)
    assert bad.size == 0, "first mismatches (row, byte): %s" % bad[:8].tolist()
    assert np.array_equal(s, scales)
    assert _same_floats(host(L.G_hat), mx.dequantize(codes, scales))
    assert int(host(flags)[0]) == fl == og.FLAG_ZERO_AMAX


def test_mx_nonfinite_blocks():
    say("mxfp4 nonfinite")
    G = np.ones((2, 64), dtype=np.float32)
    G[0, 3], G[0, 4], G[0, 5] = np.nan, np.inf, -7.0
    G[1, 40] = -np.inf
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    L = _euclid(G, flags)
    codes, scales, fl = mx.quantize(G)
    assert np.array_equal(host(L.q), codes) and np.array_equal(host(L.inv_scale), scales)
    assert scales[0, 0] == 0xFF and scales[1, 1] == 0xFF
    assert _same_floats(host(L.G_hat), mx.dequantize(codes, scales))
    assert int(host(flags)[0]) == fl == og.FLAG_NONFINITE


@pytest.mark.parametrize("shape", [(256, 512), (37, 96), (1, 32), (1031, 1024), (5, 4096)])
def test_euclid_mx_bit_exact(shape):
    say("euclid mxfp4 %s" % (shape,))
    rng = np.random.default_rng(shape[0] + shape[1])
    G = (rng.standard_normal(shape) * np.exp(2 * rng.standard_normal((shape[0], 1)))).astype(np.float32)
    L = _euclid(G)
    codes, scales, gh, _ = og.euclid_roundtrip_mx(G)
    assert np.array_equal(host(L.q), codes)
    assert np.array_equal(host(L.inv_scale), scales)
    assert np.array_equal(host(L.G_hat), gh)
    # send / receive halves through the grouped entry points give the same
    L2 = fg.Layer(to_dev(G), mxfp4=True)
    fg.gift_whiten_quantize([L2], scaling=fg.SCALE_MXFP4)
    fg.gift_dequant_unwhiten([L2], scaling=fg.SCALE_MXFP4)
    assert np.array_equal(host(L2.q), codes)
    assert np.array_equal(host(L2.G_hat), gh)


def _factor_for(d_in, seed, tokens=2048):
    spec = synth.InputSpec("x", d_in, tokens, 1.5, bf16=False)
    inp = synth.draw_input(spec, seed=seed)
    omega = synth.gaussian_sketch(d_in, og.SKETCH_WIDTH, seed=seed + 1).numpy()
    return inp, og.refresh_factor(inp["X"].numpy(), omega)


@pytest.mark.parametrize("d_out,d_in", [(256, 512), (37, 512), (1, 64), (300, 96),
                                        (513, 160), (200, 1024)])
def test_gift_mx_parity(d_out, d_in):
    say("gift mxfp4 parity %dx%d" % (d_out, d_in))
    inp, f = _factor_for(d_in, seed=d_in + 11)
    G = synth.draw_gradient(d_out, inp["Q"], inp["ev"], seed=d_out + 5).numpy()
    df = upload_factor(f)
    Gd = to_dev(G)
    W = torch.empty_like(Gd)
    L = fg.Layer(Gd, factor=df, W_out=W, mxfp4=True)
    fg.gift_whiten_quantize([L], scaling=fg.SCALE_MXFP4)
    fg.gift_dequant_unwhiten([L], scaling=fg.SCALE_MXFP4)
    U, alpha, beta, dw, du = factor_host(df)
    Wg, q, s, gh = host(W), host(L.q), host(L.inv_scale), host(L.G_hat)
    assert rel_fro(Wg, og.whiten_with(G, U, alpha, dw)) <= TOL
    codes, scales, _ = mx.quantize(Wg)
    assert np.array_equal(q, codes)
    assert np.array_equal(s, scales)
    ref = og.unwhiten_with(mx.dequantize(q, s), U, beta, du)
    assert rel_fro(gh, ref) <= TOL
    # the production instantiation (no W_out) writes the same codes
    L2 = fg.Layer(Gd, factor=df, mxfp4=True)
    fg.gift_whiten_quantize([L2], scaling=fg.SCALE_MXFP4)
    assert np.array_equal(host(L2.q), q) and np.array_equal(host(L2.inv_scale), s)


def test_gift_mx_grouped_mixed_layers():
    """Whitened and Euclidean layers of ragged shapes in one grouped MXFP4
    call equal one call per layer bit for bit."""
    say("gift mxfp4 grouped mixed")
    rng = np.random.default_rng(21)
    inp, f = _factor_for(256, seed=41)
    df = upload_factor(f)
    specs = []
    for i in range(9):
        d_out = int(rng.integers(1, 200))
        if i % 3 == 2:
            specs.append((rng.standard_normal((d_out, 96)).astype(np.float32), None))
        else:
            specs.append((synth.draw_gradient(d_out, inp["Q"], inp["ev"], seed=300 + i).numpy(), df))
    group = [fg.Layer(to_dev(G), factor=fa, mxfp4=True) for G, fa in specs]
    fg.gift_whiten_quantize(group, scaling=fg.SCALE_MXFP4)
    fg.gift_dequant_unwhiten(group, scaling=fg.SCALE_MXFP4)
    for i, (G, fa) in enumerate(specs):
        one = fg.Layer(to_dev(G), factor=fa, mxfp4=True)
        fg.gift_whiten_quantize([one], scaling=fg.SCALE_MXFP4)
        fg.gift_dequant_unwhiten([one], scaling=fg.SCALE_MXFP4)
        assert np.array_equal(host(group[i].q), host(one.q)), i
        assert np.array_equal(host(group[i].inv_scale), host(one.inv_scale)), i
        assert np.array_equal(host(group[i].G_hat), host(one.G_hat)), i
