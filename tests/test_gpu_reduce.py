"""Device parity of the simulated data-parallel reduction: every rank's
payload dequantized and summed in fp32 in rank order (bit-exact against the
oracle's fp32 sum), then one un-whitening of the sum (within 1e-5 of the
oracle's fp64 un-whitening of the device's sum)."""

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
FMT = {"tensor": fg.SCALE_TENSOR, "block128": fg.SCALE_BLOCK128, "mxfp4": fg.SCALE_MXFP4}


def _factor_for(d_in, seed):
    spec = synth.InputSpec("x", d_in, 2048, 1.5, bf16=False)
    inp = synth.draw_input(spec, seed=seed)
    omega = synth.gaussian_sketch(d_in, og.SKETCH_WIDTH, seed=seed + 1).numpy()
    return inp, og.refresh_factor(inp["X"].numpy(), omega)


def _layer(G, f, fmt, **kw):
    return fg.Layer(G, factor=f, block128=fmt == "block128", mxfp4=fmt == "mxfp4", **kw)


@pytest.mark.parametrize("fmt", ["tensor", "block128", "mxfp4"])
def test_reduce_ranks_parity(fmt):
    say("reduce 5 ranks %s" % fmt)
    R = 5
    ia, fa = _factor_for(256, seed=61)
    ib, fb = _factor_for(384, seed=62)
    da, db = upload_factor(fa), upload_factor(fb)
    shapes = [(ia, da, 200), (ib, db, 37), (None, None, 90)]
    grads = []
    for r in range(R):
        row = []
        for k, (inp, df, d_out) in enumerate(shapes):
            if inp is None:
                G = np.random.default_rng(100 * r + k).standard_normal((d_out, 384)).astype(np.float32)
            else:
                G = synth.draw_gradient(d_out, inp["Q"], inp["ev"], seed=100 * r + k).numpy()
            row.append(G)
        grads.append(row)
    sc = FMT[fmt]
    # every rank quantizes its own gradients (whitened with the shared factors)
    ranks = []
    for r in range(R):
        layers = [_layer(to_dev(G), df, fmt) for G, (_, df, _) in zip(grads[r], shapes)]
        fg.gift_whiten_quantize(layers, scaling=sc)
        ranks.append(layers)
    # the receive side: accumulate into rank 0's G_hat, then un-whiten once
    acc = [torch.empty_like(L.G) for L in ranks[0]]
    for r in range(R):
        view = [_layer(None, L.factor, fmt, q=L.q, inv_scale=L.inv_scale, G_hat=a,
                       d_out=L.d_out, d_in=L.d_in, allocate=False)
                for L, a in zip(ranks[r], acc)]
        fg.gift_dequant_accumulate(view, scaling=sc, first=r == 0)
    S = [host(a) for a in acc]
    for k in range(len(shapes)):
        payloads = [(fmt, host(ranks[r][k].q), host(ranks[r][k].inv_scale)) for r in range(R)]
        if fmt == "tensor":
            payloads = [(f_, c, s.reshape(())) for f_, c, s in payloads]
        ref = og.reduce_payloads(payloads)
        assert np.array_equal(S[k].view(np.uint32), ref.view(np.uint32)), k
    final = [_layer(None, L.factor, fmt, q=L.q, inv_scale=L.inv_scale, G_hat=a,
                    d_out=L.d_out, d_in=L.d_in, allocate=False) for L, a in zip(ranks[0], acc)]
    fg.gift_unwhiten_f32(final)
    for k, (_, df, _) in enumerate(shapes):
        out = host(acc[k])
        if df is None:
            assert np.array_equal(out, S[k])        # Euclidean layers untouched
        else:
            U, _, beta, _, du = factor_host(df)
            assert rel_fro(out, og.unwhiten_with(S[k], U, beta, du)) <= TOL, k


def test_accumulate_order_is_rank_order():
    """Payload values 2^24, 1, -2^24 in that order sum to 0 in fp32."""
    say("reduce order")
    codes_one = torch.full((1, 128), 0x38, dtype=torch.uint8, device=DEV)
    codes_mone = torch.full((1, 128), 0xB8, dtype=torch.uint8, device=DEV)
    acc = torch.empty(1, 128, device=DEV)
    pays = [(codes_one, 2.0 ** 24), (codes_one, 1.0), (codes_mone, 2.0 ** 24)]
    for r, (c, inv) in enumerate(pays):
        L = fg.Layer(None, q=c, inv_scale=torch.tensor([inv], device=DEV, dtype=torch.float32),
                     G_hat=acc, d_out=1, d_in=128, allocate=False)
        fg.gift_dequant_accumulate([L], first=r == 0)
    assert np.all(host(acc) == 0.0)
