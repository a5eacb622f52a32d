"""Device parity of the slab whiten: rank-r whitened layers of at least
2^22 elements with per-tensor scaling whiten one workgroup per 64-row block
(c', then the block's amax of |W|), then quantize on the 64-row tile
kernels; their dequantize + un-whiten runs on the tile kernels.

Shapes cover ragged last row blocks, chunk counts that leave some waves one
chunk short (d_in / 32 not a multiple of 8) or with no chunk at all
(d_in = 64), long rows, and layers of more row blocks than the quantize
pass reduces itself.  Protocol as for the tile kernels: W within 1e-5 of
the oracle, codes and scale bit-exact against the oracle's encoding of the
device's W, G^ within 1e-5 of the oracle's un-whitening of the device's
codes, error sums within 1e-12.  A grouped call gives every layer the
results of its own call (the slab / tile choice depends on the layer alone),
also when the slab pass runs over more layers than one launch holds inline.
"""

import numpy as np
import pytest
import torch

import fac_whitening_gift_amd as fg
from oracle import gift as og
from gpu_util import host, say, to_dev, upload_factor
from test_gpu_roundtrip import _cheap_factor, _gift_parity

pytestmark = pytest.mark.gpu

SLAB_MIN = 1 << 22


def _anisotropic(d_out, d_in, U, seed):
    rng = np.random.default_rng(seed)
    Z = rng.standard_normal((d_out, d_in))
    return (np.exp(rng.standard_normal((d_out, 1))) *
            (Z + 10.0 * rng.standard_normal((d_out, 32)) @ U.T)).astype(np.float32)


@pytest.mark.parametrize("d_out,d_in", [(16411, 288), (70001, 64), (4097, 1056), (1000, 4224),
                                        (140003, 32 * 40)])
def test_slab_parity(d_out, d_in):
    assert d_out * d_in >= SLAB_MIN
    say("slab parity %dx%d" % (d_out, d_in))
    f, U = _cheap_factor(d_in, seed=d_in + 7)
    G = _anisotropic(d_out, d_in, U, seed=d_out)
    _gift_parity(G, upload_factor(f), False)


def test_slab_layers_in_a_group_match_their_own_calls():
    say("slab + tile layers grouped vs alone")
    fa, Ua = _cheap_factor(1024, seed=3)
    fb, Ub = _cheap_factor(512, seed=4)
    da, db = upload_factor(fa), upload_factor(fb)
    specs = [(_anisotropic(4100, 1024, Ua, 1), da), (_anisotropic(300, 512, Ub, 2), db),
             (_anisotropic(8200, 512, Ub, 3), db), (np.random.default_rng(4).standard_normal(
                 (64, 256)).astype(np.float32), None)]
    group = [fg.Layer(to_dev(G), factor=f) for G, f in specs]
    fg.gift_whiten_quantize(group)
    fg.gift_dequant_unwhiten(group)
    for i, (G, f) in enumerate(specs):
        one = fg.Layer(to_dev(G), factor=f)
        fg.gift_whiten_quantize([one])
        fg.gift_dequant_unwhiten([one])
        assert np.array_equal(host(group[i].q), host(one.q)), i
        assert host(group[i].inv_scale)[0] == host(one.inv_scale)[0], i
        assert np.array_equal(host(group[i].G_hat).view(np.uint32), host(one.G_hat).view(np.uint32)), i


def test_slab_nonfinite_and_zero():
    """A NaN in one row of a slab layer: every code and the scale are what the
    oracle gives for the device's W (the layer amax is NaN); an all-zero slab
    layer gives zero codes, scale 1 and the zero flag."""
    say("slab nonfinite / zero")
    f, U = _cheap_factor(256, seed=9)
    df = upload_factor(f)
    G = _anisotropic(16400, 256, U, seed=10)
    G[7000, 31] = np.nan
    for case in ("nan", "zero"):
        Gc = np.zeros_like(G) if case == "zero" else G
        Gd = to_dev(Gc)
        W = torch.empty_like(Gd)
        flags = torch.zeros(1, dtype=torch.int32, device="cuda")
        L = fg.Layer(Gd, factor=df, W_out=W)
        fg.gift_whiten_quantize([L], flags=flags)
        fg.gift_dequant_unwhiten([L])
        codes, inv, fl = og.quantize_tensor(host(W))
        assert np.array_equal(host(L.q), codes), case
        got = host(L.inv_scale)[0]
        assert (np.isnan(got) and np.isnan(inv)) or got == inv, case
        assert int(host(flags)[0]) == fl, case
        if case == "zero":
            assert fl == og.FLAG_ZERO_AMAX and not np.any(host(L.q)) and not np.any(host(L.G_hat))
        else:
            assert fl & og.FLAG_NONFINITE and np.all(np.isnan(host(L.G_hat)))


def test_slab_group_beyond_inline_descriptors():
    """More slab layers than a launch holds inline (the slab pass then reads
    its layer descriptors from the workspace), mixed with tile-path and
    Euclidean layers: every layer's codes, scale and reconstruction are
    bit-identical to those of its own call, and the flags to the OR of the
    single calls' flags."""
    say("slab group of 20 + 3 other layers vs alone")
    fa, Ua = _cheap_factor(1024, seed=21)
    fb, Ub = _cheap_factor(512, seed=22)
    da, db = upload_factor(fa), upload_factor(fb)
    rng = np.random.default_rng(23)
    specs = []
    for k in range(20):
        d_in, U, f = (512, Ub, db) if k % 2 else (1024, Ua, da)
        specs.append((_anisotropic(SLAB_MIN // d_in + 37 * k, d_in, U, seed=100 + k), f))
        if k in (4, 10, 16):  # a tile-path layer, a Euclidean layer, a tile-path layer
            small = _anisotropic(300 + k, 512, Ub, seed=200 + k)
            specs.append((small, None if k == 10 else db))
    assert sum(1 for G, f in specs if f is not None and G.size >= SLAB_MIN) == 20
    group = [fg.Layer(to_dev(G), factor=f) for G, f in specs]
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    fg.gift_whiten_quantize(group, flags=flags)
    fg.gift_dequant_unwhiten(group)
    want_flags = 0
    for i, (G, f) in enumerate(specs):
        one = fg.Layer(to_dev(G), factor=f)
        fl1 = torch.zeros(1, dtype=torch.int32, device="cuda")
        fg.gift_whiten_quantize([one], flags=fl1)
        fg.gift_dequant_unwhiten([one])
        want_flags |= int(host(fl1)[0])
        assert np.array_equal(host(group[i].q), host(one.q)), i
        assert host(group[i].inv_scale)[0] == host(one.inv_scale)[0], i
        assert np.array_equal(host(group[i].G_hat).view(np.uint32), host(one.G_hat).view(np.uint32)), i
    assert int(host(flags)[0]) == want_flags
