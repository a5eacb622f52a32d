"""The tile height of the round-trip kernels does not change results.

A call whose whitened layers hold fewer than 2^25 elements runs the tile
kernels with 32-row tiles, a larger call the 64-row ones.  A row's partial
products depend only on the column grouping, which both share, and the
16-row MFMA tiles are the same, so the codes, scales and reconstruction of
a small group must be bit-identical whether it is called alone or together
with a large layer that moves the call to 64-row tiles.  Per-tensor E4M3,
1x128 E4M3 and MXFP4; ragged row counts.
"""

import numpy as np
import pytest
import torch

import synth
import fac_whitening_gift_amd as fg
from oracle import gift as og
from gpu_util import DEV, host, say, to_dev, upload_factor

pytestmark = pytest.mark.gpu


def _small_group(scaling):
    out = []
    for k, (d_out, d_in) in enumerate([(300, 512), (77, 1024), (1024, 256)]):
        spec = synth.InputSpec("x", d_in, 2048, 1.5, bf16=False)
        inp = synth.draw_input(spec, seed=40 + k)
        omega = synth.gaussian_sketch(d_in, og.SKETCH_WIDTH, seed=50 + k).numpy()
        f = upload_factor(og.refresh_factor(inp["X"].numpy(), omega))
        G = to_dev(synth.draw_gradient(d_out, inp["Q"], inp["ev"], seed=60 + k).numpy())
        out.append((G, f))
    return out


def _layers(group, scaling):
    return [fg.Layer(G, factor=f, block128=scaling == fg.SCALE_BLOCK128,
                     mxfp4=scaling == fg.SCALE_MXFP4) for G, f in group]


@pytest.mark.parametrize("scaling", [fg.SCALE_TENSOR, fg.SCALE_BLOCK128, fg.SCALE_MXFP4])
def test_tile_height_does_not_change_results(scaling):
    say("tile heights: scaling %d" % scaling)
    group = _small_group(scaling)
    alone = _layers(group, scaling)
    fg.gift_whiten_quantize(alone, scaling=scaling)
    fg.gift_dequant_unwhiten(alone, scaling=scaling)
    # one large layer (8192 x 4096 = 2^25 elements) in the same calls
    spec = synth.InputSpec("big", 4096, 1024, 1.5, bf16=True)
    inp = synth.draw_input(spec, seed=70, device=DEV, as_bf16=True)
    fbig = fg.Factor(4096, device=DEV)
    fg.gift_refresh_factors([dict(X=inp["X"], factor=fbig, seed=1)], power_steps=1)
    Gbig = torch.randn(8192, 4096, device=DEV)
    big = fg.Layer(Gbig, factor=fbig, block128=scaling == fg.SCALE_BLOCK128,
                   mxfp4=scaling == fg.SCALE_MXFP4)
    mixed = _layers(group, scaling)
    fg.gift_whiten_quantize(mixed + [big], scaling=scaling)
    fg.gift_dequant_unwhiten(mixed + [big], scaling=scaling)
    for a, b in zip(alone, mixed):
        assert np.array_equal(host(a.q), host(b.q))
        assert np.array_equal(host(a.inv_scale), host(b.inv_scale))
        assert np.array_equal(host(a.G_hat), host(b.G_hat))
