"""The allocation-free send side, gift_whiten_quantize_static (its scratch
is the library's static device array, no workspace argument), against
gift_whiten_quantize with a caller workspace: two calls in a row on the same
GPU -- the second with a smaller group, so it runs on what the first left
in the array -- each bit-identical to the workspace entry point (codes,
scales, flags, and the whitened tensor where W_out is given), per-tensor,
1x128 and MXFP4; a factor without operand packs (packed into the scratch);
and a group too large for the array is refused before anything runs."""

import numpy as np
import pytest
import torch

import synth
import fac_whitening_gift_amd as fg
from oracle import gift as og
from gpu_util import DEV, host, say, to_dev, upload_factor

pytestmark = pytest.mark.gpu


def _factor(d_in, seed, packs=True):
    spec = synth.InputSpec("x", d_in, 2048, 1.5, bf16=False)
    inp = synth.draw_input(spec, seed=seed)
    omega = synth.gaussian_sketch(d_in, og.SKETCH_WIDTH, seed=seed + 1).numpy()
    df = upload_factor(og.refresh_factor(inp["X"].numpy(), omega))
    if not packs:
        df = fg.Factor(d_in, U=df.U, theta=df.theta, coef=df.coef, packs=False)
    return inp, df


def _group(specs, scaling, rng):
    layers = []
    for d_out, d_in, inp, f in specs:
        if f is None:
            G = (rng.standard_normal((d_out, d_in)) * np.exp(rng.standard_normal((d_out, 1))))
        else:
            G = synth.draw_gradient(d_out, inp["Q"], inp["ev"], seed=int(rng.integers(1 << 30))).numpy()
        Gd = to_dev(np.asarray(G, dtype=np.float32))
        layers.append(fg.Layer(Gd, factor=f, W_out=torch.empty_like(Gd),
                               block128=scaling == fg.SCALE_BLOCK128,
                               mxfp4=scaling == fg.SCALE_MXFP4))
    return layers


def _twin(layers, scaling):
    return [fg.Layer(L.G, factor=L.factor, W_out=torch.empty_like(L.G),
                     block128=scaling == fg.SCALE_BLOCK128, mxfp4=scaling == fg.SCALE_MXFP4)
            for L in layers]


@pytest.mark.parametrize("scaling", [fg.SCALE_TENSOR, fg.SCALE_BLOCK128, fg.SCALE_MXFP4])
def test_static_scratch_whiten_matches_workspace_entry(scaling):
    rng = np.random.default_rng(100 + scaling)
    inp_a, fa = _factor(1024, 11)
    inp_b, fb = _factor(512, 13, packs=False)
    first = [(700, 1024, inp_a, fa), (300, 512, inp_b, fb), (129, 1024, inp_a, fa),
             (64, 256, None, None)]
    second = [(40, 512, inp_b, fb), (17, 128, None, None)]
    for k, specs in enumerate((first, second)):
        say("static scratch scaling=%d call %d (%d layers)" % (scaling, k + 1, len(specs)))
        layers = _group(specs, scaling, rng)
        ref = _twin(layers, scaling)
        need = fg.gift_group_workspace_bytes(fg.OP_WHITEN_QUANTIZE, layers, scaling)
        assert 0 < need <= fg.gift_static_scratch_bytes()
        f_static = torch.zeros(1, dtype=torch.int32, device=DEV)
        f_ws = torch.zeros(1, dtype=torch.int32, device=DEV)
        fg.gift_whiten_quantize_static(layers, scaling=scaling, flags=f_static)
        fg.gift_whiten_quantize(ref, scaling=scaling, flags=f_ws)
        torch.cuda.synchronize()
        for L, R in zip(layers, ref):
            assert np.array_equal(host(L.q), host(R.q))
            assert np.array_equal(host(L.inv_scale).view(np.uint8), host(R.inv_scale).view(np.uint8))
            assert np.array_equal(host(L.W_out).view(np.uint32), host(R.W_out).view(np.uint32))
        assert int(host(f_static)[0]) == int(host(f_ws)[0])
        # the receive side takes the static call's payload like any other
        fg.gift_dequant_unwhiten(layers, scaling=scaling)
        fg.gift_dequant_unwhiten(ref, scaling=scaling)
        for L, R in zip(layers, ref):
            assert np.array_equal(host(L.G_hat).view(np.uint32), host(R.G_hat).view(np.uint32))


def test_static_scratch_refuses_a_group_beyond_the_array():
    say("static scratch size limit")
    _, f = _factor(1024, 17)
    G = torch.zeros(32768, 1024, device=DEV)
    L = fg.Layer(G, factor=f)
    need = fg.gift_group_workspace_bytes(fg.OP_WHITEN_QUANTIZE, [L], fg.SCALE_TENSOR)
    assert need > fg.gift_static_scratch_bytes()
    with pytest.raises(fg.GiftError) as e:
        fg.gift_whiten_quantize_static([L])
    assert e.value.status == 3
