"""Device parity of the block-diagonal factor (block-A-32, block-A-64).

* refresh: S_i, S_i^-1 and each block's eigenvalues against the oracle's
  block factor of the device's own A (fp64 eigh per block), within 1e-5;
* round trip (per-tensor and 1x128): the whitened tensor within 1e-5 of the
  oracle's block product with the device's S; codes bit-exact against the
  oracle's quantization of the device's whitened tensor; G^ within 1e-5 of
  the oracle's un-whitening of the device's codes with the device's S^-1;
* grouped: one call over rank-32, block-32, block-64 and Euclidean layers
  gives each layer the codes and G^ of its own call;
* packs written by gift_prepare_factor from oracle values equal the
  refresh's.
"""

import numpy as np
import pytest
import torch

import synth
import fac_whitening_gift_amd as fg
from oracle import gift as og
from gpu_util import DEV, host, rel_fro, say

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _block_refresh(d, b, tokens=4096, seed=0, bf16=False):
    spec = synth.InputSpec("x", d, tokens, 1.5, bf16=bf16)
    inp = synth.draw_input(spec, seed=seed + d + b, as_bf16=bf16)
    f = fg.Factor(d, block=b)
    A = torch.empty(d, d, dtype=torch.float32, device=DEV)
    fg.gift_refresh_factor(inp["X"].to(DEV), f, A_out=A)
    torch.cuda.synchronize()
    return f, host(A).astype(np.float64), inp


def _gradient(d_out, inp, seed):
    return synth.draw_gradient(d_out, inp["Q"], inp["ev"], seed=seed).numpy()


@pytest.mark.parametrize("d,b", [(512, 32), (512, 64), (1024, 64), (192, 32)])
def test_block_refresh_matches_oracle(d, b):
    say("block refresh d=%d b=%d" % (d, b))
    f, A, _ = _block_refresh(d, b)
    bo = og.block_factor(A, b)
    S, Si, th = host(f.S), host(f.S_inv), host(f.theta)
    c = host(f.coef)
    assert abs(c[fg.COEF_LAMBDA_ISO] - bo.lambda_iso) <= 1e-5 * bo.lambda_iso
    assert abs(c[fg.COEF_TRACE] - bo.trace) <= 1e-5 * bo.trace
    for i in range(d // b):
        sl = slice(i * b, (i + 1) * b)
        assert rel_fro(S[sl], bo.S[sl]) <= TOL, i
        assert rel_fro(Si[sl], bo.S_inv[sl]) <= TOL, i
        assert np.allclose(th[sl], bo.theta[sl], rtol=1e-5, atol=1e-6 * bo.theta[sl][0])


def _roundtrip_parity(G, f, block128):
    sc = fg.SCALE_BLOCK128 if block128 else fg.SCALE_TENSOR
    Gd = torch.from_numpy(np.ascontiguousarray(G, dtype=np.float32)).to(DEV)
    W = torch.empty_like(Gd)
    L = fg.Layer(Gd, factor=f, W_out=W, block128=block128)
    fg.gift_whiten_quantize([L], scaling=sc)
    fg.gift_dequant_unwhiten([L], scaling=sc)
    S, Si = host(f.S), host(f.S_inv)
    Wg, q, inv, gh = host(W), host(L.q), host(L.inv_scale), host(L.G_hat)
    assert rel_fro(Wg, og.block_apply(G, S)) <= TOL
    codes, inv_o, _ = og.quantize(Wg, block128)
    assert np.array_equal(q, codes)
    assert np.array_equal(inv.reshape(np.shape(inv_o)), inv_o)
    ref = og.block_apply(og.dequantize(q, inv.reshape(np.shape(inv_o)), block128), Si)
    assert rel_fro(gh, ref) <= TOL
    # the production instantiation (no W_out) writes the same codes
    L2 = fg.Layer(Gd, factor=f, block128=block128)
    fg.gift_whiten_quantize([L2], scaling=sc)
    assert np.array_equal(host(L2.q), q)
    return q, gh


@pytest.mark.parametrize("d_out,d_in,b,block128", [
    (256, 512, 32, False), (256, 512, 32, True), (256, 512, 64, False), (256, 512, 64, True),
    (37, 512, 32, False), (37, 512, 64, True), (129, 128, 64, False), (700, 384, 64, True),
    (300, 192, 32, False), (1, 64, 64, False)])
def test_block_roundtrip_parity(d_out, d_in, b, block128):
    say("block round trip %dx%d b=%d block128=%s" % (d_out, d_in, b, block128))
    f, _, inp = _block_refresh(d_in, b, tokens=2048, seed=d_out)
    G = _gradient(d_out, inp, seed=d_out + 1)
    _roundtrip_parity(G, f, block128)


def test_block_end_to_end_close_to_independent_oracle():
    """The independent oracle pipeline from X (fp64 A, eigh per block) lands on
    the same reconstruction error (code flips allowed)."""
    say("block end to end d=512 b=64")
    f, A, inp = _block_refresh(512, 64, tokens=4096, seed=7)
    G = _gradient(256, inp, seed=8)
    _, gh = _roundtrip_parity(G, f, False)
    bo = og.block_factor(og.covariance(inp["X"].numpy()), 64)
    _, _, _, gh_o, _ = og.block_roundtrip(G, bo)
    e_dev, e_orc = og.rel_frobenius(G, gh), og.rel_frobenius(G, gh_o)
    assert abs(e_dev / e_orc - 1) < 1e-2


def test_grouped_mixed_factor_kinds():
    say("grouped rank-32 + block-32 + block-64 + Euclid")
    d = 512
    spec = synth.InputSpec("x", d, 2048, 1.5, bf16=False)
    inp = synth.draw_input(spec, seed=99)
    X = inp["X"].to(DEV)
    f32 = fg.Factor(d)
    fg.gift_refresh_factor(X, f32)
    fb = {b: fg.Factor(d, block=b) for b in (32, 64)}
    for b in (32, 64):
        fg.gift_refresh_factor(X, fb[b])
    Gs = [torch.from_numpy(_gradient(n, inp, seed=n)).to(DEV) for n in (64, 100, 129, 77, 200)]
    facs = [f32, fb[32], fb[64], None, fb[32]]
    for block128 in (False, True):
        sc = fg.SCALE_BLOCK128 if block128 else fg.SCALE_TENSOR
        grouped = [fg.Layer(G, factor=f, block128=block128) for G, f in zip(Gs, facs)]
        fg.gift_whiten_quantize(grouped, scaling=sc)
        fg.gift_dequant_unwhiten(grouped, scaling=sc)
        for L in grouped:
            one = fg.Layer(L.G, factor=L.factor, block128=block128)
            if L.factor is None:
                fg.gift_euclid_fp8_roundtrip([one], scaling=sc)
            else:
                fg.gift_whiten_quantize([one], scaling=sc)
                fg.gift_dequant_unwhiten([one], scaling=sc)
            assert np.array_equal(host(L.q), host(one.q))
            assert np.array_equal(host(L.inv_scale), host(one.inv_scale))
            if L.factor is not None:
                assert np.array_equal(host(L.G_hat), host(one.G_hat))


def test_prepare_factor_packs_match_refresh():
    say("block packs from gift_prepare_factor")
    f, _, inp = _block_refresh(256, 64, tokens=2048, seed=5)
    g = fg.Factor(256, U=f.U.clone(), theta=f.theta.clone(), coef=f.coef.clone(), block=64)
    fg.gift_prepare_factor(g)
    assert torch.equal(g.packs, f.packs)


def test_grouped_block_refresh_chain():
    """Eighteen block-32 factors (widths 128, 192, 256; bf16 and fp32
    inputs) in one refresh call, so the eigensolve runs over the whole call
    with its descriptors in the workspace and the packs go out in two
    groups: each factor against the oracle's block factor of the device's A,
    its packs equal to gift_prepare_factor's."""
    dims = [128, 192, 256]
    items = []
    for k in range(18):
        d = dims[k % 3]
        bf16 = k % 4 != 1
        spec = synth.InputSpec("b%d" % k, d, 1500 + 100 * k, 1.5, bf16=bf16)
        inp = synth.draw_input(spec, seed=500 + k, as_bf16=bf16)
        A = torch.empty(d, d, dtype=torch.float32, device=DEV)
        items.append(dict(X=inp["X"].to(DEV), factor=fg.Factor(d, block=32), A_out=A))
    say("grouped block-32 refresh: %d inputs" % len(items))
    fg.gift_refresh_factors(items)
    torch.cuda.synchronize()
    for k, it in enumerate(items):
        f = it["factor"]
        d = f.d_in
        bo = og.block_factor(host(it["A_out"]).astype(np.float64), 32)
        S, Si, th = host(f.S), host(f.S_inv), host(f.theta)
        for i in range(d // 32):
            sl = slice(i * 32, (i + 1) * 32)
            assert rel_fro(S[sl], bo.S[sl]) <= TOL, (k, i)
            assert rel_fro(Si[sl], bo.S_inv[sl]) <= TOL, (k, i)
            assert np.allclose(th[sl], bo.theta[sl], rtol=1e-5, atol=1e-6 * bo.theta[sl][0]), (k, i)
        g = fg.Factor(d, U=f.U.clone(), theta=f.theta.clone(), coef=f.coef.clone(), block=32)
        fg.gift_prepare_factor(g)
        assert torch.equal(g.packs, f.packs), k
