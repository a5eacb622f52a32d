"""Device parity of the round trip: the HIP path through the C ABI against the
oracle, element by element.

Protocol: (a) the whitened fp32 tensor within 1e-5 relative Frobenius of the
oracle's fp64 whitening of the same G with the factor values the device
holds; (b) codes and inverse scale bit-exact against the oracle's E4M3
encoding of the device's own whitened tensor; (c) the reconstruction within
1e-5 of the oracle's un-whitening of the device's codes; the Euclidean
baseline and every E4M3 decision bit-exact.
"""

import numpy as np
import pytest
import torch

import synth
import fac_whitening_gift_amd as fg
from oracle import e4m3
from oracle import gift as og
from gpu_util import DEV, factor_host, host, rel_fro, say, to_dev, upload_factor

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _factor_for(d_in, seed, tokens=2048, exponent=1.5):
    spec = synth.InputSpec("x", d_in, tokens, exponent, bf16=False)
    inp = synth.draw_input(spec, seed=seed)
    omega = synth.gaussian_sketch(d_in, og.SKETCH_WIDTH, seed=seed + 1).numpy()
    f = og.refresh_factor(inp["X"].numpy(), omega)
    return inp, f


def _gradient(d_out, inp, seed):
    return synth.draw_gradient(d_out, inp["Q"], inp["ev"], seed=seed).numpy()


# --------------------------------------------------------------------------- codec

def _codec_values():
    t = e4m3.decode_table()
    pos = t[:0x7F]
    vals = [pos, -pos]
    mids = (pos[:-1] + pos[1:]) / 2
    m32 = mids.astype(np.float32)
    vals += [mids, -mids,
             np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(-np.inf)),
             -np.nextafter(m32, np.float32(np.inf))]
    rng = np.random.default_rng(0)
    mags = np.exp2(rng.uniform(-16, np.log2(448), size=60_000))
    vals += [mags * rng.choice([-1, 1], size=mags.size)]
    vals += [np.array([0.0, -0.0, 1e-40, -1e-40, 1e-45, 2.0 ** -10, -(2.0 ** -10), 447.99, 448.0])]
    v = np.concatenate([np.asarray(x, dtype=np.float32).ravel() for x in vals])
    pad = (-v.size) % 128
    v = np.concatenate([v, np.zeros(pad, dtype=np.float32)])
    return v.reshape(-1, 128)


def test_e4m3_hardware_codec_matches_oracle():
    """amax = 448 makes scale = inv = 1, so codes are E4M3(G) and G^ = decode."""
    say("euclid codec sweep")
    G = _codec_values()
    assert np.abs(G).max() == 448.0
    L = fg.Layer(to_dev(G))
    fg.gift_euclid_fp8_roundtrip([L])
    q, inv, gh = host(L.q), host(L.inv_scale), host(L.G_hat)
    assert inv[0] == 1.0
    ref = e4m3.encode(G)
    bad = np.flatnonzero(q.ravel() != ref.ravel())
    assert bad.size == 0, "first mismatches: %s" % [
        (float(G.ravel()[i]), hex(q.ravel()[i]), hex(ref.ravel()[i])) for i in bad[:8]]
    dec = e4m3.decode(ref)
    assert np.array_equal(gh.view(np.uint32), dec.view(np.uint32))


def test_nonfinite_and_zero_tensors():
    say("euclid nonfinite / zero")
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    G = np.ones((4, 128), dtype=np.float32)
    G[1, 5] = np.nan
    L = fg.Layer(to_dev(G))
    fg.gift_euclid_fp8_roundtrip([L], flags=flags)
    codes, inv, fl = og.quantize_tensor(G)
    assert np.array_equal(host(L.q), codes) and np.isnan(host(L.inv_scale)[0])
    assert int(host(flags)[0]) == og.FLAG_NONFINITE
    G[1, 5] = -np.inf
    flags.zero_()
    L = fg.Layer(to_dev(G))
    fg.gift_euclid_fp8_roundtrip([L], flags=flags)
    codes, inv, fl = og.quantize_tensor(G)
    assert np.array_equal(host(L.q), codes) and np.isinf(host(L.inv_scale)[0])
    assert int(host(flags)[0]) == og.FLAG_NONFINITE
    Z = np.zeros((3, 64), dtype=np.float32)
    Z[2, 7] = -0.0
    flags.zero_()
    L = fg.Layer(to_dev(Z))
    fg.gift_euclid_fp8_roundtrip([L], flags=flags)
    codes, inv, fl = og.quantize_tensor(Z)
    assert np.array_equal(host(L.q), codes) and host(L.inv_scale)[0] == 1.0
    assert int(host(flags)[0]) == og.FLAG_ZERO_AMAX


# --------------------------------------------------------------------------- Euclid

@pytest.mark.parametrize("shape,block", [((256, 512), False), ((256, 512), True),
                                         ((37, 100), False), ((1, 4), False),
                                         ((3, 128), True), ((1031, 1024), False),
                                         ((1031, 1024), True)])
def test_euclid_bit_exact(shape, block):
    say("euclid %s block=%s" % (shape, block))
    rng = np.random.default_rng(shape[0])
    G = (rng.standard_normal(shape) * np.exp(rng.standard_normal((shape[0], 1)))).astype(np.float32)
    L = fg.Layer(to_dev(G), block128=block)
    sc = fg.SCALE_BLOCK128 if block else fg.SCALE_TENSOR
    fg.gift_euclid_fp8_roundtrip([L], scaling=sc)
    codes, inv, gh, _ = og.euclid_roundtrip(G, block128=block)
    assert np.array_equal(host(L.q), codes)
    assert np.array_equal(host(L.inv_scale).reshape(np.shape(inv)), inv)
    assert np.array_equal(host(L.G_hat), gh)
    # send / receive halves through the grouped entry points give the same
    L2 = fg.Layer(to_dev(G), block128=block)
    fg.gift_whiten_quantize([L2], scaling=sc)
    fg.gift_dequant_unwhiten([L2], scaling=sc)
    assert np.array_equal(host(L2.q), codes)
    assert np.array_equal(host(L2.G_hat), gh)


# --------------------------------------------------------------------------- GIFT

def _gift_parity(G, df, block):
    sc = fg.SCALE_BLOCK128 if block else fg.SCALE_TENSOR
    Gd = to_dev(G)
    W = torch.empty_like(Gd)
    L = fg.Layer(Gd, factor=df, W_out=W, block128=block)
    fg.gift_whiten_quantize([L], scaling=sc)
    fg.gift_dequant_unwhiten([L], scaling=sc)
    U, alpha, beta, dw, du = factor_host(df)
    Wg, q, inv, gh = host(W), host(L.q), host(L.inv_scale), host(L.G_hat)
    # (a) whitened tensor
    assert rel_fro(Wg, og.whiten_with(G, U, alpha, dw)) <= TOL
    # (b) codes of the device's own whitened tensor
    codes, inv_o, _ = og.quantize(Wg, block)
    assert np.array_equal(q, codes)
    assert np.array_equal(inv.reshape(np.shape(inv_o)), inv_o)
    # (c) reconstruction from the device's codes
    ref = og.unwhiten_with(og.dequantize(q, inv.reshape(np.shape(inv_o)), block), U, beta, du)
    assert rel_fro(gh, ref) <= TOL
    # the production instantiation (no W_out) writes the same codes
    L2 = fg.Layer(Gd, factor=df, block128=block)
    fg.gift_whiten_quantize([L2], scaling=sc)
    assert np.array_equal(host(L2.q), q)
    # error sums against the oracle's fp64 sums of the same tensors
    err = host(fg.gift_roundtrip_error([L]))
    e, gsum = og.error_sums(G, gh)
    assert abs(err[0, 0] - e) <= 1e-12 * e and abs(err[0, 1] - gsum) <= 1e-12 * gsum
    return q, gh


@pytest.mark.parametrize("d_out,d_in,block", [(256, 512, False), (256, 512, True),
                                              (37, 512, False), (37, 512, True),
                                              (1, 64, False), (129, 128, True),
                                              (200, 1024, False), (300, 96, False),
                                              (513, 160, False), (700, 384, True)])
def test_gift_parity(d_out, d_in, block):
    say("gift parity %dx%d block=%s" % (d_out, d_in, block))
    inp, f = _factor_for(d_in, seed=d_in + 3)
    G = _gradient(d_out, inp, seed=d_out)
    _gift_parity(G, upload_factor(f), block)


def _cheap_factor(d_in, seed):
    """A factor with a random orthonormal U and a power-law theta, for row
    lengths where the oracle's full refresh would take minutes."""
    rng = np.random.default_rng(seed)
    U = np.linalg.qr(rng.standard_normal((d_in, 32)))[0]
    theta = 50.0 * np.arange(1, 33, dtype=np.float64) ** -1.5
    return og.factor_from_parts(U, theta, 1e-2), U


@pytest.mark.parametrize("d_out,d_in,block", [(48, 4096, False), (40, 4096, True),
                                              (24, 8448, False), (20, 8448, True),
                                              (32784, 64, False)])
def test_gift_parity_long_and_tall(d_out, d_in, block):
    """Rows longer than the chunks a wave keeps in registers (part of the row
    is read twice), and a layer with more strips than the quantize pass
    reduces itself (its amax goes through one reduction workgroup)."""
    say("gift parity long/tall %dx%d block=%s" % (d_out, d_in, block))
    f, U = _cheap_factor(d_in, seed=d_in + d_out)
    rng = np.random.default_rng(d_out)
    Z = rng.standard_normal((d_out, d_in))
    G = (np.exp(rng.standard_normal((d_out, 1))) *
         (Z + 10.0 * rng.standard_normal((d_out, 32)) @ U.T)).astype(np.float32)
    _gift_parity(G, upload_factor(f), block)


def test_gift_end_to_end_close_to_independent_oracle():
    """The oracle's own pipeline from G (fp64 whitening, its own rounding)
    agrees with the device to a few code flips."""
    say("gift end-to-end single layer")
    inp, f = _factor_for(512, seed=21, tokens=4096)
    G = _gradient(256, inp, seed=22)
    df = upload_factor(f)
    q, gh = _gift_parity(G, df, False)
    codes, inv, W32, gh_o, _ = og.gift_roundtrip(G, og.factor_from_parts(*_parts(df)))
    flips = np.count_nonzero(codes != q)
    assert flips <= max(2, 1e-4 * q.size)
    assert abs(og.rel_frobenius(G, gh) - og.rel_frobenius(G, gh_o)) <= 1e-3 * og.rel_frobenius(G, gh_o)


def _parts(df):
    U = df.U.cpu().numpy().astype(np.float64)
    c = df.coef.cpu().numpy().astype(np.float64)
    return U, df.theta.cpu().numpy().astype(np.float64), c[fg.COEF_LAMBDA_ISO]


def test_isotropic_factor_gives_euclid_codes():
    """Theta = 0, lambda_iso = 4^-3: whitening multiplies by 8 exactly, so the
    device's GIFT codes equal its Euclidean codes bit for bit."""
    say("gift isotropic factor")
    d_in = 256
    U = np.linalg.qr(np.random.default_rng(5).standard_normal((d_in, 32)))[0]
    f = og.factor_from_parts(U, np.zeros(32), 4.0 ** -3)
    df = upload_factor(f)
    G = np.random.default_rng(6).standard_normal((64, d_in)).astype(np.float32)
    Gd = to_dev(G)
    Lg, Le = fg.Layer(Gd, factor=df), fg.Layer(Gd)
    fg.gift_whiten_quantize([Lg])
    fg.gift_euclid_fp8_roundtrip([Le])
    assert np.array_equal(host(Lg.q), host(Le.q))
    assert host(Lg.inv_scale)[0] == 8 * host(Le.inv_scale)[0]


def test_grouped_launch_over_many_mixed_layers():
    """20 layers (more than one launch chunk), whitened and Euclidean mixed,
    ragged shapes: the grouped call equals one call per layer bit for bit."""
    say("grouped mixed 20 layers")
    rng = np.random.default_rng(9)
    inp_a, fa = _factor_for(256, seed=31)
    inp_b, fb = _factor_for(384, seed=32)
    da, db = upload_factor(fa), upload_factor(fb)
    specs = []
    for i in range(20):
        kind = i % 3
        d_out = int(rng.integers(1, 300))
        if kind == 0:
            specs.append((_gradient(d_out, inp_a, 100 + i), da))
        elif kind == 1:
            specs.append((_gradient(d_out, inp_b, 100 + i), db))
        else:
            specs.append((rng.standard_normal((d_out, 128)).astype(np.float32), None))
    for block in (False, True):
        sc = fg.SCALE_BLOCK128 if block else fg.SCALE_TENSOR
        # W_out on every other layer only: a launch writes W for exactly those
        group = []
        for i, (G, f) in enumerate(specs):
            Gd = to_dev(G)
            group.append(fg.Layer(Gd, factor=f, block128=block,
                                  W_out=torch.full_like(Gd, 7.0) if i % 2 else None))
        fg.gift_whiten_quantize(group, scaling=sc)
        fg.gift_dequant_unwhiten(group, scaling=sc)
        err = host(fg.gift_roundtrip_error(group))
        for i, (G, f) in enumerate(specs):
            one = fg.Layer(to_dev(G), factor=f, block128=block)
            fg.gift_whiten_quantize([one], scaling=sc)
            fg.gift_dequant_unwhiten([one], scaling=sc)
            assert np.array_equal(host(group[i].q), host(one.q)), i
            assert np.array_equal(host(group[i].G_hat), host(one.G_hat)), i
            if i % 2:
                Wg = host(group[i].W_out)
                if f is None:
                    assert np.array_equal(Wg, G), i
                else:
                    U, alpha, _, dw, _ = factor_host(f)
                    assert rel_fro(Wg, og.whiten_with(G, U, alpha, dw)) <= TOL, i
            e, gs = og.error_sums(G, host(one.G_hat))
            assert abs(err[i, 0] - e) <= 1e-12 * max(e, 1e-300) and abs(err[i, 1] - gs) <= 1e-12 * gs
        # Euclidean layers of the group also match the oracle exactly
        for i, (G, f) in enumerate(specs):
            if f is None:
                codes, inv, gh, _ = og.euclid_roundtrip(G, block128=block)
                assert np.array_equal(host(group[i].q), codes)
                assert np.array_equal(host(group[i].G_hat), gh)


# --------------------------------------------------------------------------- full size

@pytest.fixture(scope="module")
def block_1024():
    """One Llama-style block at hidden 1024 (q,k,v,o 1024^2, gate/up 2816x1024,
    down 1024x2816), factors from the oracle (8192 bf16 tokens per input)."""
    w = synth.llama_block()
    facs, grads = {}, []
    for k, spec in enumerate(w.inputs):
        inp = synth.draw_input(spec, seed=500 + k)
        omega = synth.gaussian_sketch(spec.d_in, og.SKETCH_WIDTH, seed=600 + k).numpy()
        facs[spec.name] = (inp, og.refresh_factor(inp["X"].numpy(), omega))
    for i, l in enumerate(w.layers):
        inp, f = facs[l.input]
        grads.append((l, _gradient(l.d_out, inp, 700 + i), f))
    return grads


@pytest.mark.parametrize("block", [False, True])
def test_full_block_grouped_parity(block_1024, block):
    say("gift full block hidden 1024 grouped block=%s" % block)
    sc = fg.SCALE_BLOCK128 if block else fg.SCALE_TENSOR
    dfs = {}
    layers = []
    for l, G, f in block_1024:
        if l.input not in dfs:
            dfs[l.input] = upload_factor(f)
        Gd = to_dev(G)
        layers.append(fg.Layer(Gd, factor=dfs[l.input], W_out=torch.empty_like(Gd), block128=block))
    fg.gift_whiten_quantize(layers, scaling=sc)
    fg.gift_dequant_unwhiten(layers, scaling=sc)
    err = host(fg.gift_roundtrip_error(layers))
    for i, ((l, G, f), L) in enumerate(zip(block_1024, layers)):
        U, alpha, beta, dw, du = factor_host(L.factor)
        Wg, q, inv, gh = host(L.W_out), host(L.q), host(L.inv_scale), host(L.G_hat)
        assert rel_fro(Wg, og.whiten_with(G, U, alpha, dw)) <= TOL, l.name
        codes, inv_o, _ = og.quantize(Wg, block)
        assert np.array_equal(q, codes), l.name
        assert np.array_equal(inv.reshape(np.shape(inv_o)), inv_o), l.name
        ref = og.unwhiten_with(og.dequantize(q, inv_o, block), U, beta, du)
        assert rel_fro(gh, ref) <= TOL, l.name
        e, gs = og.error_sums(G, gh)
        assert abs(err[i, 0] - e) <= 1e-12 * e


def test_factor_packs_and_workspace_packing_agree():
    """A factor carrying its operand packs and one without (packed into the
    workspace on every call) give identical codes and reconstructions."""
    say("packs vs workspace packing")
    inp, f = _factor_for(512, seed=71)
    G = _gradient(100, inp, seed=72)
    with_p = upload_factor(f)
    without = fg.Factor(512, U=with_p.U, theta=with_p.theta, coef=with_p.coef, packs=False)
    assert without.packs is None
    for block in (False, True):
        sc = fg.SCALE_BLOCK128 if block else fg.SCALE_TENSOR
        La = fg.Layer(to_dev(G), factor=with_p, block128=block)
        Lb = fg.Layer(to_dev(G), factor=without, block128=block)
        for L in (La, Lb):
            fg.gift_whiten_quantize([L], scaling=sc)
            fg.gift_dequant_unwhiten([L], scaling=sc)
        assert np.array_equal(host(La.q), host(Lb.q))
        assert np.array_equal(host(La.G_hat), host(Lb.G_hat))
