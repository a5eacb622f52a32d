"""The round trip captured in a HIP graph (torch.cuda.CUDAGraph over the
library's launches on the capture stream) and replayed: every replay, with
eager work and synchronisations in between, equals the eager calls bit for
bit, and a replay reads the live contents of G."""

import numpy as np
import pytest
import torch

import fac_whitening_gift_amd as fg
from oracle import gift as og
from gpu_util import DEV, say, to_dev, upload_factor

pytestmark = pytest.mark.gpu


def _factor(d_in, seed):
    rng = np.random.default_rng(seed)
    U = np.linalg.qr(rng.standard_normal((d_in, 32)))[0]
    theta = 40.0 * np.arange(1, 33, dtype=np.float64) ** -1.5
    return og.factor_from_parts(U, theta, 1e-2), U


def _layers(block):
    rng = np.random.default_rng(3)
    out = []
    for d_out, d_in, white in [(300, 256, True), (77, 384, True), (130, 256, True), (90, 512, False)]:
        f, U = _factor(d_in, d_in + d_out)
        G = (rng.standard_normal((d_out, d_in)) + 8 * rng.standard_normal((d_out, 32)) @ U.T)
        G = (G * np.exp(rng.standard_normal((d_out, 1)))).astype(np.float32)
        out.append((to_dev(G), upload_factor(f) if white else None))
    return out


def _snapshot(layers):
    torch.cuda.synchronize()
    return [(L.q.clone(), L.inv_scale.clone(), L.G_hat.clone()) for L in layers]


@pytest.mark.parametrize("block", [False, True])
def test_graph_replays_equal_eager(block):
    say("graph replay block=%s" % block)
    sc = fg.SCALE_BLOCK128 if block else fg.SCALE_TENSOR
    specs = _layers(block)
    white = [fg.Layer(G, factor=f, block128=block) for G, f in specs if f is not None]
    eucl = [fg.Layer(G, block128=block) for G, f in specs if f is None]
    calls = [fg.GroupCall(fg.OP_WHITEN_QUANTIZE, white, sc),
             fg.GroupCall(fg.OP_DEQUANT_UNWHITEN, white, sc),
             fg.GroupCall(fg.OP_EUCLID_ROUNDTRIP, eucl, sc)]
    for c in calls:
        c()
    ref = _snapshot(white + eucl)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the side stream, as capture requires
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for c in calls:
            c()
    err = fg.GroupCall(fg.OP_ROUNDTRIP_ERROR, white + eucl)
    for rep in range(3):
        for L in white + eucl:  # eager work between replays
            L.q.fill_(0x55)
            L.inv_scale.fill_(-1.0)
            L.G_hat.fill_(float("nan"))
        err()
        torch.cuda.synchronize()
        graph.replay()
        got = _snapshot(white + eucl)
        for (q0, i0, g0), (q1, i1, g1) in zip(ref, got):
            assert torch.equal(q0, q1) and torch.equal(i0, i1) and torch.equal(g0, g1), rep

    # a replay reads the current G: doubling every G doubles inv and G_hat,
    # and leaves the codes alone (the scale is a power of two apart)
    for G, _ in specs:
        G.mul_(2.0)
    graph.replay()
    got = _snapshot(white + eucl)
    for (q0, i0, g0), (q1, i1, g1) in zip(ref, got):
        assert torch.equal(q0, q1)
        assert torch.equal(i0 * 2, i1) and torch.equal(g0 * 2, g1)
