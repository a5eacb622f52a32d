"""The staleness study at a small scale: the factor from step 0 loses its
advantage as the eigenbasis rotates; a fresh factor keeps it; Euclidean FP8
is unaffected."""

import argparse

import numpy as np
import pytest

import bench
from gpu_util import say

pytestmark = pytest.mark.gpu


def test_staleness_small():
    say("staleness study hidden 256 mlp 512, 6 steps of 0.15 rad")
    args = argparse.Namespace(blocks=1, hidden=256, mlp=512, tokens=4096, angle=0.15,
                              study_steps=6, quiet=True)
    out = bench.staleness_study(args)
    rows = out["rows"]
    assert len(rows) == 6
    r0, r5 = rows[0], rows[-1]
    # at t = 0 the stale factor is the fresh one
    assert abs(r0["m2_stale_tensor"] - r0["m2_fresh_tensor"]) <= 1e-6
    # GIFT beats Euclid in the K-FAC metric while fresh
    for r in rows:
        assert r["m2_fresh_tensor"] < 0.7 * r["m2_euclid_tensor"]
        assert r["m2_fresh_b128"] < 0.8 * r["m2_euclid_b128"]
    # the stale factor degrades with the rotation
    assert r5["m2_stale_tensor"] > 1.5 * r0["m2_stale_tensor"]
    assert np.all(np.diff([r["m2_stale_tensor"] for r in rows]) > -1e-3)


def test_interval_small():
    say("interval study hidden 256 mlp 512, K in 1,2,4 over 8 steps of 0.15 rad")
    args = argparse.Namespace(blocks=1, hidden=256, mlp=512, tokens=4096, angle=0.15,
                              study_steps=8, intervals="1,2,4", quiet=True)
    out = bench.interval_study(args)
    rows = {r["K"]: r for r in out["rows"]}
    assert [rows[k]["refreshes"] for k in (1, 2, 4)] == [8, 4, 2]
    # refreshing every step keeps GIFT's advantage in the K-FAC metric
    assert rows[1]["m2_mean"] < 0.7 * out["euclid"]["m2_mean"]
    # a longer interval means staler factors on a rotating eigenbasis
    assert rows[1]["m2_mean"] <= rows[2]["m2_mean"] + 1e-4
    assert rows[2]["m2_mean"] <= rows[4]["m2_mean"] + 1e-4
    assert rows[4]["m2_worst"] >= rows[1]["m2_worst"]
    assert out["refresh_ms"] > 0 and rows[4]["refresh_ms_per_step"] < rows[1]["refresh_ms_per_step"]


def test_reference_study_small():
    """Full-rank input-side whitening beats the rank-32 factor, which beats
    Euclidean FP8, in the input-side K-FAC metric; the Cholesky form and the
    two-sided transform also beat Euclid."""
    say("reference study hidden 256 mlp 512 tokens 4096")
    args = argparse.Namespace(ref_shape="256,512,4096", quiet=True)
    rows = bench.reference_study(args)["rows"]
    assert rows["input_full"]["m2"] < rows["gift_rank32"]["m2"] < rows["euclid"]["m2"]
    assert rows["input_cholesky"]["m2"] < rows["euclid"]["m2"]
    assert rows["two_sided"]["m2"] < rows["euclid"]["m2"]


def test_staleness_values_match_oracle():
    """The study's M2 at step 1 against the oracle on the same seeded inputs:
    the factors from the oracle's refresh (its own Philox sketch of the seeds
    the device uses), the oracle's round trips, and the metric
    (C_t + lambda I)^-1/2 of the population covariance C_t = Q_t diag(ev) Q_t^T
    by the oracle's eigendecomposition instead of the study's closed form;
    M2 pooled over the layers as the study pools it.  Euclidean codes are the
    same on both sides, so its M2 agrees to rounding; the GIFT factors differ
    by fp32 against fp64, which can move a few codes (measured: 2e-5
    relative).  The interval study runs the same refresh and error helpers."""
    import torch

    import synth
    from oracle import gift as og
    from oracle import philox

    say("staleness values vs oracle, hidden 256 mlp 512, 2 steps of 0.15 rad")
    args = argparse.Namespace(blocks=1, hidden=256, mlp=512, tokens=4096, angle=0.15,
                              study_steps=2, quiet=True)
    out = bench.staleness_study(args)
    row = out["rows"][1]
    dev = torch.device("cuda:0")
    w, base, rots = bench._rotating_block(args, dev)
    stale, fresh, S = {}, {}, {}
    for t in (0, 1):
        Qt, X = bench._inputs_at(w, base, rots, t, args.angle, dev)
        for k, spec in enumerate(w.inputs):
            Xh = X[spec.name]["X"].float().cpu().numpy()
            f = og.refresh_factor(Xh, philox.gaussian_sketch(spec.d_in, 64, k))
            if t == 0:
                stale[spec.name] = f
            else:
                fresh[spec.name] = f
                ev = X[spec.name]["ev"].double().cpu().numpy()
                Q = Qt[spec.name].double().cpu().numpy()
                lam = 1e-3 * ev.sum() / spec.d_in
                S[spec.name] = og.metric_sqrt_inv((Q * ev) @ Q.T, lam)
    num = {"euclid": 0.0, "stale": 0.0, "fresh": 0.0}
    den = 0.0
    for i, l in enumerate(w.layers):
        G = synth.draw_gradient(l.d_out, Qt[l.input], X[l.input]["ev"], seed=9000 + 100 + i,
                                device=dev).cpu().numpy().astype(np.float64)
        M = S[l.input]
        den += np.linalg.norm(G @ M) ** 2
        for m, G_hat in (("euclid", og.euclid_roundtrip(G)[2]),
                         ("stale", og.gift_roundtrip(G, stale[l.input])[3]),
                         ("fresh", og.gift_roundtrip(G, fresh[l.input])[3])):
            num[m] += np.linalg.norm((np.asarray(G_hat, dtype=np.float64) - G) @ M) ** 2
    m2 = {m: np.sqrt(v / den) for m, v in num.items()}
    say("M2 study %s, oracle %s" % ({m: row["m2_%s_tensor" % m] for m in m2},
                                    {m: round(float(v), 6) for m, v in m2.items()}))
    assert abs(row["m2_euclid_tensor"] - m2["euclid"]) <= 1e-4 * m2["euclid"]
    for m in ("stale", "fresh"):
        assert abs(row["m2_%s_tensor" % m] - m2[m]) <= 1e-3 * m2[m], (m, row, m2)
