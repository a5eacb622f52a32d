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
