"""Selective deployment: which layers get the GIFT transform.

The GIFT review (referee report, major comment 3; free-parameter ledger)
describes GIFT as applied only to the most numerically vulnerable layers
(13 fc2 layers of their 600M model, picked by a profiling score the pages do
not define).  The reading here: a layer's vulnerability is the anisotropy of
its input-side factor, rho = theta_1 / tr(A) (largest eigenvalue over trace,
both produced by the factor refresh); the k layers with the largest rho are
whitened and the rest use Euclidean FP8.  Layers sharing an input share rho;
ties go to the lower layer index.  Host logic run once per refresh (it reads
two scalars per factor from the device).
"""

import torch

from ._lib import COEF_TRACE


def anisotropy(factor):
    """rho = theta_1 / tr(A) of one device factor (one device->host copy)."""
    v = torch.stack([factor.theta[0], factor.coef[COEF_TRACE]]).double().cpu()
    th1, tr = float(v[0]), float(v[1])
    return th1 / tr if tr > 0 else 0.0


def rank_by_rho(rhos, k):
    """Indices of the k largest values of rhos (None = not eligible), ties by
    index, returned in increasing index order."""
    cand = [(-r, i) for i, r in enumerate(rhos) if r is not None]
    cand.sort()
    chosen = sorted(i for _, i in cand[:max(0, k)])
    return chosen


def select_layers(layer_factors, k):
    """layer_factors: per layer, its Factor or None (Euclidean-only layer).
    Returns the sorted indices of the k layers to whiten."""
    cache = {}
    rhos = []
    for f in layer_factors:
        if f is None:
            rhos.append(None)
            continue
        if id(f) not in cache:
            cache[id(f)] = anisotropy(f)
        rhos.append(cache[id(f)])
    return rank_by_rho(rhos, k)
