"""Layer selection: the host rule against the oracle's, and the oracle's
against hand-worked cases."""

import numpy as np
import pytest

from fac_whitening_gift_amd.select import rank_by_rho
from oracle import gift as og


def test_oracle_selection_hand_cases():
    assert og.select_top_k([0.1, 0.5, 0.3], 2) == [1, 2]
    assert og.select_top_k([0.2, 0.2, 0.2], 2) == [0, 1]          # ties to lower index
    assert og.select_top_k([None, 0.9, None, 0.1], 5) == [1, 3]   # k > eligible
    assert og.select_top_k([0.4, 0.9], 0) == []
    assert og.select_top_k([], 3) == []


def test_oracle_anisotropy_closed_form():
    U = np.linalg.qr(np.random.default_rng(0).standard_normal((64, 32)))[0]
    f = og.factor_from_parts(U, np.linspace(4, 1, 32), 0.1, trace=40.0)
    assert og.anisotropy(f) == 0.1


@pytest.mark.parametrize("seed", range(20))
def test_host_rule_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 30))
    rhos = [None if rng.random() < 0.2 else float(rng.integers(0, 6)) / 5 for _ in range(n)]
    for k in (0, 1, 3, 8, n, n + 4):
        assert rank_by_rho(rhos, k) == og.select_top_k(rhos, k)
