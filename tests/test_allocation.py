"""Sparsity allocation (technical summary, Sparsity Allocation): the oracle's
reading pinned by hand-worked cases and invariants, and the library's
host-only C implementation checked against it.  No GPU needed."""
import numpy as np
import pytest

import oracle
import free_sparse_swiglu_stage1_amd as P


# A proportional model worked by hand: the proxy costs 20% of the dense layer
# at full keep, Stage 2 costs the dense layer times the kept fraction.
#   E(keep, s) = 1 - (20 keep + 100 (1 - s)) / 100
HAND = (0.0, 20.0, 0.0, 100.0, 100.0)


@pytest.mark.parametrize("target,keep,sp", [
    (0.5, 1.0, 0.7),    # 1 - (20 + 30)/100: the anchor with every input
    (0.6, 0.5, 0.7),    # 20 keep = 10
    (0.55, 0.75, 0.7),  # 20 keep = 15
    (0.4, 1.0, 0.6),    # slack: keep 1, 100 kappa = 40
    (0.65, 0.3, 0.71),  # keep floor: 6 + 100 kappa = 35
    (0.0, 1.0, 0.2),    # 20 + 100 kappa = 100
    (-1.0, 1.0, 0.0),   # more than dense allowed: every channel
])
def test_oracle_hand_cases(target, keep, sp):
    k, s = oracle.allocate_sparsity(HAND, target)
    assert abs(k - keep) < 1e-12 and abs(s - sp) < 1e-12


def test_oracle_unreachable_and_zero_slope():
    # the most this model can skip: keep 0.3, every channel dropped -> E = 0.94
    assert oracle.allocate_sparsity(HAND, 0.94) is not None
    assert oracle.allocate_sparsity(HAND, 0.9401) is None
    # a keep-independent Stage 1 keeps every input and sets the sparsity from the budget
    k, s = oracle.allocate_sparsity((5.0, 0.0, 2.0, 50.0, 100.0), 0.5)
    assert k == 1.0 and abs(s - (1.0 - (50.0 - 5.0 - 2.0) / 50.0)) < 1e-12


def test_oracle_meets_the_target_and_is_monotone():
    rng = np.random.default_rng(41)
    for _ in range(200):
        m = (rng.uniform(0, 10), rng.uniform(0, 30), rng.uniform(0, 10), rng.uniform(20, 80), rng.uniform(80, 120))
        prev = None
        for t in np.linspace(-0.2, 0.95, 24):
            r = oracle.allocate_sparsity(m, t)
            if r is None:
                continue
            k, s = r
            assert 0.3 - 1e-12 <= k <= 1.0 + 1e-12 and 0.0 <= s <= 1.0
            e = oracle.effective_sparsity(m, k, s)
            assert e >= t - 1e-9                     # the budget is met ...
            if 0.0 < s < 1.0:
                assert abs(e - t) < 1e-9             # ... exactly, unless a bound binds
            if prev is not None:                     # a higher target never keeps more
                assert k <= prev[0] + 1e-12 and s >= prev[1] - 1e-12
            prev = (k, s)


def test_library_matches_oracle():
    rng = np.random.default_rng(42)
    for _ in range(400):
        m = (rng.uniform(0, 10), rng.uniform(0, 30) * (rng.random() > 0.1), rng.uniform(0, 10),
             rng.uniform(20, 80), rng.uniform(80, 120))
        t = rng.uniform(-0.3, 0.99)
        anchor, min_keep = rng.uniform(0.4, 0.9), rng.uniform(0.1, 0.6)
        want = oracle.allocate_sparsity(m, t, anchor, min_keep)
        got = P.allocate_sparsity(m, t, anchor, min_keep)
        if want is None:
            assert got is None
        else:
            assert abs(got[0] - want[0]) < 1e-12 and abs(got[1] - want[1]) < 1e-12
        k, s = rng.uniform(0, 1), rng.uniform(0, 1)
        assert abs(P.effective_sparsity(m, k, s) - oracle.effective_sparsity(m, k, s)) < 1e-12


def test_library_rejects_bad_models():
    for m in ((0.0, 20.0, 0.0, 0.0, 100.0), (0.0, 20.0, 0.0, 100.0, 0.0), (-1.0, 20.0, 0.0, 100.0, 100.0)):
        with pytest.raises(P.ProxError):
            P.allocate_sparsity(m, 0.5)
    with pytest.raises(P.ProxError):
        P.allocate_sparsity(HAND, 1.0)
    with pytest.raises(P.ProxError):
        P.allocate_sparsity(HAND, 0.5, s2_anchor=1.5)
    with pytest.raises(P.ProxError):
        P.effective_sparsity(HAND, 1.5, 0.7)
