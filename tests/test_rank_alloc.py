"""The library's adaptive rank allocation (host code, no GPU) against the oracle's
exact dynamic programme: the kept energy is unique and must agree; the ranks must be a
valid allocation (multiples of the granule, within [r_min, r_max], within the budget)
that keeps that energy.  Allocations that tie may differ."""
import numpy as np
import pytest

import kv_cache_cross_amd as xk
import oracle


def _check(spectra, budget, granule, r_min, r_max):
    ranks, kept = xk.rank_allocate(spectra, budget, granule, r_min, r_max)
    ref_ranks, ref_kept = oracle.allocate_ranks(spectra, budget, granule, r_min, r_max)
    assert sum(ranks) <= budget
    assert all(r_min <= r <= r_max and r % granule == 0 for r in ranks)
    mine = sum(float(np.sum(np.clip(l[:r], 0, None))) for l, r in zip(spectra, ranks))
    assert kept == pytest.approx(mine, rel=1e-12)
    assert kept == pytest.approx(ref_kept, rel=1e-12)
    return ranks, ref_ranks


def test_hand_case():
    ranks, _ = _check([np.array([10.0, 1, 1, 1]), np.array([5.0, 4, 3, 2])], 4, 1, 0, 4)
    assert ranks == [1, 3]


@pytest.mark.parametrize("seed", range(8))
def test_random_spectra(seed):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 17))
    granule = int(rng.choice([1, 8, 128]))
    kmax = int(rng.integers(2, 9))
    r_max = granule * kmax
    r_min = granule * int(rng.integers(0, 2))
    spectra = [np.sort(rng.exponential(size=r_max) ** rng.uniform(1, 4) * rng.uniform(0.1, 10))[::-1]
               for _ in range(S)]
    for budget in (S * r_min, S * r_min + granule * 3, S * (r_min + r_max) // 2, S * r_max, S * r_max + 7):
        _check(spectra, budget, granule, r_min, r_max)


def test_equal_spectra_uniform_and_validation():
    lam = 1.0 / np.arange(1, 1025) ** 0.8
    ranks, _ = _check([lam] * 16, 16 * 512, 128, 128, 1024)
    assert ranks == [512] * 16
    for bad in [dict(budget=100), dict(granule=0), dict(r_min=100), dict(r_max=1000)]:
        kw = dict(budget=16 * 512, granule=128, r_min=128, r_max=1024)
        kw.update(bad)
        with pytest.raises(xk.XkvError):
            xk.rank_allocate([lam] * 16, **kw)
