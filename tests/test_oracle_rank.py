"""Pins of the oracle's rank diagnostics: effective rank and NER ([KV-CoRE] 2.B) and
the cumulative-eigenvalue (energy) rank ([xKV blog] figure 2(c)).

Each pin would fail for a plausible slip: using the eigenvalues instead of the
singular values in the entropy, dropping the normalisation, a base-2 logarithm,
counting zero singular values in r, an off-by-one in the energy rank or a strict
instead of a non-strict threshold.
"""
import math

import numpy as np
import pytest

import oracle
from synth import make_workload


def test_flat_spectrum():
    # k equal singular values: entropy log k, erank k, NER 1 (for any scale).
    for k in (1, 3, 64):
        lam = np.zeros(100)
        lam[:k] = 7.5
        assert oracle.numerical_rank(lam) == k
        assert oracle.effective_rank(lam) == pytest.approx(k, rel=1e-12)
        assert oracle.ner(lam) == pytest.approx(1.0, rel=1e-12)


def test_two_level_spectrum_uses_singular_values():
    # lambda = (4, 1): sigma = (2, 1), p = (2/3, 1/3), exp(H) = 3 / 2^(2/3) = 1.88988...
    # (with the eigenvalues themselves, p = (0.8, 0.2) and exp(H) = 1.649 instead).
    e = oracle.effective_rank([4.0, 1.0])
    assert e == pytest.approx(3.0 / 2.0 ** (2.0 / 3.0), rel=1e-12)
    assert oracle.ner([4.0, 1.0]) == pytest.approx(e / 2.0, rel=1e-12)


def test_dominant_direction_and_bounds():
    assert oracle.effective_rank([3.0, 0.0, 0.0]) == pytest.approx(1.0)
    assert oracle.numerical_rank([1.0, 1e-40, 0.0]) == 1        # below n * eps of sigma_1
    rng = np.random.default_rng(3)
    for _ in range(20):
        lam = rng.exponential(size=50) ** 3
        r = oracle.numerical_rank(lam)
        n = oracle.ner(lam)
        assert 1.0 / r - 1e-12 <= n <= 1.0 + 1e-12
        assert oracle.effective_rank(lam * 123.0) == pytest.approx(oracle.effective_rank(lam), rel=1e-12)


def test_effective_rank_matches_svd_of_the_matrix():
    # Independent route: singular values of X from LAPACK's SVD, entropy written out.
    rng = np.random.default_rng(0)
    X = rng.standard_normal((300, 40)) @ np.diag(np.linspace(3.0, 0.1, 40))
    sv = np.linalg.svd(X, compute_uv=False)
    p = sv / sv.sum()
    want = math.exp(-sum(pi * math.log(pi) for pi in p))
    assert oracle.effective_rank(np.linalg.eigvalsh(X.T @ X)) == pytest.approx(want, rel=1e-9)


def test_energy_rank_thresholds():
    assert oracle.energy_rank(np.ones(100)) == 95
    assert oracle.energy_rank([0.5, 0.45, 0.05], 0.95) == 2      # reaching the target counts
    assert oracle.energy_rank([0.5, 0.45, 0.05], 0.951) == 3
    assert oracle.energy_rank([0.05, 0.5, 0.45], 0.5) == 1       # order of the input is irrelevant
    # Partial spectrum against a given total (trace of the Gram).
    assert oracle.energy_rank([5.0, 3.0], 0.8, total=10.0) == 2
    assert oracle.energy_rank([5.0, 3.0], 0.9, total=10.0) == -1


def test_grouping_lowers_the_energy_rank_fraction():
    # The figure-2(c) effect on the shared-latent generator: the concatenation of a group's
    # layers needs a smaller fraction of its dimension for 95 % of the energy than a layer.
    wl = make_workload("llama16k", T=2048, n_layers=4, n_kv_heads=2, n_q_heads=8, rank=64, latent_rank=96)
    layers = [x.double().numpy() for x in wl.group_kv(0, "K", 0)]
    per_layer = np.mean([oracle.energy_rank(np.linalg.eigvalsh(x.T @ x)) / x.shape[1] for x in layers])
    X = oracle.group_matrix(layers)
    grouped = oracle.energy_rank(np.linalg.eigvalsh(oracle.gram(X))) / X.shape[1]
    assert grouped < per_layer


def test_energy_rank_full_fraction_reaches_last_nonzero():
    # frac = 1 with the spectrum's own total: the count of nonzero eigenvalues (values of
    # one magnitude, so that none is absorbed by the rounding of the running sum).
    rng = np.random.default_rng(5)
    for n in (7, 100, 1000):
        lam = np.r_[rng.random(n) + 0.5, np.zeros(5)]
        assert oracle.energy_rank(lam, 1.0) == n


# ------------------------------------------------------------------ adaptive rank
def _brute_alloc(spectra, budget, granule, r_min, r_max):
    """Every combination of ranks, the best kept energy (independent of the DP)."""
    import itertools
    opts = list(range(r_min, r_max + 1, granule))
    best = -1.0
    for combo in itertools.product(opts, repeat=len(spectra)):
        if sum(combo) > budget:
            continue
        e = sum(float(np.sum(np.sort(lam)[::-1][:r])) for lam, r in zip(spectra, combo))
        best = max(best, e)
    return best


def test_allocate_ranks_hand_case():
    # Sides (10, 1, 1, 1) and (5, 4, 3, 2), one eigenvalue per granule, four in all: the
    # four largest are 10, 5, 4, 3, so side 0 keeps one and side 1 three (kept 22).
    ranks, kept = oracle.allocate_ranks([[10, 1, 1, 1], [5, 4, 3, 2]], budget=4, granule=1, r_min=0, r_max=4)
    assert ranks == [1, 3] and kept == 22.0
    # A floor of two per side: 10 + 1 + 5 + 4 = 20.
    ranks, kept = oracle.allocate_ranks([[10, 1, 1, 1], [5, 4, 3, 2]], budget=4, granule=1, r_min=2, r_max=4)
    assert ranks == [2, 2] and kept == 20.0


@pytest.mark.parametrize("seed", range(5))
def test_allocate_ranks_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    S, g = 3, 2
    spectra = [np.sort(rng.exponential(size=8) ** 2)[::-1] * rng.uniform(0.2, 5) for _ in range(S)]
    for budget in (6, 9, 12, 17, 24):
        ranks, kept = oracle.allocate_ranks(spectra, budget, g, 2, 8)
        assert sum(ranks) <= budget and all(2 <= r <= 8 and r % g == 0 for r in ranks)
        assert kept == pytest.approx(sum(float(np.sum(l[:r])) for l, r in zip(spectra, ranks)), rel=1e-14)
        assert kept == pytest.approx(_brute_alloc(spectra, budget, g, 2, 8), rel=1e-14)


def test_allocate_ranks_equal_spectra_is_uniform():
    # Identical, strictly decreasing spectra: every extra granule is worth less than the one
    # before, so the budget splits evenly.
    lam = 1.0 / np.arange(1, 65) ** 0.8
    ranks, _ = oracle.allocate_ranks([lam] * 4, budget=4 * 24, granule=8, r_min=8, r_max=64)
    assert ranks == [24, 24, 24, 24]


def test_allocated_ranks_minimise_the_reconstruction_error():
    # The objective is the reconstruction error of the truncated factorisations: the tail
    # sums equal ||X_s - A_s B_s||_F^2 of the oracle's own rank-r_s compressions, and no
    # other allocation of the same budget does better.
    rng = np.random.default_rng(7)
    sides = []
    for s, decay in enumerate((0.4, 1.2, 2.0)):
        U = rng.standard_normal((200, 24))
        W = rng.standard_normal((24, 24)) * (np.arange(1, 25) ** -decay)[:, None]
        sides.append([U @ W[:, :12] + 0.01 * rng.standard_normal((200, 12)),
                      U @ W[:, 12:] + 0.01 * rng.standard_normal((200, 12))])
    spectra = [np.linalg.eigvalsh(oracle.gram(oracle.group_matrix(x)))[::-1] for x in sides]
    ranks, kept = oracle.allocate_ranks(spectra, budget=24, granule=4, r_min=4, r_max=20)
    err = sum(np.linalg.norm(oracle.group_matrix(x) - (lambda c: c["A"] @ c["B"])(oracle.compress_group(x, r))) ** 2
              for x, r in zip(sides, ranks))
    total = sum(float(np.sum(l)) for l in spectra)
    assert err == pytest.approx(total - kept, rel=1e-9)
    assert ranks[0] > ranks[2]     # the slowly decaying side gets the larger share
    for alt in ([8, 8, 8], [12, 8, 4], [4, 8, 12]):
        e_alt = sum(np.linalg.norm(oracle.group_matrix(x) - (lambda c: c["A"] @ c["B"])(oracle.compress_group(x, r)))
                    ** 2 for x, r in zip(sides, alt))
        assert err <= e_alt * (1 + 1e-12)


def test_allocate_ranks_budget_monotone_and_errors():
    rng = np.random.default_rng(9)
    spectra = [np.sort(rng.random(32))[::-1] for _ in range(5)]
    prev = -1.0
    for budget in range(20, 161, 20):
        _, kept = oracle.allocate_ranks(spectra, budget, 4, 4, 32)
        assert kept >= prev
        prev = kept
    with pytest.raises(ValueError):
        oracle.allocate_ranks(spectra, 10, 4, 4, 32)          # 5 sides x 4 > 10
