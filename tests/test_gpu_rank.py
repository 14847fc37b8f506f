"""Rank diagnostics from the GPU compression vs the float64 oracle on the same X.

A compression at r = n spans the whole space, so its Ritz values are the exact
spectrum of the GPU's Gram; with stats[4] = trace(C) they give the effective rank,
NER ([KV-CoRE] 2.B) and the cumulative-eigenvalue rank ([xKV blog] figure 2(c)).
The integer energy rank is compared exactly unless the oracle's cumulative sum lies
within the Gram's rounding (1e-5 relative) of the threshold, where a neighbour is
also accepted.
"""
import numpy as np
import pytest
import torch

import kv_cache_cross_amd as xk
import oracle
from parity_util import f64
from synth import make_workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MINI = dict(T=2000, n_layers=4, n_kv_heads=2, n_q_heads=8, rank=128, latent_rank=192, top_k=32)


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def ctx():
    c = xk.Context(0)
    yield c
    c.close()


def _energy_rank_ok(got, lam_ref, frac, total):
    want = oracle.energy_rank(lam_ref, frac, total=total)
    if got == want:
        return True
    csum = np.cumsum(np.sort(lam_ref)[::-1])
    near = np.abs(csum - frac * total) <= 1e-5 * total
    return abs(got - want) == 1 and near[min(got, want) - 1]


@pytest.mark.parametrize("side", ["K", "V"])
def test_rank_stats_full_spectrum(ctx, side):
    wl = make_workload("llama16k", device=DEV, **MINI)
    X = wl.group_kv(0, side, 0)[0]                       # one layer: n = 256
    n = X.shape[1]
    out = xk.compress(ctx, [[X]], r=n, n_kv_heads=2, head_dim=128, landmarks=[False])[0]
    torch.cuda.synchronize()
    lam_ref = np.linalg.eigvalsh(oracle.gram(f64(X)))
    trace = out["stats"]["energy"]
    assert trace == pytest.approx(lam_ref.sum(), rel=1e-6)
    got = xk.rank_stats(out["eigvals"], total=trace, frac=0.95, complete=True)
    log(f"  {side}: NER {got['ner']:.6f} (oracle {oracle.ner(lam_ref):.6f}), erank {got['erank']:.3f}, "
        f"rank95 {got['energy_rank']} (oracle {oracle.energy_rank(lam_ref, 0.95)})")
    assert got["numerical_rank"] == oracle.numerical_rank(lam_ref)
    assert got["erank"] == pytest.approx(oracle.effective_rank(lam_ref), rel=1e-4)
    assert got["ner"] == pytest.approx(oracle.ner(lam_ref), rel=1e-4)
    for frac in (0.5, 0.9, 0.95, 0.99):
        g = xk.rank_stats(out["eigvals"], total=trace, frac=frac)["energy_rank"]
        assert _energy_rank_ok(g, lam_ref, frac, lam_ref.sum()), (frac, g)


def test_rank_stats_group_leading_ritz_values(ctx):
    # A group of 4 layers (n = 1024) at r = 128: the energy rank from the leading Ritz
    # values and the trace, against the oracle's full spectrum.
    wl = make_workload("llama16k", device=DEV, **MINI)
    layers = wl.group_kv(0, "K", 0)
    out = xk.compress(ctx, [layers], r=128, n_kv_heads=2, head_dim=128, landmarks=[False])[0]
    torch.cuda.synchronize()
    lam_ref = np.linalg.eigvalsh(oracle.gram(oracle.group_matrix([f64(x) for x in layers])))
    trace = out["stats"]["energy"]
    assert trace == pytest.approx(lam_ref.sum(), rel=1e-6)
    for frac in (0.5, 0.8, 0.9):
        got = xk.rank_stats(out["eigvals"], total=trace, frac=frac)
        want = oracle.energy_rank(lam_ref, frac)
        log(f"  group frac {frac}: {got['energy_rank']} (oracle {want}), covered {got['covered']:.4f}")
        if want <= 128:
            assert _energy_rank_ok(got["energy_rank"], lam_ref, frac, lam_ref.sum())
        else:
            assert got["energy_rank"] == -1
