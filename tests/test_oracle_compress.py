"""Pins for the oracle's group factorisation (no GPU).

What the pages fix: a group's layers are concatenated horizontally and factored
once into a shared basis A and per-layer B_l (xKV blog, section on what xKV
does); the top right singular vectors come from the eigendecomposition of the
uncentred covariance (KV-CoRE section 2.A); the rank-R projector V V^T is the
Eckart-Young optimum (KQ-SVD section 3.3).  Group size 1 is the single-layer
SVD baseline (xKV blog, Table 2).
"""
import json
import os

import numpy as np
import pytest

import oracle
from synth import make_workload

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def jacobi_svd(X, sweeps=60):
    """One-sided (Hestenes) Jacobi SVD, written independently of LAPACK.

    Returns singular values (descending) and right singular vectors.
    """
    U = np.array(X, dtype=np.float64)
    n = U.shape[1]
    V = np.eye(n)
    for _ in range(sweeps):
        off = 0.0
        for p in range(n - 1):
            for q in range(p + 1, n):
                a = U[:, p] @ U[:, p]
                b = U[:, q] @ U[:, q]
                g = U[:, p] @ U[:, q]
                if abs(g) <= 1e-15 * np.sqrt(a * b) or g == 0.0:
                    continue
                off = max(off, abs(g) / np.sqrt(a * b))
                zeta = (b - a) / (2.0 * g)
                t = np.sign(zeta) / (abs(zeta) + np.sqrt(1.0 + zeta * zeta)) if zeta != 0 else 1.0
                c = 1.0 / np.sqrt(1.0 + t * t)
                s = c * t
                up, uq = U[:, p].copy(), U[:, q].copy()
                U[:, p], U[:, q] = c * up - s * uq, s * up + c * uq
                vp, vq = V[:, p].copy(), V[:, q].copy()
                V[:, p], V[:, q] = c * vp - s * vq, s * vp + c * vq
        if off < 1e-14:
            break
    sig = np.linalg.norm(U, axis=0)
    order = np.argsort(sig)[::-1]
    return sig[order], V[:, order]


def _layers(rng, T, G, d_kv, R, sigma=0.05):
    U = rng.standard_normal((T, R))
    s = np.arange(1, R + 1) ** -0.8
    return [U @ (s[:, None] * rng.standard_normal((R, d_kv))) + sigma * rng.standard_normal((T, d_kv))
            for _ in range(G)]


def test_golden_2x2():
    g = json.load(open(os.path.join(GOLD, "svd_2x2.json")))
    X = np.array(g["X"])
    res = oracle.compress_group([X], 1)
    np.testing.assert_allclose(res["eigvals"], g["eigvals"], atol=1e-12)
    np.testing.assert_allclose(res["A"] @ res["B"], g["rank1_reconstruction"], atol=1e-12)
    assert abs(np.sum((X - res["A"] @ res["B"]) ** 2) - g["rank1_sq_residual"]) < 1e-12


@pytest.mark.parametrize("T,G,d_kv,R,r", [(96, 2, 16, 12, 5), (200, 4, 8, 20, 7), (64, 1, 24, 30, 10)])
def test_eckart_young_closed_form(T, G, d_kv, R, r):
    rng = np.random.default_rng(T + G + r)
    layers = _layers(rng, T, G, d_kv, R)
    res = oracle.compress_group(layers, r)
    X = np.concatenate(layers, axis=1)
    sig = np.linalg.svd(X, compute_uv=False)        # independent LAPACK route (gesdd)
    sq_err = np.sum((X - res["A"] @ res["B"]) ** 2)
    assert abs(sq_err - np.sum(sig[r:] ** 2)) <= 1e-10 * np.sum(sig ** 2)
    # Covariance route: eigenvalues of X^T X are the squared singular values.
    np.testing.assert_allclose(res["eigvals"][: sig.size], sig ** 2, rtol=1e-9, atol=1e-9 * sig[0] ** 2)
    # Orthonormal basis columns.
    np.testing.assert_allclose(res["Vr"].T @ res["Vr"], np.eye(r), atol=1e-12)
    # rel_err is the plain Frobenius ratio.
    assert abs(res["rel_err"] - np.sqrt(sq_err) / np.linalg.norm(X)) < 1e-14


def test_full_rank_is_exact():
    rng = np.random.default_rng(5)
    layers = _layers(rng, 50, 3, 6, 10)
    res = oracle.compress_group(layers, 18)
    np.testing.assert_allclose(res["A"] @ res["B"], np.concatenate(layers, axis=1), atol=1e-11)
    for l in range(3):
        np.testing.assert_allclose(oracle.reconstruct_layer(res["A"], res["B"], l, 6), layers[l], atol=1e-11)


def test_group_size_one_is_per_layer_svd():
    rng = np.random.default_rng(6)
    K = _layers(rng, 60, 1, 10, 14)[0]
    r = 4
    res = oracle.compress_group([K], r)
    U, s, Vt = np.linalg.svd(K, full_matrices=False)
    trunc = (U[:, :r] * s[:r]) @ Vt[:r]
    np.testing.assert_allclose(res["A"] @ res["B"], trunc, atol=1e-10)
    sig, V = jacobi_svd(K)
    np.testing.assert_allclose(sig, s, rtol=1e-10)
    P_jac = V[:, :r] @ V[:, :r].T
    np.testing.assert_allclose(res["Vr"] @ res["Vr"].T, P_jac, atol=1e-9)


def test_jacobi_covariance_route_on_group():
    # The covariance eigenvectors span the same top-r subspace as an SVD of X itself.
    rng = np.random.default_rng(7)
    layers = _layers(rng, 80, 2, 6, 9)
    res = oracle.compress_group(layers, 5)
    sig, V = jacobi_svd(np.concatenate(layers, axis=1))
    np.testing.assert_allclose(res["Vr"] @ res["Vr"].T, V[:, :5] @ V[:, :5].T, atol=1e-9)
    np.testing.assert_allclose(res["eigvals"][:12], sig ** 2, rtol=1e-9)


def test_rotation_invariance_of_reconstruction():
    rng = np.random.default_rng(8)
    layers = _layers(rng, 70, 2, 8, 10)
    res = oracle.compress_group(layers, 6)
    O, _ = np.linalg.qr(rng.standard_normal((6, 6)))
    X = res["X"]
    Vr2 = res["Vr"] @ O
    np.testing.assert_allclose((X @ Vr2) @ Vr2.T, res["A"] @ res["B"], atol=1e-10)


def test_error_decreases_with_rank():
    rng = np.random.default_rng(9)
    layers = _layers(rng, 120, 2, 12, 16)
    errs = [oracle.compress_group(layers, r)["rel_err"] for r in range(1, 25)]
    assert all(a >= b - 1e-14 for a, b in zip(errs, errs[1:]))
    assert errs[-1] < 1e-12


def test_grouping_helps_on_shared_latent():
    # xKV blog Table 2: at a fixed compression ratio, a larger group reconstructs
    # better when the layers share their dominant subspace.  Sanity only.
    rng = np.random.default_rng(10)
    T, d_kv, R = 400, 16, 12
    U = rng.standard_normal((T, R))
    s = np.arange(1, R + 1) ** -0.8
    layers = [U @ (s[:, None] * rng.standard_normal((R, d_kv))) + 0.02 * rng.standard_normal((T, d_kv))
              for _ in range(4)]
    r1 = 4
    err_g1 = np.sqrt(sum(oracle.compress_group([K], r1)["rel_err"] ** 2 * np.sum(K ** 2) for K in layers)
                     / sum(np.sum(K ** 2) for K in layers))
    err_g4 = oracle.compress_group(layers, 4 * r1)["rel_err"]
    assert err_g4 < err_g1


def test_tiny_workload_runs_through_oracle():
    wl = make_workload("tiny")
    cfg = wl.cfg
    layers = [t.double().numpy() for t in wl.group_kv(0, "K", 0)]
    res = oracle.compress_group(layers, cfg.rank)
    assert res["A"].shape == (cfg.T, cfg.rank) and res["B"].shape == (cfg.rank, cfg.n)
    assert 0.0 < res["rel_err"] < 1.0
    assert np.all(np.diff(res["eigvals"]) <= 1e-9 * res["eigvals"][0])


def test_tiny_regression_fixture():
    # Guards the oracle against silent drift; regenerate with tests/golden/make_golden.py
    # only together with a change whose commit message names the passage behind it.
    import sys
    sys.path.insert(0, GOLD)
    from make_golden import tiny_reference
    stored = json.load(open(os.path.join(GOLD, "tiny_oracle.json")))
    now = tiny_reference()
    assert abs(now["rel_err_K"] - stored["rel_err_K"]) < 1e-12
    assert abs(now["rel_err_V"] - stored["rel_err_V"]) < 1e-12
    for a, b in zip(now["layers"], stored["layers"]):
        assert a["sel"] == b["sel"]
        np.testing.assert_allclose(a["out"], b["out"], atol=1e-12)
