"""Pins of the oracle's token append (multi-turn growth): projecting rows that were
part of a factored prefix onto its basis gives back that prefix's A rows, landmarks of
appended rows equal the matching slice of the whole sequence's landmarks, and a
complete basis reconstructs appended rows exactly."""
import numpy as np

import oracle


def _layers(T, G=2, d_kv=16, seed=0):
    rng = np.random.default_rng(seed)
    U = rng.standard_normal((T, 6))
    return [U @ rng.standard_normal((6, d_kv)) + 0.01 * rng.standard_normal((T, d_kv)) for _ in range(G)]


def test_append_reproduces_prefix_rows():
    layers = _layers(96)
    ref = oracle.compress_group(layers, r=5)
    Bt = ref["B"].T                                   # n x r, V_r as stored
    tail = [x[64:] for x in layers]
    got = oracle.append_tokens(tail, Bt, pos0=64)["A"]
    np.testing.assert_allclose(got, ref["A"][64:], rtol=0, atol=1e-12)


def test_append_landmarks_are_the_whole_sequences_slice():
    K = _layers(64, G=1, d_kv=8)[0]                   # 2 heads x 4 dims
    whole = oracle.landmarks(K, 2, 4, chunk=8)
    part = oracle.append_tokens([K[40:]], np.eye(8), pos0=40, n_kv_heads=2, head_dim=4, chunk=8,
                                with_landmarks=True)["landmarks"][0]
    np.testing.assert_allclose(part, whole[:, 5:], rtol=0, atol=1e-12)


def test_full_basis_reconstructs_appended_rows():
    layers = _layers(80, G=2, d_kv=8)
    n = 16
    ref = oracle.compress_group([x[:48] for x in layers], r=n)   # complete basis of R^n
    new = [x[48:] for x in layers]
    A_new = oracle.append_tokens(new, ref["B"].T, pos0=48)["A"]
    for l in range(2):
        np.testing.assert_allclose(oracle.reconstruct_layer(A_new, ref["B"], l, 8), new[l], atol=1e-10)
