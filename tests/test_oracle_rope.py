"""Pins for the oracle's RoPE and landmark means (closed forms, no GPU).

RoPE is applied to reconstructed pre-RoPE keys (KQ-SVD section 2 recalls the
pre-RoPE key compression precedent).  The rotate-half convention and the
base 10000 are readings; these tests fix them through independent
formulations so that a swapped pair, a wrong sign or a wrong frequency fails.
"""
import math

import numpy as np
import pytest

import oracle


def rope_complex(x, pos, theta=10000.0):
    """Independent RoPE: pair (x_i, x_{i+d/2}) as the complex number x_i + j x_{i+d/2}
    multiplied by exp(j * pos * theta**(-2i/d))."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    z = x[..., :half] + 1j * x[..., half:]
    f = np.array([theta ** (-2.0 * i / d) for i in range(half)])
    z = z * np.exp(1j * np.multiply.outer(np.asarray(pos, dtype=np.float64), f))
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rope_hand_values_d4():
    # d = 4: frequencies 1 and 10000**-0.5 = 0.01.
    e0 = np.array([1.0, 0, 0, 0])
    e1 = np.array([0, 1.0, 0, 0])
    e2 = np.array([0, 0, 1.0, 0])
    np.testing.assert_allclose(oracle.rope(e0, 1), [math.cos(1), 0, math.sin(1), 0], atol=1e-15)
    np.testing.assert_allclose(oracle.rope(e2, 1), [-math.sin(1), 0, math.cos(1), 0], atol=1e-15)
    np.testing.assert_allclose(oracle.rope(e1, 2), [0, math.cos(0.02), 0, math.sin(0.02)], atol=1e-15)


def test_rope_identity_at_zero_and_norm():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 128))
    np.testing.assert_allclose(oracle.rope(x, 0), x, atol=0)
    y = oracle.rope(x, np.array([3, 70000, 122879, 5, 9]))
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_rope_matches_complex_form():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 64))
    pos = np.array([0, 1, 17, 255, 4096, 65535, 122880])
    np.testing.assert_allclose(oracle.rope(x, pos), rope_complex(x, pos), atol=1e-12)


def test_rope_relative_position():
    # <RoPE(q, a), RoPE(k, b)> depends only on a - b.
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    ref = oracle.rope(q, 7) @ oracle.rope(k, 0)
    for a, b in [(10, 3), (65543, 65536), (122887, 122880)]:
        assert abs(oracle.rope(q, a) @ oracle.rope(k, b) - ref) < 1e-9


def test_landmark_closed_form_d2():
    # d = 2: RoPE multiplies z = k0 + j k1 by exp(j t).  The mean over chunk c of a
    # constant key is z exp(8jc) (1 - exp(8j)) / (8 (1 - exp(j))).
    T, chunk = 64, 8
    k = np.array([0.7, -1.3])
    K = np.tile(k, (T, 1))
    m = oracle.landmarks(K, n_kv_heads=1, head_dim=2, chunk=chunk)
    z = complex(k[0], k[1])
    for c in range(T // chunk):
        ref = z * np.exp(1j * chunk * c) * (1 - np.exp(1j * chunk)) / (chunk * (1 - np.exp(1j)))
        np.testing.assert_allclose(m[0, c], [ref.real, ref.imag], atol=1e-14)


def test_landmark_is_chunk_mean_per_head():
    rng = np.random.default_rng(4)
    H, d, T, chunk = 3, 8, 40, 8
    K = rng.standard_normal((T, H * d))
    m = oracle.landmarks(K, n_kv_heads=H, head_dim=d, chunk=chunk)
    assert m.shape == (H, T // chunk, d)
    for h in range(H):
        for c in range(T // chunk):
            acc = np.zeros(d)
            for t in range(c * chunk, (c + 1) * chunk):
                acc += rope_complex(K[t, h * d:(h + 1) * d], t)
            np.testing.assert_allclose(m[h, c], acc / chunk, atol=1e-13)


@pytest.mark.parametrize("t", [122879, 65535])
def test_rope_phase_is_float64(t):
    # A float32 phase would be off by ~1e-2 rad at these positions; the oracle is exact
    # to double rounding.  Compare against math.cos of the exactly formed angle.
    d = 128
    x = np.zeros(d)
    x[0] = 1.0
    y = oracle.rope(x, t)
    assert abs(y[0] - math.cos(t * 1.0)) < 1e-12
