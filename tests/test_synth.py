"""The seeded generator: shapes, dtypes, determinism, and the low-rank premise."""
import numpy as np
import torch

from synth import CONFIGS, make_workload


def test_shapes_and_determinism():
    a = make_workload("tiny", seed=0)
    b = make_workload("tiny", seed=0)
    c = make_workload("tiny", seed=1)
    ka, kb, kc = a.layer_kv(0, "K", 1), b.layer_kv(0, "K", 1), c.layer_kv(0, "K", 1)
    assert ka.shape == (256, 64) and ka.dtype == torch.float32
    assert torch.equal(ka, kb) and not torch.equal(ka, kc)
    assert not torch.equal(a.layer_kv(0, "K", 0), a.layer_kv(0, "V", 0))
    assert a.query(0, 0, 0).shape == (1, 64)


def test_bf16_rounding_and_sharing():
    wl = make_workload("llama64k", T=64, n_layers=8)
    k0 = wl.layer_kv(0, "K", 0)
    assert k0.dtype == torch.bfloat16 and k0.shape == (64, 1024)
    # Neighbouring latent blocks share the first 70 % of their latent columns.
    U0, U1 = wl.latent(0, "K", 0), wl.latent(0, "K", 1)
    m = int(0.7 * 768)
    assert torch.equal(U0[:, :m], U1[:, :m]) and not torch.equal(U0[:, m:], U1[:, m:])


def test_low_rank_premise():
    # The group matrix has a spectral cliff at the latent rank.
    wl = make_workload("tiny")
    X = torch.cat(wl.group_kv(0, "K", 0), dim=1).double().numpy()
    s = np.linalg.svd(X, compute_uv=False)
    assert s[31] / s[32] > 5.0


def test_config_table():
    assert CONFIGS["llama64k"].n == 4096 and CONFIGS["qwen122k"].n == 2048
    assert [CONFIGS[f"batch8_g{g}"].rank for g in (1, 2, 4, 8)] == [128, 256, 512, 1024]
