"""Helpers shared by the GPU parity tests (comparison rules and input assembly)."""
from __future__ import annotations

import numpy as np
import torch

# Tolerances of the parity protocol.
NEAR_TIE = 1e-3          # chunk scores within this of the k-th score may be selected either way
PROJ_TOL = 1e-3          # ||P_gpu - P_ref||_F
RECON_TOL = 1e-4         # |rel_err_gpu - rel_err_ref|
ATT_REL_BF16, ATT_ABS_BF16 = 1e-2, 2e-2
ATT_REL_F32 = 1e-4


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().double().cpu().numpy()


def check_selection(gpu_sel, scores, k: int, band: float = NEAR_TIE):
    """The GPU's chunk set must equal the oracle's top-k except for chunks whose oracle
    score lies within ``band`` of the k-th score.  Returns the number of near-tie swaps."""
    gpu = [int(c) for c in np.asarray(gpu_sel).tolist() if c >= 0]
    n = len(scores)
    keff = min(k, n)
    assert len(gpu) == keff, f"selected {len(gpu)} chunks, expected {keff}"
    assert len(set(gpu)) == keff, "duplicate chunk ids"
    assert gpu == sorted(gpu), "chunk ids not ascending"
    if keff == 0:
        return 0
    if keff == n:
        assert gpu == list(range(n))
        return 0
    s = np.asarray(scores, dtype=np.float64)
    kth = np.sort(s)[::-1][keff - 1]
    sure_in = set(np.nonzero(s > kth + band)[0].tolist())
    sure_out = set(np.nonzero(s < kth - band)[0].tolist())
    g = set(gpu)
    assert sure_in <= g, f"missing clearly selected chunks {sorted(sure_in - g)[:10]}"
    assert not (g & sure_out), f"selected clearly rejected chunks {sorted(g & sure_out)[:10]}"
    ref = set(np.lexsort((np.arange(n), -s))[:keff].tolist())
    return len(g - ref)


def projector_distance(V1: np.ndarray, V2: np.ndarray) -> float:
    """||V1 V1^T - V2 V2^T||_F without forming n x n matrices (V1, V2 n x r, orthonormal-ish)."""
    a = np.sum((V1.T @ V1) ** 2)
    b = np.sum((V2.T @ V2) ** 2)
    c = np.sum((V1.T @ V2) ** 2)
    return float(np.sqrt(max(a + b - 2 * c, 0.0)))


def attention_errors(got: np.ndarray, ref: np.ndarray):
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    mx = float(np.max(np.abs(got - ref)))
    return rel, mx


def tail_rows(T: int, n_sink: int, n_local: int):
    return list(range(n_sink)) + list(range(T - n_local, T))


def check_selection_banded(gpu_sel, scores, k: int, band):
    """The GPU's chunk set must be a top-k of the oracle's scores after some perturbation
    of each score s_c by at most band[c]: with S the GPU's set, min over S of (s_c + band_c)
    must reach max over the other candidates of (s_c - band_c).  Returns the number of
    chunks in S outside the oracle's own top-k."""
    gpu = [int(c) for c in np.asarray(gpu_sel).tolist() if c >= 0]
    s = np.asarray(scores, dtype=np.float64)
    n = len(s)
    keff = min(k, n)
    assert len(gpu) == keff, f"selected {len(gpu)} chunks, expected {keff}"
    assert len(set(gpu)) == keff and gpu == sorted(gpu), "chunk ids not distinct and ascending"
    if keff == 0 or keff == n:
        assert gpu == list(range(keff))
        return 0
    band = np.broadcast_to(np.asarray(band, dtype=np.float64), s.shape)
    inside = np.zeros(n, dtype=bool)
    inside[gpu] = True
    lo_in = np.min(s[inside] + band[inside])
    hi_out = np.max(s[~inside] - band[~inside])
    assert lo_in >= hi_out, f"selection not a top-{keff} within the band ({lo_in:.6g} < {hi_out:.6g})"
    ref = set(np.lexsort((np.arange(n), -s))[:keff].tolist())
    return len(set(gpu) - ref)
