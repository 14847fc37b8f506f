"""Pins for the oracle's Selective Reconstruction decode (no GPU).

Decode appends the new key/value and attends softmax(q K^T / sqrt(d)) V
(KQ-SVD section 3.2).  Selective Reconstruction rebuilds only the rows of the
chunks that a landmark-guided top-k selector picks (xKV blog, section on
Selective Reconstruction).  Selecting every chunk at full rank must therefore
give dense attention, and at rank r it must give attention over the fully
reconstructed cache ("xKV without SR").
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from test_oracle_rope import rope_complex

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- selection
def brute_topk(scores, k):
    """Chunk c is selected iff fewer than k chunks beat it (higher score, or equal score
    and lower id)."""
    s = list(scores)
    sel = []
    for c in range(len(s)):
        better = sum(1 for c2 in range(len(s)) if s[c2] > s[c] or (s[c2] == s[c] and c2 < c))
        if better < k:
            sel.append(c)
    return sel


def test_topk_golden():
    g = json.load(open(os.path.join(GOLD, "topk_ties.json")))
    for case in g["cases"]:
        assert oracle.select_topk(np.array(g["scores"]), case["k"]).tolist() == case["sel"]


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 60))
    scores = rng.integers(0, 7, size=n).astype(np.float64) / 4.0   # many ties
    for k in [1, 2, 5, n // 2 + 1, n, n + 3]:
        assert oracle.select_topk(scores, k).tolist() == brute_topk(scores, k)


def test_attended_set_golden():
    g = json.load(open(os.path.join(GOLD, "attended_set.json")))
    assert oracle.candidate_chunks(g["T"], g["n_local"], g["chunk"]) == g["n_candidates"]
    pos = oracle.attended_positions(g["sel"], g["T"], g["n_sink"], g["n_local"], g["n_gen"], g["chunk"])
    assert pos.tolist() == g["positions"]


def test_candidates_partial_local_chunk():
    # A chunk that is only partly inside the local window stays a candidate.
    assert oracle.candidate_chunks(64, 12, 8) == 7
    assert oracle.candidate_chunks(64, 16, 8) == 6


# ---------------------------------------------------------------- attention
def test_dense_decode_hand_example_d2():
    # d = 2, one head: keys (1,0) at positions 0 and 1, query (1,0) at position 1.
    # Rotations by t radians give logits cos(1)/sqrt2 and 1/sqrt2.
    K = np.array([[1.0, 0.0], [1.0, 0.0]])
    V = np.array([[1.0, 0.0], [0.0, 1.0]])
    out = oracle.dense_decode(np.array([[1.0, 0.0]]), K, V, p=1, n_kv_heads=1)
    w1 = 1.0 / (1.0 + math.exp((math.cos(1.0) - 1.0) / math.sqrt(2.0)))
    np.testing.assert_allclose(out[0], [1.0 - w1, w1], atol=1e-15)


def _dense_complex(q, K, V, p, n_kv_heads):
    """Attention written from scratch with the complex-number RoPE."""
    H_q, d = q.shape
    grp = H_q // n_kv_heads
    out = np.zeros((H_q, d))
    for j in range(H_q):
        h = j // grp
        qr = rope_complex(q[j], p)
        kr = rope_complex(K[:, h * d:(h + 1) * d], np.arange(K.shape[0]))
        z = kr @ qr / math.sqrt(d)
        w = np.exp(z - z.max())
        out[j] = (w / w.sum()) @ V[:, h * d:(h + 1) * d]
    return out


def _setup(seed, T=64, G=2, H_kv=2, H_q=4, d=8, n_gen=3, R=10):
    rng = np.random.default_rng(seed)
    d_kv = H_kv * d
    U = rng.standard_normal((T + n_gen, R))
    Ks = [U @ rng.standard_normal((R, d_kv)) + 0.1 * rng.standard_normal((T + n_gen, d_kv)) for _ in range(G)]
    Vs = [rng.standard_normal((T + n_gen, d_kv)) for _ in range(G)]
    q = rng.standard_normal((H_q, d))
    return rng, Ks, Vs, q


def _decode(q, Ks, Vs, layer, r, top_k, T=64, n_gen=3, H_kv=2, d=8, chunk=8, n_sink=4, n_local=16):
    d_kv = H_kv * d
    ck = oracle.compress_group([K[:T] for K in Ks], r)
    cv = oracle.compress_group([V[:T] for V in Vs], r)
    lm = oracle.landmarks(Ks[layer][:T], H_kv, d, chunk)
    exact = [t for t in range(T + n_gen) if t < n_sink or t >= T - n_local]
    res = oracle.sr_decode_layer(
        q, T=T, n_gen=n_gen, n_kv_heads=H_kv, chunk=chunk, top_k=top_k, n_sink=n_sink,
        n_local=n_local, landmarks_l=lm, A_k=ck["A"], B_k_l=ck["B"][:, layer * d_kv:(layer + 1) * d_kv],
        A_v=cv["A"], B_v_l=cv["B"][:, layer * d_kv:(layer + 1) * d_kv],
        k_exact={t: Ks[layer][t] for t in exact}, v_exact={t: Vs[layer][t] for t in exact})
    return res, ck, cv


@pytest.mark.parametrize("seed", [0, 1])
def test_all_chunks_full_rank_is_dense(seed):
    _, Ks, Vs, q = _setup(seed)
    T, n_gen, d_kv = 64, 3, 16
    for layer in range(2):
        res, _, _ = _decode(q, Ks, Vs, layer, r=2 * d_kv, top_k=1000)
        ref = _dense_complex(q, Ks[layer], Vs[layer], T + n_gen - 1, 2)
        np.testing.assert_allclose(res["out"], ref, atol=1e-10)
        ref2 = oracle.dense_decode(q, Ks[layer], Vs[layer], T + n_gen - 1, 2)
        np.testing.assert_allclose(res["out"], ref2, atol=1e-10)


def test_all_chunks_at_rank_r_is_full_reconstruction():
    _, Ks, Vs, q = _setup(3)
    T, n_gen, d_kv, n_sink, n_local = 64, 3, 16, 4, 16
    layer, r = 1, 6
    res, ck, cv = _decode(q, Ks, Vs, layer, r=r, top_k=1000)
    Kr = Ks[layer].copy()
    Vr = Vs[layer].copy()
    mid = slice(n_sink, T - n_local)
    Kr[mid] = oracle.reconstruct_layer(ck["A"], ck["B"], layer, d_kv)[mid]
    Vr[mid] = oracle.reconstruct_layer(cv["A"], cv["B"], layer, d_kv)[mid]
    np.testing.assert_allclose(res["out"], _dense_complex(q, Kr, Vr, T + n_gen - 1, 2), atol=1e-10)


def test_selected_subset_matches_masked_dense():
    # With a partial selection the output is attention restricted to the attended set.
    _, Ks, Vs, q = _setup(4)
    T, n_gen, d_kv, d = 64, 3, 16, 8
    layer, r, k = 0, 5, 2
    res, ck, cv = _decode(q, Ks, Vs, layer, r=r, top_k=k)
    Kr = Ks[layer].copy()
    Vr = Vs[layer].copy()
    Kr[4:48] = oracle.reconstruct_layer(ck["A"], ck["B"], layer, d_kv)[4:48]
    Vr[4:48] = oracle.reconstruct_layer(cv["A"], cv["B"], layer, d_kv)[4:48]
    p = T + n_gen - 1
    for h in range(2):
        pos = res["positions"][h]
        assert len(set(pos.tolist())) == pos.size
        for j in (2 * h, 2 * h + 1):
            qr = rope_complex(q[j], p)
            kr = rope_complex(Kr[pos][:, h * d:(h + 1) * d], pos)
            z = kr @ qr / math.sqrt(d)
            w = np.exp(z - z.max())
            np.testing.assert_allclose(res["out"][j], (w / w.sum()) @ Vr[pos][:, h * d:(h + 1) * d], atol=1e-10)
        # The selection is the top-k of the group-summed landmark scores.
        lm = oracle.landmarks(Ks[layer][:T], 2, d, 8)
        n_cand = oracle.candidate_chunks(T, 16, 8)
        sc = [sum(rope_complex(q[j], p) @ lm[h, c] for j in (2 * h, 2 * h + 1)) / math.sqrt(d)
              for c in range(n_cand)]
        np.testing.assert_allclose(res["scores"][h], sc, atol=1e-12)
        assert res["sel"][h].tolist() == brute_topk(sc, k)


def test_no_generated_tokens_query_at_T():
    # Tiny workload reading: one query at position T, nothing appended.
    _, Ks, Vs, q = _setup(5, n_gen=0)
    res, _, _ = _decode(q, Ks, Vs, 0, r=32, top_k=1000, n_gen=0)
    assert res["q_pos"] == 64
    np.testing.assert_allclose(res["out"], _dense_complex(q, Ks[0][:64], Vs[0][:64], 64, 2), atol=1e-10)


def test_split_merge_identity():
    # Partial softmax states (max, denominator, weighted sum) over a partition of the
    # attended rows merge exactly into the one-pass result.
    rng = np.random.default_rng(11)
    z = rng.standard_normal(37) * 3
    V = rng.standard_normal((37, 5))
    w = np.exp(z - z.max())
    ref = (w / w.sum()) @ V
    parts = [slice(0, 9), slice(9, 10), slice(10, 30), slice(30, 37)]
    ms = [z[s].max() for s in parts]
    ls = [np.exp(z[s] - m).sum() for s, m in zip(parts, ms)]
    os_ = [np.exp(z[s] - m) @ V[s] for s, m in zip(parts, ms)]
    M = max(ms)
    L = sum(l * np.exp(m - M) for l, m in zip(ls, ms))
    O = sum(o * np.exp(m - M) for o, m in zip(os_, ms))
    np.testing.assert_allclose(O / L, ref, atol=1e-14)


def test_value_absorption_identity():
    # sum_t p_t (a_t B) = (sum_t p_t a_t) B: reconstructing values after the softmax
    # weighting is exact.
    rng = np.random.default_rng(12)
    A = rng.standard_normal((20, 6))
    B = rng.standard_normal((6, 4))
    p = rng.random(20)
    np.testing.assert_allclose(p @ (A @ B), (p @ A) @ B, atol=1e-12)


def test_selection_override_with_padding_matches_masked_dense():
    # The `selection` argument (used when a near-tie swap makes the GPU attend a different
    # but valid chunk set) attends exactly the given chunks: -1 entries are padding, the
    # scores are still the landmark scores, and the output is attention over sink + the
    # given chunks + local window + generated tokens, written out here with the
    # complex-number RoPE.
    _, Ks, Vs, q = _setup(6)
    T, n_gen, d_kv, d, H_kv, n_sink, n_local, chunk = 64, 3, 16, 8, 2, 4, 16, 8
    layer, r, k = 1, 5, 3
    res_top, ck, cv = _decode(q, Ks, Vs, layer, r=r, top_k=k)
    # The lowest-scoring chunks (never the top-k), padded with -1 at both ends.
    worst = [np.argsort(res_top["scores"][h], kind="stable")[:2].tolist() for h in range(H_kv)]
    selection = np.array([[-1] + worst[h] + [-1] for h in range(H_kv)])
    lm = oracle.landmarks(Ks[layer][:T], H_kv, d, chunk)
    exact = [t for t in range(T + n_gen) if t < n_sink or t >= T - n_local]
    res = oracle.sr_decode_layer(
        q, T=T, n_gen=n_gen, n_kv_heads=H_kv, chunk=chunk, top_k=k, n_sink=n_sink, n_local=n_local,
        landmarks_l=lm, A_k=ck["A"], B_k_l=ck["B"][:, layer * d_kv:(layer + 1) * d_kv], A_v=cv["A"],
        B_v_l=cv["B"][:, layer * d_kv:(layer + 1) * d_kv], k_exact={t: Ks[layer][t] for t in exact},
        v_exact={t: Vs[layer][t] for t in exact}, selection=selection)
    np.testing.assert_array_equal(res["scores"], res_top["scores"])
    Kr = Ks[layer].copy()
    Vr = Vs[layer].copy()
    Kr[n_sink:T - n_local] = oracle.reconstruct_layer(ck["A"], ck["B"], layer, d_kv)[n_sink:T - n_local]
    Vr[n_sink:T - n_local] = oracle.reconstruct_layer(cv["A"], cv["B"], layer, d_kv)[n_sink:T - n_local]
    p = T + n_gen - 1
    for h in range(H_kv):
        want = set(range(n_sink)) | set(range(T - n_local, T + n_gen))
        for c in worst[h]:
            want |= set(range(c * chunk, (c + 1) * chunk))
        pos = np.array(sorted(want))
        assert res["positions"][h].tolist() == pos.tolist()
        assert res["sel"][h].tolist() == worst[h]
        for j in (2 * h, 2 * h + 1):
            qr = rope_complex(q[j], p)
            kr = rope_complex(Kr[pos][:, h * d:(h + 1) * d], pos)
            z = kr @ qr / math.sqrt(d)
            w = np.exp(z - z.max())
            np.testing.assert_allclose(res["out"][j], (w / w.sum()) @ Vr[pos][:, h * d:(h + 1) * d], atol=1e-10)
        assert not np.allclose(res["out"][2 * h], res_top["out"][2 * h])
