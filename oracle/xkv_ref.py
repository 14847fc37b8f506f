"""Plain float64 reference of the xKV hot path (test infrastructure only).

Sources (page titles as published):

* [xKV blog]  "xKV大模型压缩秘籍：跨层共享..." (jsqmd.com explainer of the ICLR 2026
  xKV paper), sections "xKV 到底做了什么？" (grouping, horizontal concatenation,
  shared basis A, per-layer B_l) and "仅仅压缩还不够，xKV 还做了'选择性重建'"
  (Selective Reconstruction with a landmark-guided top-k chunk selector).
* [xKV abstract]  "xKV: Cross-Layer KV-Cache Compression via Aligned Singular
  Vector Extraction" (paperdance.org, arXiv 2503.18893), abstract.
* [KV-CoRE]  "KV-CoRE: Benchmarking Data-Dependent Low-Rank Compressibility of
  KV-Caches in LLMs" (gist.science), section 2.A: the uncentred covariance
  C = sum_t k_t^T k_t and its eigendecomposition give the singular values and
  right singular vectors.
* [KQ-SVD]  "KQ-SVD: ..." (bittide.aicompass.dev article, arXiv 2512.05916),
  section 3.1 (SVD notation, truncation), section 3.2 (decode: append k_T,
  v_T, then h_T = softmax(q_T K^T / sqrt(d)) V) and section 3.3 (Eckart-Young:
  the rank-R projector V V^T of the right singular vectors is optimal; the
  cache stores K V).

Readings where the pages are silent (each repeated where it is used):

* RoPE is the rotate-half form on pairs (i, i + d/2) with frequencies
  theta**(-2i/d), theta = 10000; the phase t*f_i is formed in float64.
  Keys are compressed before RoPE and rotated after reconstruction.
* No centring; K and V are factored separately at the same rank; all KV heads
  of a layer are concatenated (d_kv = H_kv * d).
* A landmark is the mean of the post-RoPE original keys of one chunk.
* Candidates are the chunks not wholly inside the local window; the attended
  set is the union of sink, selected chunks, local window and generated
  tokens, each position once.  Rows in the sink, local and generated ranges
  are exact; every other attended row is reconstructed.
* A KV head's chunk score is the sum over its query group of the scaled dot
  products; ties in the top-k go to the lower chunk index.
"""
from __future__ import annotations

import numpy as np

ROPE_THETA = 10000.0


# ---------------------------------------------------------------------------
# RoPE (applied after reconstruction; keys are compressed pre-RoPE, following
# the ShadowKV precedent recalled in KQ-SVD section 2)
# ---------------------------------------------------------------------------
def rope(x, pos, theta: float = ROPE_THETA) -> np.ndarray:
    """Rotate-half RoPE of ``x`` (..., d) at integer position(s) ``pos``.

    Pair (x_i, x_{i+d/2}) is rotated by the angle pos * theta**(-2 i / d).
    ``pos`` broadcasts against ``x.shape[:-1]``.  The angle is float64.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * freq
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


# ---------------------------------------------------------------------------
# Compression of one group side  ([xKV blog] "xKV 到底做了什么？")
# ---------------------------------------------------------------------------
def group_matrix(layers) -> np.ndarray:
    """X = [K_l1 | ... | K_lG]: the group's layers concatenated horizontally (T x G*d_kv)."""
    return np.concatenate([np.asarray(K, dtype=np.float64) for K in layers], axis=1)


def gram(X) -> np.ndarray:
    """C = X^T X, the uncentred covariance of the rows ([KV-CoRE] 2.A)."""
    X = np.asarray(X, dtype=np.float64)
    return X.T @ X


def eig_desc(C):
    """Eigenvalues (descending) and matching orthonormal eigenvectors of symmetric C."""
    w, V = np.linalg.eigh(C)
    order = np.argsort(w)[::-1]
    return w[order], V[:, order]


def compress_group(layers, r: int) -> dict:
    """Factor one group side: X ~= A B with a shared token basis A and per-layer B_l.

    X (T x n) is the horizontal concatenation.  V_r holds the top-r right
    singular vectors of X, obtained as the top-r eigenvectors of C = X^T X
    ([KV-CoRE] 2.A).  A = X V_r (T x r) is the shared basis; B = V_r^T (r x n)
    and B_l = B[:, l*d_kv:(l+1)*d_kv] reconstructs layer l as A B_l
    ([xKV blog] "xKV 到底做了什么？"; the projector V_r V_r^T is the
    Eckart-Young optimum of [KQ-SVD] 3.3).
    """
    X = group_matrix(layers)
    lam, V = eig_desc(gram(X))
    Vr = V[:, :r]
    A = X @ Vr
    B = Vr.T
    resid = X - A @ B
    return dict(X=X, A=A, B=B, Vr=Vr, eigvals=lam,
                rel_err=float(np.linalg.norm(resid) / np.linalg.norm(X)))


def reconstruct_layer(A, B, layer: int, d_kv: int) -> np.ndarray:
    """Layer ``layer`` of the group rebuilt from the shared basis: A B_l."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    return A @ B[:, layer * d_kv:(layer + 1) * d_kv]


def landmarks(K_layer, n_kv_heads: int, head_dim: int, chunk: int,
              theta: float = ROPE_THETA, pos0: int = 0) -> np.ndarray:
    """Per-chunk landmark of every KV head: the mean of the post-RoPE original keys.

    Returns (H_kv, T/chunk, d).  Chunks start at row 0 and have ``chunk`` tokens; row t
    sits at position pos0 + t (pos0 > 0 for rows appended after a prefix).
    """
    K = np.asarray(K_layer, dtype=np.float64)
    T = K.shape[0]
    n_chunks = T // chunk
    out = np.zeros((n_kv_heads, n_chunks, head_dim))
    for h in range(n_kv_heads):
        rot = rope(K[:, h * head_dim:(h + 1) * head_dim], pos0 + np.arange(T), theta)
        for c in range(n_chunks):
            out[h, c] = rot[c * chunk:(c + 1) * chunk].mean(axis=0)
    return out


def append_tokens(new_layers, Bt, pos0: int, *, n_kv_heads: int | None = None, head_dim: int | None = None,
                  chunk: int | None = None, theta: float = ROPE_THETA, with_landmarks: bool = False) -> dict:
    """Rows appended after a compressed prefix (multi-turn growth), projected onto the
    stored basis: a_new = [x_l1 | ... | x_lG] V_r with V_r = Bt as stored (n x r), so that
    A_new B_l reconstructs them like the prefix rows ([xKV blog] "xKV 到底做了什么？": the
    shared token basis A = X V_r; the pages name the compression of generated tokens as a
    limitation).  Landmarks of the new chunks use positions pos0 + t."""
    X = group_matrix(new_layers)
    out = dict(A=X @ np.asarray(Bt, dtype=np.float64))
    if with_landmarks:
        out["landmarks"] = [landmarks(x, n_kv_heads, head_dim, chunk, theta, pos0) for x in new_layers]
    return out


# ---------------------------------------------------------------------------
# Selective Reconstruction decode ([xKV blog] "选择性重建"; [KQ-SVD] 3.2)
# ---------------------------------------------------------------------------
def candidate_chunks(T: int, n_local: int, chunk: int) -> int:
    """Number of candidate chunks: every chunk not wholly inside the local window."""
    return -(-(T - n_local) // chunk)


def landmark_scores(q_rot, lm_head, scale: float) -> np.ndarray:
    """Chunk scores of one KV head: sum over its query heads of scale * (q_j . m_c).

    ``q_rot`` (g x d) are the group's post-RoPE queries, ``lm_head`` (C x d).
    """
    q_rot = np.asarray(q_rot, dtype=np.float64)
    lm_head = np.asarray(lm_head, dtype=np.float64)
    return scale * (lm_head @ q_rot.T).sum(axis=1)


def select_topk(scores, k: int) -> np.ndarray:
    """The k highest-scoring chunk ids, ties to the lower id, returned ascending.

    With fewer than k candidates every candidate is selected.
    """
    s = np.asarray(scores, dtype=np.float64)
    order = np.lexsort((np.arange(s.size), -s))   # by score descending, then id ascending
    return np.sort(order[:k])


def attended_positions(sel, T: int, n_sink: int, n_local: int, n_gen: int, chunk: int):
    """Attended set: sink + selected chunks + local window + generated tokens (a set union)."""
    pos = set(range(min(n_sink, T)))
    for c in np.asarray(sel).tolist():
        pos.update(range(c * chunk, min((c + 1) * chunk, T)))
    pos.update(range(max(T - n_local, 0), T))
    pos.update(range(T, T + n_gen))
    return np.array(sorted(pos), dtype=np.int64)


def _softmax_rows(logits):
    m = logits.max(axis=-1, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=-1, keepdims=True)


def sr_decode_layer(q, *, T: int, n_gen: int, n_kv_heads: int, chunk: int, top_k: int,
                    n_sink: int, n_local: int, landmarks_l, A_k, B_k_l,
                    k_exact, v_exact, A_v=None, B_v_l=None, V_full=None,
                    scale: float | None = None, theta: float = ROPE_THETA, selection=None) -> dict:
    """One decode step of one layer with Selective Reconstruction.

    q          (H_q x d) pre-RoPE query at position p = T + n_gen - 1 (p = T if n_gen == 0)
    landmarks_l (H_kv x T/chunk x d)
    A_k (T x r_k), B_k_l (r_k x d_kv)       compressed keys of this layer (pre-RoPE)
    A_v, B_v_l                               compressed values, or V_full (T x d_kv) when
                                             values are kept exact
    k_exact, v_exact  dicts {position: d_kv row} for every sink, local-window and
                      generated position (pre-RoPE keys)
    selection  optional (H_kv x k) chunk ids to attend instead of the top-k (ids < 0 are
               ignored); the scores are still computed and returned

    Returns out (H_q x d), sel (H_kv x min(k, C)) ascending chunk ids, scores (H_kv x C)
    and the attended positions of each KV head.
    """
    q = np.asarray(q, dtype=np.float64)
    H_q, d = q.shape
    grp = H_q // n_kv_heads
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    p = T + n_gen - 1 if n_gen > 0 else T
    q_rot = rope(q, p, theta)
    n_cand = candidate_chunks(T, n_local, chunk)
    A_k = np.asarray(A_k, dtype=np.float64)
    B_k_l = np.asarray(B_k_l, dtype=np.float64)
    if V_full is None:
        A_v = np.asarray(A_v, dtype=np.float64)
        B_v_l = np.asarray(B_v_l, dtype=np.float64)

    out = np.zeros((H_q, d))
    sels, all_scores, all_pos = [], [], []
    for h in range(n_kv_heads):
        qh = q_rot[h * grp:(h + 1) * grp]
        s = landmark_scores(qh, np.asarray(landmarks_l)[h, :n_cand], scale)
        sel = select_topk(s, top_k)
        if selection is not None:
            sel = np.array([c for c in np.asarray(selection[h]).tolist() if c >= 0], dtype=np.int64)
        pos = attended_positions(sel, T, n_sink, n_local, n_gen, chunk)
        cols = slice(h * d, (h + 1) * d)
        keys = np.zeros((pos.size, d))
        vals = np.zeros((pos.size, d))
        for i, t in enumerate(pos.tolist()):
            exact = t < n_sink or t >= T - n_local
            if exact:
                k_row = np.asarray(k_exact[t], dtype=np.float64)[cols]
                v_row = np.asarray(v_exact[t], dtype=np.float64)[cols]
            else:
                k_row = A_k[t] @ B_k_l[:, cols]
                if V_full is None:
                    v_row = A_v[t] @ B_v_l[:, cols]
                else:
                    v_row = np.asarray(V_full[t], dtype=np.float64)[cols]
            keys[i] = rope(k_row, t, theta)
            vals[i] = v_row
        w = _softmax_rows(scale * qh @ keys.T)          # (grp x |P_h|)
        out[h * grp:(h + 1) * grp] = w @ vals
        sels.append(sel)
        all_scores.append(s)
        all_pos.append(pos)
    return dict(out=out, sel=np.stack(sels), scores=np.stack(all_scores), positions=all_pos,
                q_pos=p)


def dense_decode(q, K_full, V_full, p: int, n_kv_heads: int, scale: float | None = None,
                 theta: float = ROPE_THETA) -> np.ndarray:
    """Full attention of the query at position p over rows 0..K_full.shape[0]-1.

    K_full, V_full (N x d_kv) are pre-RoPE; row t sits at position t ([KQ-SVD] 3.2).
    """
    q = np.asarray(q, dtype=np.float64)
    H_q, d = q.shape
    grp = H_q // n_kv_heads
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    K_full = np.asarray(K_full, dtype=np.float64)
    V_full = np.asarray(V_full, dtype=np.float64)
    N = K_full.shape[0]
    q_rot = rope(q, p, theta)
    out = np.zeros((H_q, d))
    for h in range(n_kv_heads):
        cols = slice(h * d, (h + 1) * d)
        keys = rope(K_full[:, cols], np.arange(N), theta)
        w = _softmax_rows(scale * q_rot[h * grp:(h + 1) * grp] @ keys.T)
        out[h * grp:(h + 1) * grp] = w @ V_full[:, cols]
    return out


# ---------------------------------------------------------------------------
# Rank diagnostics (the eigenvalues of C = X^T X are the squared singular
# values of X, [KV-CoRE] 2.A)
# ---------------------------------------------------------------------------
def numerical_rank(eigvals, rel_tol: float | None = None) -> int:
    """Count of singular values sigma_i = sqrt(lambda_i) above rel_tol * sigma_1.

    The pages call r "the actual rank"; the reading here is the numerical rank
    with the usual tolerance n * eps (relative to the largest singular value).
    """
    lam = np.clip(np.asarray(eigvals, dtype=np.float64), 0.0, None)
    sv = np.sqrt(np.sort(lam)[::-1])
    if sv.size == 0 or sv[0] == 0.0:
        return 0
    tol = (sv.size * np.finfo(np.float64).eps) if rel_tol is None else rel_tol
    return int(np.count_nonzero(sv > tol * sv[0]))


def effective_rank(eigvals, rel_tol: float | None = None) -> float:
    """Effective rank: the exponential of the Shannon entropy (natural log) of the
    singular values normalised to sum to one, over the numerical rank
    ([KV-CoRE] 2.B: a rank measured by the entropy of the singular value
    distribution).  Reading: the distribution is sigma_i / sum_j sigma_j (singular
    values, not their squares)."""
    lam = np.clip(np.asarray(eigvals, dtype=np.float64), 0.0, None)
    sv = np.sqrt(np.sort(lam)[::-1])
    k = numerical_rank(lam, rel_tol)
    if k == 0:
        return 0.0
    p = sv[:k] / sv[:k].sum()
    return float(np.exp(-np.sum(p * np.log(p))))


def ner(eigvals, rel_tol: float | None = None) -> float:
    """Normalised effective rank erank / r, r the numerical rank ([KV-CoRE] 2.B);
    it lies in [1/r, 1]."""
    k = numerical_rank(eigvals, rel_tol)
    return effective_rank(eigvals, rel_tol) / k if k else 0.0


def energy_rank(eigvals, frac: float = 0.95, total: float | None = None) -> int:
    """Smallest k whose k largest eigenvalues hold at least `frac` of the total
    ([xKV blog] figure 2(c): the rank that keeps 95 % of the cumulative
    eigenvalues).  `total` defaults to the sum of the given eigenvalues (a full
    spectrum); with a partial spectrum pass trace(C).  Returns -1 when the given
    eigenvalues do not reach the target."""
    lam = np.sort(np.clip(np.asarray(eigvals, dtype=np.float64), 0.0, None))[::-1]
    csum = np.cumsum(lam)
    # The total of a full spectrum is the last cumulative sum (one summation order for
    # both, so that frac = 1 is reached exactly at the last nonzero eigenvalue).
    tot = (csum[-1] if csum.size else 0.0) if total is None else float(total)
    if tot <= 0.0:
        return 0
    hit = np.nonzero(csum >= frac * tot)[0]
    return int(hit[0]) + 1 if hit.size else -1


# ---------------------------------------------------------------------------
# Adaptive rank: per-side ranks from the spectra at a fixed total budget
# ([KV-CoRE] implications: compressibility differs across layers and should
# guide a layer-aware compression strategy; [xKV blog] figure 5: the rank that
# pays off differs by task)
# ---------------------------------------------------------------------------
def allocate_ranks(spectra, budget: int, granule: int, r_min: int, r_max: int):
    """Ranks r_s (multiples of `granule` in [r_min, r_max]) with sum r_s <= budget that
    keep the most energy sum_s sum_{i < r_s} lambda_i^(s), i.e. (Eckart-Young, [KQ-SVD]
    3.3) that minimise the total squared reconstruction error sum_s sum_{i >= r_s}
    lambda_i^(s) of the sides' rank-r_s truncations.  `spectra[s]` holds side s's
    leading eigenvalues (at least r_max, any order).  Exact dynamic programme over the
    sides.  Returns (ranks, kept energy); ValueError when even r_min everywhere does
    not fit the budget."""
    S = len(spectra)
    if granule <= 0 or r_min % granule or r_max % granule or r_min > r_max:
        raise ValueError("ranks must be multiples of the granule with r_min <= r_max")
    kmin, kmax, B = r_min // granule, r_max // granule, budget // granule
    if S * kmin > B:
        raise ValueError("budget below r_min on every side")
    # kept[s][k]: energy of side s's first k granules.
    kept = []
    for lam in spectra:
        lam = np.sort(np.clip(np.asarray(lam, dtype=np.float64), 0.0, None))[::-1]
        if lam.size < r_max:
            raise ValueError("each spectrum needs at least r_max values")
        kept.append([float(np.sum(lam[:k * granule])) for k in range(kmax + 1)])
    NEG = -np.inf
    best = [[NEG] * (B + 1) for _ in range(S + 1)]   # best[s][b]: first s sides, b granules
    pick = [[-1] * (B + 1) for _ in range(S + 1)]
    best[0][0] = 0.0
    for s in range(S):
        for b in range(B + 1):
            if best[s][b] == NEG:
                continue
            for k in range(kmin, kmax + 1):
                if b + k > B:
                    break
                v = best[s][b] + kept[s][k]
                if v > best[s + 1][b + k]:
                    best[s + 1][b + k] = v
                    pick[s + 1][b + k] = k
    b_end = int(np.argmax(best[S]))
    total = best[S][b_end]
    ranks = [0] * S
    b = b_end
    for s in range(S, 0, -1):
        k = pick[s][b]
        ranks[s - 1] = k * granule
        b -= k
    return ranks, total
