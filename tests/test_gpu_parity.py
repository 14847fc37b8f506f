"""HIP path vs the float64 oracle on identical seeded inputs (small and ragged sizes).

Tolerances (parity protocol): chunk sets exact outside a 1e-3 near-tie band of
the k-th score; ||P_gpu - P_ref||_F <= 1e-3; reconstruction relative error
within 1e-4 of the oracle's; attention relative L2 <= 1e-2 and max abs <= 2e-2
for bf16, <= 1e-4 relative for float32.  Decode parity gives both sides the same
cache, built by the oracle's own factorisation and rounded to the storage dtype,
so the only difference is arithmetic precision and the tighter bound 1e-3 is
asserted too.
"""
import math

import numpy as np
import pytest
import torch

import kv_cache_cross_amd as xk
import oracle
from parity_util import (ATT_ABS_BF16, ATT_REL_BF16, ATT_REL_F32, PROJ_TOL, RECON_TOL, attention_errors,
                         check_selection, f64, projector_distance, tail_rows)
from synth import gaussian, make_workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def ctx():
    c = xk.Context(0)
    yield c
    c.close()


# ----------------------------------------------------------------------------- Gram
@pytest.mark.parametrize("T,G,d_kv,dt", [(256, 2, 64, torch.float32), (1000, 2, 256, torch.bfloat16),
                                          (777, 3, 136, torch.bfloat16), (64, 1, 8, torch.bfloat16),
                                          (4133, 4, 128, torch.bfloat16), (25810, 4, 128, torch.bfloat16),
                                          (65536, 2, 256, torch.bfloat16)])
def test_gram(T, G, d_kv, dt):
    # The long cases sum 51 and 128 matrix-core partials of 512 tokens (the first with a
    # ragged last slab) into the compensated float32 totals: the same bar as the short ones.
    log(f"gram T={T} G={G} d_kv={d_kv} {dt}")
    layers = [gaussian((T, d_kv), seed=100 + l, scale=1.5, dtype=dt, device=DEV) for l in range(G)]
    C = xk.gram(layers)
    torch.cuda.synchronize()
    ref = oracle.gram(oracle.group_matrix([f64(x) for x in layers]))
    err = np.linalg.norm(f64(C) - ref) / np.linalg.norm(ref)
    log(f"  rel Frobenius {err:.2e}")
    assert err <= (1e-13 if dt == torch.float32 else 2e-6)
    np.testing.assert_array_equal(f64(C), f64(C).T)


# ----------------------------------------------------------------------------- top-k
@pytest.mark.parametrize("n_cand,k", [(1, 1), (7, 3), (300, 8), (8184, 256), (15352, 384), (1000, 1000),
                                      (50, 64), (4097, 1), (2048, 2047), (30000, 512)])
def test_topk_bit_exact(n_cand, k):
    log(f"topk n_cand={n_cand} k={k}")
    rows, ld = 6, n_cand + 5
    g = torch.Generator().manual_seed(n_cand * 31 + k)
    coarse = (torch.randint(-40, 40, (rows, ld), generator=g).float() / 8.0)   # many exact ties
    fine = torch.randn((rows, ld), generator=g)
    scores = torch.where(torch.rand((rows, ld), generator=g) < 0.5, coarse, fine)
    scores[1] = scores[1].abs() * 0.0 + 0.25                                    # one row all equal
    # Infinite extremes; a range near the float limit; denormals mixed with -0.0 and +0.0.
    scores[3, ::7] = float("inf")
    scores[3, 3::11] = float("-inf")
    scores[4] = fine[4] * 3e37
    tiny = torch.randint(-3, 4, (ld,), generator=g).float() * 1e-45
    scores[5] = torch.where(torch.rand(ld, generator=g) < 0.3, torch.tensor(-0.0), tiny)
    sel = xk.topk(scores.to(DEV), n_cand, k).cpu().numpy()
    for r in range(rows):
        ref = oracle.select_topk(scores[r, :n_cand].double().numpy(), k).tolist()
        ref = ref + [-1] * (k - len(ref))
        assert sel[r].tolist() == ref


# ----------------------------------------------------------------------------- compression
def _check_side(ctx, layers, r, *, with_lm, n_kv_heads, head_dim, chunk, label):
    T = layers[0].shape[0]
    out = xk.compress(ctx, [layers], r=r, n_kv_heads=n_kv_heads, head_dim=head_dim, chunk=chunk,
                      landmarks=[with_lm], keep_vr64=True)[0]
    torch.cuda.synchronize()
    ref = oracle.compress_group([f64(x) for x in layers], r)
    Vg = f64(out["Vr64"])
    dP = projector_distance(Vg, ref["Vr"])
    orth = np.abs(Vg.T @ Vg - np.eye(r)).max()
    X = ref["X"]
    Ag, Bg = f64(out["A"]), f64(out["Bt"]).T
    rel_gpu = np.linalg.norm(X - Ag @ Bg) / np.linalg.norm(X)
    lam_err = np.max(np.abs(out["eigvals"] - ref["eigvals"][:r]) / ref["eigvals"][:r])
    log(f"  {label}: ||dP||_F={dP:.2e} orth={orth:.1e} rel_err gpu={rel_gpu:.6f} ref={ref['rel_err']:.6f} "
        f"eig rel={lam_err:.1e} stats={out['stats']}")
    # stats["err_est"] bounds the iteration error against the GPU's own Gram; the Gram's
    # rounding (a floor of ~2e-4 here) is outside what that estimate can see.
    assert out["stats"]["err_est"] <= 1e-4
    assert dP <= PROJ_TOL
    assert orth <= 1e-10
    assert abs(rel_gpu - ref["rel_err"]) <= RECON_TOL
    # Eigenvalue bar (not fixed by the pages; derived from the Gram's arithmetic): the
    # Gram sums up to 8192 tokens in float32, 512 matrix-core accumulations of 16 tokens,
    # each rounded to 2^-24 of the running partial; a random walk over them gives entry
    # errors of ~sqrt(512) * 2^-24 ~ 1.3e-6 relative, which Weyl's bound carries to the
    # eigenvalues.  1e-5 leaves a margin of ~5 over the ~2e-6 observed.
    assert lam_err <= 1e-5
    if with_lm:
        d_kv = layers[0].shape[1]
        for l, K in enumerate(layers):
            lm_ref = oracle.landmarks(f64(K), n_kv_heads, head_dim, chunk)
            lm = f64(out["landmarks"][l])
            if K.dtype == torch.float32:
                np.testing.assert_allclose(lm, lm_ref, rtol=1e-5, atol=1e-5 * np.abs(lm_ref).max())
            else:  # bf16 storage: half an ulp of the stored value plus float32 sums
                np.testing.assert_allclose(lm, lm_ref, rtol=2 ** -8, atol=1e-3 * np.abs(lm_ref).max())
    return out, ref


def test_compress_tiny_fp32(ctx):
    wl = make_workload("tiny", device=DEV)
    c = wl.cfg
    for side in ("K", "V"):
        _check_side(ctx, wl.group_kv(0, side, 0), c.rank, with_lm=(side == "K"), n_kv_heads=c.n_kv_heads,
                    head_dim=c.head_dim, chunk=c.chunk, label=f"tiny {side}")


MINI = dict(T=2000, n_layers=4, n_kv_heads=2, n_q_heads=8, rank=128, latent_rank=192, top_k=32)


def test_compress_mini_bf16_ragged(ctx):
    # T = 2000 is not a multiple of the 64-token slab or the 128-row tiles; n = 1024.
    wl = make_workload("llama16k", device=DEV, **MINI)
    c = wl.cfg
    for side in ("K", "V"):
        _check_side(ctx, wl.group_kv(0, side, 0), c.rank, with_lm=(side == "K"), n_kv_heads=c.n_kv_heads,
                    head_dim=c.head_dim, chunk=c.chunk, label=f"mini {side}")


def test_compress_batched_sides_match_single(ctx):
    # Several sides in one call give the same factorisation as one side per call.
    wl = make_workload("llama16k", device=DEV, **dict(MINI, T=512))
    c = wl.cfg
    sides = [wl.group_kv(0, "K", 0), wl.group_kv(0, "V", 0)]
    kw = dict(r=c.rank, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim, chunk=c.chunk, keep_vr64=True)
    both = xk.compress(ctx, sides, landmarks=[True, False], **kw)
    one = xk.compress(ctx, sides[1:], landmarks=[False], **kw)
    torch.cuda.synchronize()
    assert torch.equal(both[1]["A"], one[0]["A"]) and torch.equal(both[1]["Bt"], one[0]["Bt"])
    assert torch.equal(both[1]["Vr64"], one[0]["Vr64"])


def test_compress_rank_deficient_reports_breakdown(ctx):
    # X with only 8 non-zero columns has rank 8 and cannot support a 24-column iteration
    # block: CholeskyQR must report the breakdown instead of returning a basis.
    T, d = 256, 64
    K0 = torch.zeros((T, d))
    K0[:, :8] = gaussian((T, 8), seed=5, dtype=torch.float32)
    layers = [K0.to(DEV), torch.zeros((T, d), device=DEV)]
    with pytest.raises(xk.XkvError) as e:
        xk.compress(ctx, [layers], r=16, n_kv_heads=1, head_dim=64, landmarks=[False])
    assert e.value.code == xk._lib.XKV_ENUMERIC


# ----------------------------------------------------------------------------- decode
def oracle_cache(wl, r, layer):
    """The compressed cache of group 0 of sequence 0 as the oracle builds it (float64
    truncated SVD and landmarks of the original keys), rounded to the workload's storage
    dtype.  Both the GPU decode and the oracle decode consume these same tensors, so no
    oracle input comes from the GPU path."""
    c = wl.cfg
    Ks = [f64(x) for x in wl.group_kv(0, "K", 0)]
    Vs = [f64(x) for x in wl.group_kv(0, "V", 0)]
    ok, ov = oracle.compress_group(Ks, r), oracle.compress_group(Vs, r)
    lm = oracle.landmarks(Ks[layer], c.n_kv_heads, c.head_dim, c.chunk, c.rope_theta)
    dt, d_kv = c.torch_dtype, c.d_kv
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(DEV)
    return dict(A_k=to(ok["A"]), Bt_k=to(ok["B"][:, layer * d_kv:(layer + 1) * d_kv].T),
                A_v=to(ov["A"]), Bt_v=to(ov["B"][:, layer * d_kv:(layer + 1) * d_kv].T), lm=to(lm))


def _run_decode_case(ctx, wl, *, steps, top_k=None, r=None, values="compressed", layer=0, label=""):
    """Run `steps` decode steps of one layer of group 0, sequence 0 on the GPU and compare
    each with the oracle on the same inputs (the oracle-built cache, exact tails, queries
    and appended tokens)."""
    c = wl.cfg
    top_k = c.top_k if top_k is None else top_k
    r = c.rank if r is None else r
    Ks, Vs = wl.group_kv(0, "K", 0), wl.group_kv(0, "V", 0)
    cache = oracle_cache(wl, r, layer)
    d_kv, T = c.d_kv, c.T
    r_v = r if values == "compressed" else 0
    dec = xk.LayerDecoder(ctx, batch=1, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim,
                          T=T, chunk=c.chunk, top_k=top_k, n_sink=c.n_sink, n_local=c.n_local, r_k=r, r_v=r_v,
                          dtype=c.torch_dtype, device=DEV, max_gen=steps)
    rows = tail_rows(T, c.n_sink, c.n_local)
    n_tail = len(rows) + steps
    k_tail = torch.zeros((n_tail, d_kv), dtype=c.torch_dtype, device=DEV)
    v_tail = torch.zeros_like(k_tail)
    k_tail[: len(rows)] = Ks[layer][rows]
    v_tail[: len(rows)] = Vs[layer][rows]
    Kl, Vl = f64(Ks[layer]), f64(Vs[layer])
    k_exact = {t: Kl[t] for t in rows}
    v_exact = {t: Vl[t] for t in rows}
    A_k, Bt_k, A_v, Bt_v, lm = cache["A_k"], cache["Bt_k"], cache["A_v"], cache["Bt_v"], cache["lm"]
    worst = (0.0, 0.0)
    for s in range(steps):
        n_gen = s + 1 if c.append else 0
        q = wl.query(0, layer, s)
        kn = vn = None
        if c.append:
            kn, vn = wl.new_token(0, "K", layer, s), wl.new_token(0, "V", layer, s)
            k_exact[T + s], v_exact[T + s] = f64(kn), f64(vn)
        args = dec.args(n_gen=n_gen, q=q, A_k=A_k, Bt_k=Bt_k, A_v=A_v if r_v else None,
                        Bt_v=Bt_v if r_v else None, V_full=None if r_v else Vs[layer],
                        landmarks=lm, k_tail=k_tail, v_tail=v_tail, k_new=kn, v_new=vn)
        out = dec.decode(args)
        torch.cuda.synchronize()
        kw = dict(T=T, n_gen=n_gen, n_kv_heads=c.n_kv_heads, chunk=c.chunk, top_k=top_k, n_sink=c.n_sink,
                  n_local=c.n_local, landmarks_l=f64(lm), A_k=f64(A_k), B_k_l=f64(Bt_k).T,
                  k_exact=k_exact, v_exact=v_exact)
        if r_v:
            kw.update(A_v=f64(A_v), B_v_l=f64(Bt_v).T)
        else:
            kw.update(V_full=Vl)
        ref = oracle.sr_decode_layer(f64(q), **kw)
        sel = dec.sel.cpu().numpy()[0]
        swaps = 0
        for h in range(c.n_kv_heads):
            swaps += check_selection(sel[h], ref["scores"][h], top_k)
        if swaps:
            ref = oracle.sr_decode_layer(f64(q), selection=sel, **kw)
        rel, mx = attention_errors(f64(out)[0], ref["out"])
        worst = (max(worst[0], rel), max(worst[1], mx))
        if c.dtype == "fp32":
            assert rel <= ATT_REL_F32, (s, rel)
        else:
            assert rel <= 1e-3 and mx <= ATT_ABS_BF16, (s, rel, mx)
    # The tail now holds the appended tokens exactly.
    if c.append:
        for s in range(steps):
            assert torch.equal(k_tail[len(rows) + s], wl.new_token(0, "K", layer, s))
    log(f"  {label}: worst rel L2 {worst[0]:.2e}, max abs {worst[1]:.2e}")
    return worst


def test_decode_tiny_fp32(ctx):
    wl = make_workload("tiny", device=DEV)
    for layer in range(2):
        _run_decode_case(ctx, wl, steps=1, layer=layer, label=f"tiny layer {layer}")


def test_decode_mini_bf16_steps(ctx):
    wl = make_workload("llama16k", device=DEV, **MINI)
    _run_decode_case(ctx, wl, steps=4, layer=2, label="mini bf16 xKV-SR")


def test_select_then_attend_honours_edited_selection(ctx):
    # The separate entry points hand the selection over through `sel`: xkv_sr_select
    # writes the top-k, xkv_sr_attend attends over whatever `sel` holds.  Here the
    # selection is replaced, between the two calls, by the k lowest-scoring candidate
    # chunks (ascending ids), and the output must match the oracle on that edited set.
    wl = make_workload("llama16k", device=DEV, **MINI)
    c = wl.cfg
    layer = 1
    cache = oracle_cache(wl, c.rank, layer)
    Ks, Vs = wl.group_kv(0, "K", 0), wl.group_kv(0, "V", 0)
    dec = xk.LayerDecoder(ctx, batch=1, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim,
                          T=c.T, chunk=c.chunk, top_k=c.top_k, n_sink=c.n_sink, n_local=c.n_local, r_k=c.rank,
                          r_v=c.rank, dtype=c.torch_dtype, device=DEV, max_gen=1)
    rows = tail_rows(c.T, c.n_sink, c.n_local)
    k_tail = torch.zeros((len(rows) + 1, c.d_kv), dtype=c.torch_dtype, device=DEV)
    v_tail = torch.zeros_like(k_tail)
    k_tail[: len(rows)] = Ks[layer][rows]
    v_tail[: len(rows)] = Vs[layer][rows]
    q = wl.query(0, layer, 0)
    kn, vn = wl.new_token(0, "K", layer, 0), wl.new_token(0, "V", layer, 0)
    args = dec.args(n_gen=1, q=q, A_k=cache["A_k"], Bt_k=cache["Bt_k"], A_v=cache["A_v"], Bt_v=cache["Bt_v"],
                    landmarks=cache["lm"], k_tail=k_tail, v_tail=v_tail, k_new=kn, v_new=vn)
    Kl, Vl = f64(Ks[layer]), f64(Vs[layer])
    kw = dict(T=c.T, n_gen=1, n_kv_heads=c.n_kv_heads, chunk=c.chunk, top_k=c.top_k, n_sink=c.n_sink,
              n_local=c.n_local, landmarks_l=f64(cache["lm"]), A_k=f64(cache["A_k"]), B_k_l=f64(cache["Bt_k"]).T,
              A_v=f64(cache["A_v"]), B_v_l=f64(cache["Bt_v"]).T,
              k_exact={**{t: Kl[t] for t in rows}, c.T: f64(kn)}, v_exact={**{t: Vl[t] for t in rows}, c.T: f64(vn)})
    ref = oracle.sr_decode_layer(f64(q), **kw)
    dec.select(args)
    torch.cuda.synchronize()
    sel = dec.sel.cpu().numpy()[0]
    for h in range(c.n_kv_heads):
        check_selection(sel[h], ref["scores"][h], c.top_k)
    edited = np.stack([np.sort(np.argsort(ref["scores"][h], kind="stable")[: c.top_k])
                       for h in range(c.n_kv_heads)]).astype(np.int32)
    dec.sel.copy_(torch.from_numpy(edited[None]).to(DEV))
    out = dec.attend(args)
    torch.cuda.synchronize()
    ref_e = oracle.sr_decode_layer(f64(q), selection=edited, **kw)
    rel, mx = attention_errors(f64(out)[0], ref_e["out"])
    log(f"edited selection: rel L2 {rel:.2e}, max abs {mx:.2e}")
    assert rel <= 1e-3 and mx <= ATT_ABS_BF16, (rel, mx)
    assert torch.equal(dec.sel.cpu(), torch.from_numpy(edited[None]))   # attend left `sel` as given


def test_decode_exact_tail_crosses_tiles(ctx):
    # 4 sink + 122 local rows plus 1..4 generated tokens: the exact tail grows from 127 to
    # 130 rows and crosses from eight 16-row tiles into a ninth.
    wl = make_workload("llama16k", device=DEV, **dict(MINI, n_local=122))
    _run_decode_case(ctx, wl, steps=4, layer=0, label="exact tail 127..130 rows")


@pytest.mark.parametrize("rank,values", [(384, "compressed"), (1024, "compressed"), (384, "exact"),
                                         (1024, "exact")])
def test_decode_mini_bf16_several_rank_chunks(ctx, rank, values):
    # Ranks past one rank chunk of the matrix-core attend kernel: 1024 = two chunks of
    # 512 and 384 = three of 128, so the keys are rebuilt chunk by chunk (and with
    # compressed values the rank-space value sums too); compressed and exact values.
    wl = make_workload("llama16k", device=DEV, **dict(MINI, rank=rank))
    _run_decode_case(ctx, wl, steps=2, values=values, layer=2, label=f"mini bf16 r={rank} {values} values")


@pytest.mark.parametrize("rank", [128, 96])
def test_decode_mini_bf16_exact_values(ctx, rank):
    # xK-SR variant with GPU-resident exact values (r_v = 0): rank 128 takes the
    # matrix-core key path with value-space partials, rank 96 the generic kernel.
    wl = make_workload("llama16k", device=DEV, **dict(MINI, rank=rank))
    _run_decode_case(ctx, wl, steps=2, values="exact", layer=1, label=f"mini bf16 xK-SR r={rank}")


def test_decode_xk_sr_gqa7_many_splits(ctx):
    # xK-SR on the matrix-core path with a 7-query group and 41 attend blocks per head.
    wl = make_workload("qwen122k", device=DEV, T=4096, n_layers=4, rank=128, latent_rank=192, top_k=320)
    _run_decode_case(ctx, wl, steps=2, values="exact", label="qwen-shaped xK-SR")


def test_decode_gqa7_qwen_shape(ctx):
    # Qwen-like grouping: 7 query heads per KV head, rank 256.
    wl = make_workload("qwen122k", device=DEV, T=1024, n_layers=4, rank=256, latent_rank=384, top_k=48)
    _run_decode_case(ctx, wl, steps=2, layer=3, label="qwen-shape bf16")


def test_decode_topk_exceeds_candidates(ctx):
    # Every candidate selected: each prefix position is attended exactly once.
    wl = make_workload("llama16k", device=DEV, **dict(MINI, T=512))
    _run_decode_case(ctx, wl, steps=2, top_k=10000, label="all chunks")


def test_decode_full_reconstruction_many_blocks(ctx):
    # Every candidate chunk selected at T = 20480 (2552 chunks, 319 attend blocks per head,
    # beyond the 257 blocks of the value-space merge): full reconstruction through the
    # matrix-core path.
    wl = make_workload("llama16k", device=DEV, **dict(MINI, T=20480))
    _run_decode_case(ctx, wl, steps=1, top_k=1 << 20, label="full reconstruction, 319 blocks")


def test_decode_exact_rows_only(ctx):
    # top_k = 0: no split is attended and the output comes from the exact rows alone.
    wl = make_workload("llama16k", device=DEV, **MINI)
    _run_decode_case(ctx, wl, steps=2, top_k=0, label="exact rows only")


def test_decode_full_rank_all_chunks_is_dense(ctx):
    # Full rank and every chunk selected: SR decode equals dense attention over [0, p].
    wl = make_workload("tiny", device=DEV)
    c = wl.cfg
    Ks, Vs = wl.group_kv(0, "K", 0), wl.group_kv(0, "V", 0)
    n = c.n
    cache = oracle_cache(wl, n, 1)
    rows = tail_rows(c.T, c.n_sink, c.n_local)
    dec = xk.LayerDecoder(ctx, batch=1, n_q_heads=1, n_kv_heads=1, head_dim=c.head_dim, T=c.T, chunk=c.chunk,
                          top_k=10000, n_sink=c.n_sink, n_local=c.n_local, r_k=n, r_v=n, dtype=c.torch_dtype,
                          device=DEV)
    q = wl.query(0, 1, 0)
    out = dec.decode(dec.args(n_gen=0, q=q, A_k=cache["A_k"], Bt_k=cache["Bt_k"], A_v=cache["A_v"],
                              Bt_v=cache["Bt_v"], landmarks=cache["lm"], k_tail=Ks[1][rows].contiguous(),
                              v_tail=Vs[1][rows].contiguous()))
    torch.cuda.synchronize()
    ref = oracle.dense_decode(f64(q), f64(Ks[1]), f64(Vs[1]), p=c.T, n_kv_heads=1)
    rel, _ = attention_errors(f64(out)[0], ref)
    log(f"  full rank vs dense: rel {rel:.2e}")
    assert rel <= ATT_REL_F32


def test_decode_batched_sequences(ctx):
    # batch 2 with batch strides: each sequence matches its own single-sequence decode.
    wl = make_workload("llama16k", device=DEV, **dict(MINI, T=512))
    c = wl.cfg
    d_kv, T = c.d_kv, c.T
    per = []
    for b in range(2):
        Ks, Vs = wl.group_kv(b, "K", 0), wl.group_kv(b, "V", 0)
        ck, cv = xk.compress(ctx, [Ks, Vs], r=c.rank, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim,
                             landmarks=[True, False])
        rows = tail_rows(T, c.n_sink, c.n_local)
        per.append(dict(A_k=ck["A"], Bt_k=ck["Bt"][:d_kv], A_v=cv["A"], Bt_v=cv["Bt"][:d_kv],
                        lm=ck["landmarks"][0], kt=Ks[0][rows], vt=Vs[0][rows], q=wl.query(b, 0, 0)))
    st = {k: torch.stack([p[k] for p in per]).contiguous() for k in per[0]}
    mk = lambda batch: xk.LayerDecoder(ctx, batch=batch, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads,
                                       head_dim=c.head_dim, T=T, chunk=c.chunk, top_k=c.top_k, n_sink=c.n_sink,
                                       n_local=c.n_local, r_k=c.rank, r_v=c.rank, dtype=c.torch_dtype, device=DEV)
    dec2 = mk(2)
    out2 = dec2.decode(dec2.args(
        n_gen=0, q=st["q"], A_k=st["A_k"][0], Bt_k=st["Bt_k"][0], A_v=st["A_v"][0], Bt_v=st["Bt_v"][0],
        landmarks=st["lm"], k_tail=st["kt"], v_tail=st["vt"], bstride_A_k=st["A_k"].stride(0),
        bstride_Bt_k=st["Bt_k"].stride(0), bstride_A_v=st["A_v"].stride(0), bstride_Bt_v=st["Bt_v"].stride(0),
        bstride_lm=st["lm"].stride(0), bstride_tail=st["kt"].stride(0))).clone()
    for b in range(2):
        dec1 = mk(1)
        p = per[b]
        o1 = dec1.decode(dec1.args(n_gen=0, q=p["q"], A_k=p["A_k"], Bt_k=p["Bt_k"], A_v=p["A_v"], Bt_v=p["Bt_v"],
                                   landmarks=p["lm"], k_tail=p["kt"].contiguous(), v_tail=p["vt"].contiguous()))
        torch.cuda.synchronize()
        assert torch.equal(o1[0], out2[b])


def test_decode_deterministic(ctx):
    wl = make_workload("llama16k", device=DEV, **dict(MINI, T=512))
    c = wl.cfg
    Ks, Vs = wl.group_kv(0, "K", 0), wl.group_kv(0, "V", 0)
    ck, cv = xk.compress(ctx, [Ks, Vs], r=c.rank, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim,
                         landmarks=[True, False])
    ck2, _ = xk.compress(ctx, [Ks, Vs], r=c.rank, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim,
                         landmarks=[True, False])
    torch.cuda.synchronize()
    assert torch.equal(ck["A"], ck2["A"]) and torch.equal(ck["landmarks"], ck2["landmarks"])
    rows = tail_rows(c.T, c.n_sink, c.n_local)
    dec = xk.LayerDecoder(ctx, batch=1, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim,
                          T=c.T, chunk=c.chunk, top_k=c.top_k, n_sink=c.n_sink, n_local=c.n_local, r_k=c.rank,
                          r_v=c.rank, dtype=c.torch_dtype, device=DEV)
    args = dec.args(n_gen=0, q=wl.query(0, 0, 0), A_k=ck["A"], Bt_k=ck["Bt"][: c.d_kv], A_v=cv["A"],
                    Bt_v=cv["Bt"][: c.d_kv], landmarks=ck["landmarks"][0], k_tail=Ks[0][rows].contiguous(),
                    v_tail=Vs[0][rows].contiguous())
    o1 = dec.decode(args).clone()
    o2 = dec.decode(args).clone()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_decode_unequal_key_value_ranks(ctx):
    # Keys and values compressed at different ranks (r_k = 256, r_v = 128, as an adaptive
    # allocation may choose) take the generic attend kernel; the same oracle-built cache on
    # both sides, with leading dimensions wider than the ranks (a rank-256 factorisation
    # truncated to its first 128 columns).
    wl = make_workload("llama16k", device=DEV, **dict(MINI, latent_rank=384))
    c = wl.cfg
    d_kv, T, layer, steps = c.d_kv, c.T, 1, 3
    Ks, Vs = wl.group_kv(0, "K", 0), wl.group_kv(0, "V", 0)
    ok = oracle.compress_group([f64(x) for x in Ks], 256)
    ov = oracle.compress_group([f64(x) for x in Vs], 256)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(c.torch_dtype).to(DEV)
    A_k, Bt_k = to(ok["A"]), to(ok["B"][:, layer * d_kv:(layer + 1) * d_kv].T)
    A_v, Bt_v = to(ov["A"])[:, :128], to(ov["B"][:, layer * d_kv:(layer + 1) * d_kv].T)[:, :128]
    lm = to(oracle.landmarks(f64(Ks[layer]), c.n_kv_heads, c.head_dim, c.chunk, c.rope_theta))
    dec = xk.LayerDecoder(ctx, batch=1, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim, T=T,
                          chunk=c.chunk, top_k=c.top_k, n_sink=c.n_sink, n_local=c.n_local, r_k=256, r_v=128,
                          dtype=c.torch_dtype, device=DEV, max_gen=steps)
    rows = tail_rows(T, c.n_sink, c.n_local)
    k_tail = torch.zeros((len(rows) + steps, d_kv), dtype=c.torch_dtype, device=DEV)
    v_tail = torch.zeros_like(k_tail)
    k_tail[:len(rows)] = Ks[layer][rows]
    v_tail[:len(rows)] = Vs[layer][rows]
    k_ex = {t: f64(Ks[layer][t]) for t in rows}
    v_ex = {t: f64(Vs[layer][t]) for t in rows}
    for s in range(steps):
        q = wl.query(0, layer, s)
        kn, vn = wl.new_token(0, "K", layer, s), wl.new_token(0, "V", layer, s)
        k_ex[T + s], v_ex[T + s] = f64(kn), f64(vn)
        out = dec.decode(dec.args(n_gen=s + 1, q=q, A_k=A_k, Bt_k=Bt_k, A_v=A_v, Bt_v=Bt_v, landmarks=lm,
                                  k_tail=k_tail, v_tail=v_tail, k_new=kn, v_new=vn))
        torch.cuda.synchronize()
        kw = dict(T=T, n_gen=s + 1, n_kv_heads=c.n_kv_heads, chunk=c.chunk, top_k=c.top_k, n_sink=c.n_sink,
                  n_local=c.n_local, landmarks_l=f64(lm), A_k=f64(A_k), B_k_l=f64(Bt_k).T, A_v=f64(A_v),
                  B_v_l=f64(Bt_v).T, k_exact=k_ex, v_exact=v_ex)
        ref = oracle.sr_decode_layer(f64(q), **kw)
        sel = dec.sel.cpu().numpy()[0]
        if sum(check_selection(sel[h], ref["scores"][h], c.top_k) for h in range(c.n_kv_heads)):
            ref = oracle.sr_decode_layer(f64(q), selection=sel, **kw)
        rel, mx = attention_errors(f64(out)[0], ref["out"])
        log(f"  r_k 256, r_v 128, step {s}: rel L2 {rel:.2e}, max abs {mx:.2e}")
        assert rel <= 1e-3 and mx <= ATT_ABS_BF16
