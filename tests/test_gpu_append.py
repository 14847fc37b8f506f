"""Tokens appended after a compressed prefix (multi-turn growth), GPU vs oracle.

The prefix is factored by the oracle (float64 truncated SVD, rounded to bf16); both
sides project the same appended rows onto that stored basis and form the landmarks of
the new chunks at their positions.  Bars: A rows and landmarks within bf16 rounding of
the float64 values (2^-8 relative, plus 1e-4 of the largest value for the float32
sums); a decode step over the grown prefix T' = T + m against the oracle's decode over
its own grown cache, to the attention bar (rel L2 <= 1e-2, max abs <= 2e-2).
"""
import numpy as np
import pytest
import torch

import kv_cache_cross_amd as xk
import oracle
from parity_util import ATT_ABS_BF16, ATT_REL_BF16, attention_errors, check_selection, f64, tail_rows
from synth import make_workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
T0, M = 2048, 256
MINI = dict(T=T0 + M, n_layers=4, n_kv_heads=2, n_q_heads=8, rank=128, latent_rank=192, top_k=32)


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def ctx():
    c = xk.Context(0)
    yield c
    c.close()


def _close(got, ref):
    return np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4 * np.abs(ref).max())


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(DEV)


def _grow(ctx, wl, side, r):
    """Oracle-factored prefix of `side` (rows < T0) and the GPU / oracle appends of rows
    [T0, T0 + M) onto its stored basis."""
    c = wl.cfg
    full = wl.group_kv(0, side, 0)
    ref = oracle.compress_group([f64(x[:T0]) for x in full], r)
    Bt = _bf16(ref["B"].T)                                   # n x r, the basis as stored
    A_pre = _bf16(ref["A"])
    new = [x[T0:].contiguous() for x in full]
    A = torch.empty((T0 + M, r), dtype=torch.bfloat16, device=DEV)
    A[:T0] = A_pre
    lm_new = torch.empty((c.group, c.n_kv_heads, M // c.chunk, c.head_dim), dtype=torch.bfloat16, device=DEV)
    args = xk.append_args(layers=new, Bt=Bt, A_new=A[T0:], pos0=T0, r=r, n_kv_heads=c.n_kv_heads,
                          head_dim=c.head_dim, chunk=c.chunk, landmarks_new=lm_new if side == "K" else None)
    ws = torch.empty(xk.append_ws_size(args), dtype=torch.uint8, device=DEV)
    xk.compress_append(ctx, args, ws)
    torch.cuda.synchronize()
    o = oracle.append_tokens([f64(x) for x in new], f64(Bt), T0, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim,
                             chunk=c.chunk, with_landmarks=(side == "K"))
    return dict(full=full, Bt=Bt, A=A, A_pre=A_pre, lm_new=lm_new, ref_new=o)


@pytest.mark.parametrize("side", ["K", "V"])
def test_append_rows_and_landmarks(ctx, side):
    wl = make_workload("llama16k", device=DEV, **MINI)
    g = _grow(ctx, wl, side, wl.cfg.rank)
    assert _close(f64(g["A"][T0:]), g["ref_new"]["A"])
    if side == "K":
        for l in range(wl.cfg.group):
            assert _close(f64(g["lm_new"][l]), g["ref_new"]["landmarks"][l])


def test_decode_over_grown_prefix(ctx):
    wl = make_workload("llama16k", device=DEV, **MINI)
    c = wl.cfg
    layer, r, Tn = 1, c.rank, T0 + M
    gk, gv = _grow(ctx, wl, "K", r), _grow(ctx, wl, "V", r)
    d_kv = c.d_kv
    sl = slice(layer * d_kv, (layer + 1) * d_kv)
    # Prefix landmarks (oracle) followed by the new chunks': GPU-built on the GPU side,
    # oracle-built on the oracle side; the A rows likewise.
    K = gk["full"][layer]
    lm_pre = oracle.landmarks(f64(K[:T0]), c.n_kv_heads, c.head_dim, c.chunk)
    lm_gpu = torch.cat([_bf16(lm_pre), gk["lm_new"][layer]], dim=1).contiguous()
    lm_ref = np.concatenate([f64(_bf16(lm_pre)), f64(_bf16(gk["ref_new"]["landmarks"][layer]))], axis=1)
    A_k_ref = np.concatenate([f64(gk["A_pre"]), f64(_bf16(gk["ref_new"]["A"]))])
    A_v_ref = np.concatenate([f64(gv["A_pre"]), f64(_bf16(gv["ref_new"]["A"]))])
    Bt_k, Bt_v = gk["Bt"][sl].contiguous(), gv["Bt"][sl].contiguous()
    rows = tail_rows(Tn, c.n_sink, c.n_local)
    V = gv["full"][layer]
    k_tail = torch.zeros((len(rows) + 1, d_kv), dtype=torch.bfloat16, device=DEV)
    v_tail = torch.zeros_like(k_tail)
    k_tail[:len(rows)] = K[rows]
    v_tail[:len(rows)] = V[rows]
    dec = xk.LayerDecoder(ctx, batch=1, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim, T=Tn,
                          chunk=c.chunk, top_k=c.top_k, n_sink=c.n_sink, n_local=c.n_local, r_k=r, r_v=r,
                          dtype=c.torch_dtype, device=DEV, max_gen=1)
    q = wl.query(0, layer, 0)
    kn, vn = wl.new_token(0, "K", layer, 0), wl.new_token(0, "V", layer, 0)
    out = dec.decode(dec.args(n_gen=1, q=q, A_k=gk["A"], Bt_k=Bt_k, A_v=gv["A"], Bt_v=Bt_v, landmarks=lm_gpu,
                              k_tail=k_tail, v_tail=v_tail, k_new=kn, v_new=vn))
    torch.cuda.synchronize()
    k_exact = {t: f64(K[t]) for t in rows}
    v_exact = {t: f64(V[t]) for t in rows}
    k_exact[Tn], v_exact[Tn] = f64(kn), f64(vn)
    kw = dict(T=Tn, n_gen=1, n_kv_heads=c.n_kv_heads, chunk=c.chunk, top_k=c.top_k, n_sink=c.n_sink,
              n_local=c.n_local, landmarks_l=lm_ref, A_k=A_k_ref, B_k_l=f64(Bt_k).T, k_exact=k_exact,
              v_exact=v_exact, A_v=A_v_ref, B_v_l=f64(Bt_v).T)
    ref = oracle.sr_decode_layer(f64(q), **kw)
    sel = dec.sel.cpu().numpy()[0]
    if sum(check_selection(sel[h], ref["scores"][h], c.top_k) for h in range(c.n_kv_heads)):
        ref = oracle.sr_decode_layer(f64(q), selection=sel, **kw)
    # Some selected chunks lie in the appended range (positions >= T0).
    assert (sel * c.chunk >= T0).any()
    rel, mx = attention_errors(f64(out)[0], ref["out"])
    log(f"  grown prefix T'={Tn}: rel {rel:.2e} max abs {mx:.2e}")
    assert rel <= ATT_REL_BF16 and mx <= ATT_ABS_BF16
