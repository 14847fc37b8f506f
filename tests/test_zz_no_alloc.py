"""The allocation-free decode entry point against the workspace one.

xkv_sr_decode_layers_noalloc runs the decode kernels of xkv_sr_decode_layers with
the library's own device scratch instead of a caller workspace.  Both are called
through the C ABI on the same inputs; outputs and selections must be identical
(the same kernels on the same data).  Two calls in a row, the second on a smaller
problem, show that the scratch the first call left behind does not leak into the
second.
"""
import numpy as np
import pytest
import torch

import kv_cache_cross_amd as xk
from kv_cache_cross_amd import _lib as L
from parity_util import tail_rows
from synth import make_workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _problem(ctx, batch, T, r, n_layers, top_k, n_gen, seed):
    """GPU-compressed caches of `n_layers` layers for `batch` sequences and the SrArgs of
    one decode step through them (both entry points use the same args)."""
    wl = make_workload("llama16k", device=DEV, T=T, n_layers=4, n_kv_heads=2, n_q_heads=8, rank=r,
                       latent_rank=192, top_k=top_k, seed=seed)
    c = wl.cfg
    d_kv = c.d_kv
    rows = tail_rows(T, c.n_sink, c.n_local)
    keep, per = [], []
    for b in range(batch):
        Ks, Vs = wl.group_kv(b, "K", 0), wl.group_kv(b, "V", 0)
        ck, cv = xk.compress(ctx, [Ks, Vs], r=r, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim,
                             landmarks=[True, False])
        per.append((Ks, Vs, ck, cv))
    dec = xk.LayerDecoder(ctx, batch=batch, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim,
                          T=T, chunk=c.chunk, top_k=top_k, n_sink=c.n_sink, n_local=c.n_local, r_k=r, r_v=r,
                          dtype=c.torch_dtype, device=DEV, max_gen=n_gen)
    out = torch.empty((n_layers, batch, c.n_q_heads, c.head_dim), dtype=torch.float32, device=DEV)
    sel = torch.full((n_layers, batch, c.n_kv_heads, top_k), -7, dtype=torch.int32, device=DEV)
    arr = []
    for l in range(n_layers):
        st = lambda f: torch.stack([f(p) for p in per]).contiguous()
        A_k, A_v = st(lambda p: p[2]["A"]), st(lambda p: p[3]["A"])
        Bt_k = st(lambda p: p[2]["Bt"][l * d_kv:(l + 1) * d_kv])
        Bt_v = st(lambda p: p[3]["Bt"][l * d_kv:(l + 1) * d_kv])
        lm = st(lambda p: p[2]["landmarks"][l])
        kt = torch.zeros((batch, len(rows) + n_gen, d_kv), dtype=c.torch_dtype, device=DEV)
        vt = torch.zeros_like(kt)
        for b, p in enumerate(per):
            kt[b, :len(rows)] = p[0][l][rows]
            vt[b, :len(rows)] = p[1][l][rows]
            for s in range(n_gen - 1):
                kt[b, len(rows) + s] = wl.new_token(b, "K", l, s)
                vt[b, len(rows) + s] = wl.new_token(b, "V", l, s)
        q = torch.stack([wl.query(b, l, n_gen) for b in range(batch)]).contiguous()
        kn = torch.stack([wl.new_token(b, "K", l, n_gen - 1) for b in range(batch)]).contiguous()
        vn = torch.stack([wl.new_token(b, "V", l, n_gen - 1) for b in range(batch)]).contiguous()
        a = dec.args(n_gen=n_gen, q=q, A_k=A_k[0], Bt_k=Bt_k[0], A_v=A_v[0], Bt_v=Bt_v[0], landmarks=lm,
                     k_tail=kt[0], v_tail=vt[0], k_new=kn, v_new=vn, bstride_A_k=A_k.stride(0),
                     bstride_Bt_k=Bt_k.stride(0), bstride_A_v=A_v.stride(0), bstride_Bt_v=Bt_v.stride(0),
                     bstride_lm=lm.stride(0), bstride_tail=kt.stride(0), bstride_new=kn.stride(0))
        a.out = out[l].data_ptr()
        a.sel = sel[l].data_ptr()
        arr.append(a)
        keep += [A_k, A_v, Bt_k, Bt_v, lm, kt, vt, q, kn, vn]
    return dict(arr=L.sr_args_array(arr), out=out, sel=sel, dec=dec, keep=keep, per=per)


def _both(ctx, pr):
    """Run the step with the library scratch, then (tails restored) with a workspace."""
    tails = [t.clone() for t in pr["keep"][5::10] + pr["keep"][6::10]]
    L.sr_decode_layers_noalloc(ctx, pr["arr"])
    torch.cuda.synchronize()
    out_s, sel_s = pr["out"].clone(), pr["sel"].clone()
    for t, saved in zip(pr["keep"][5::10] + pr["keep"][6::10], tails):
        t.copy_(saved)
    pr["out"].fill_(float("nan"))
    pr["sel"].fill_(-7)
    ws = torch.full_like(pr["dec"].ws, 0xA5)
    L.sr_decode_layers(ctx, pr["arr"], ws)
    torch.cuda.synchronize()
    return out_s, sel_s, pr["out"].clone(), pr["sel"].clone()


def test_noalloc_decode_matches_workspace_entry_point():
    with xk.Context(0) as ctx:
        big = _problem(ctx, batch=2, T=2048, r=128, n_layers=4, top_k=48, n_gen=3, seed=1)
        o1, s1, o1w, s1w = _both(ctx, big)
        assert torch.equal(s1, s1w) and torch.equal(o1, o1w)
        assert bool(torch.isfinite(o1).all()) and int((s1 >= 0).sum()) > 0
        # second call: a smaller problem; the scratch still holds the first call's values
        small = _problem(ctx, batch=1, T=512, r=128, n_layers=2, top_k=16, n_gen=1, seed=2)
        o2, s2, o2w, s2w = _both(ctx, small)
        assert torch.equal(s2, s2w) and torch.equal(o2, o2w)
        assert bool(torch.isfinite(o2).all())
        print(f"noalloc: outputs identical on both calls ({o1.numel()} and {o2.numel()} values)", flush=True)


def test_noalloc_rejects_scratch_overflow():
    # Every chunk of a 64000-token prefix at rank 1024 for two sequences needs far more
    # than the scratch; the call must refuse before launching anything.
    with xk.Context(0) as ctx:
        shape = dict(batch=2, n_q_heads=32, n_kv_heads=8, head_dim=128, T=64000, chunk=8, top_k=100000, n_sink=4,
                     n_local=64, r_k=1024, r_v=1024, dtype=L.XKV_BF16, rope_theta=1e4, scale=0.088)
        a = L.sr_args(**shape, n_gen=1, q=256, A_k=256, ld_A_k=1024, Bt_k=256, ld_Bt_k=1024, A_v=256, ld_A_v=1024,
                      Bt_v=256, ld_Bt_v=1024, landmarks=256, k_tail=256, v_tail=256, ld_tail=1024, out=256, sel=256)
        assert L.sr_ws_size(a) > L.SR_SCRATCH_BYTES
        with pytest.raises(L.XkvError) as e:
            L.sr_decode_layers_noalloc(ctx, L.sr_args_array([a]))
        assert e.value.code == L.XKV_EWORKSPACE
