"""Parity at the workloads' full sizes (sampled outputs and properties).

Decode runs the 64k Llama-shaped, 122k Qwen-shaped and batch-8 (G = 1, 2, 4, 8 at
r = 128 G) workloads at their real shapes, in the launch configuration the
benchmark times (``xkv_sr_decode_layers`` over consecutive layers with appends and
attend timing events).  The compressed cache is a stand-in that involves no
factorisation: the generator's own rank-r factors (``Workload.factor_cache``) with
landmarks of the original keys computed by the oracle.  Sampled layers and steps are
compared with the oracle on exactly those inputs, to the same bars as the small cases.

Compression runs one group (K and V) of the 64k workload through the batched entry
point the benchmark uses and checks what holds at any size: an orthonormal float64
basis, the a-posteriori projector error estimate within tolerance, A = X V_r on sampled
rows, sum of the returned eigenvalues = ||A||_F^2, and every landmark of one layer
against the oracle's landmarks of the same keys.
"""
import numpy as np
import pytest
import torch

import kv_cache_cross_amd as xk
from kv_cache_cross_amd import _lib as L
import oracle
from parity_util import ATT_ABS_BF16, attention_errors, check_selection, f64, tail_rows
from synth import make_workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def ctx():
    c = xk.Context(0)
    yield c
    c.close()


def _to_dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(DEV)


def _layer_inputs(wl, b, l, n_steps):
    """One layer's decode inputs for sequence b: stand-in cache, landmarks of the
    original keys (oracle), exact tail rows with room for the appended tokens."""
    c = wl.cfg
    A_k, Bt_k = wl.factor_cache(b, "K", l, c.rank)
    A_v, Bt_v = wl.factor_cache(b, "V", l, c.rank)
    K, V = wl.layer_kv(b, "K", l), wl.layer_kv(b, "V", l)
    lm = _to_dev(oracle.landmarks(f64(K), c.n_kv_heads, c.head_dim, c.chunk, c.rope_theta), c.torch_dtype)
    rows = tail_rows(c.T, c.n_sink, c.n_local)
    k_tail = torch.zeros((len(rows) + n_steps, c.d_kv), dtype=c.torch_dtype, device=DEV)
    v_tail = torch.zeros_like(k_tail)
    k_tail[:len(rows)] = K[rows]
    v_tail[:len(rows)] = V[rows]
    k_exact = {t: f64(K[t]) for t in rows}
    v_exact = {t: f64(V[t]) for t in rows}
    del K, V
    return dict(A_k=A_k, Bt_k=Bt_k, A_v=A_v, Bt_v=Bt_v, lm=lm, k_tail=k_tail, v_tail=v_tail,
                k_exact=k_exact, v_exact=v_exact, n_rows=len(rows))


def _check_layer(c, q, inp, out, sel, n_gen, label):
    kw = dict(T=c.T, n_gen=n_gen, n_kv_heads=c.n_kv_heads, chunk=c.chunk, top_k=c.top_k, n_sink=c.n_sink,
              n_local=c.n_local, landmarks_l=f64(inp["lm"]), A_k=f64(inp["A_k"]), B_k_l=f64(inp["Bt_k"]).T,
              A_v=f64(inp["A_v"]), B_v_l=f64(inp["Bt_v"]).T, k_exact=inp["k_exact"], v_exact=inp["v_exact"],
              theta=c.rope_theta)
    ref = oracle.sr_decode_layer(f64(q), **kw)
    swaps = sum(check_selection(sel[h], ref["scores"][h], c.top_k) for h in range(c.n_kv_heads))
    if swaps:
        ref = oracle.sr_decode_layer(f64(q), selection=sel, **kw)
    rel, mx = attention_errors(f64(out), ref["out"])
    log(f"  {label}: rel L2 {rel:.2e}, max abs {mx:.2e}, near-tie swaps {swaps}")
    assert rel <= 1e-3 and mx <= ATT_ABS_BF16, (label, rel, mx)


def _decode_layers_fullsize(ctx, name, layers, steps, check_layers):
    """Decode `steps` steps through `layers` (sequence 0) with xkv_sr_decode_layers and
    compare the layers in `check_layers` with the oracle after every step."""
    wl = make_workload(name, device=DEV)
    c = wl.cfg
    log(f"{name}: T={c.T} H_kv={c.n_kv_heads} H_q={c.n_q_heads} r={c.rank} layers {layers}, {steps} steps")
    inp = {l: _layer_inputs(wl, 0, l, steps) for l in layers}
    dec = xk.LayerDecoder(ctx, batch=1, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim,
                          T=c.T, chunk=c.chunk, top_k=c.top_k, n_sink=c.n_sink, n_local=c.n_local, r_k=c.rank,
                          r_v=c.rank, dtype=c.torch_dtype, device=DEV, rope_theta=c.rope_theta, max_gen=steps)
    out = torch.empty((len(layers), c.n_q_heads, c.head_dim), dtype=torch.float32, device=DEV)
    sel = torch.full((len(layers), c.n_kv_heads, c.top_k), -1, dtype=torch.int32, device=DEV)
    events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(layers))]
    for e in events:
        e.record()
    for s in range(steps):
        arr, qs = [], {}
        for i, l in enumerate(layers):
            x = inp[l]
            qs[l] = wl.query(0, l, s)
            kn, vn = wl.new_token(0, "K", l, s), wl.new_token(0, "V", l, s)
            x["k_exact"][c.T + s], x["v_exact"][c.T + s] = f64(kn), f64(vn)
            a = dec.args(n_gen=s + 1, q=qs[l], A_k=x["A_k"], Bt_k=x["Bt_k"], A_v=x["A_v"], Bt_v=x["Bt_v"],
                         landmarks=x["lm"], k_tail=x["k_tail"], v_tail=x["v_tail"], k_new=kn, v_new=vn)
            a.out = out[i].data_ptr()
            a.sel = sel[i].data_ptr()
            arr.append(a)
            x["_keep"] = (kn, vn)
        L.sr_decode_layers(ctx, L.sr_args_array(arr), dec.ws, attend_events=events)
        torch.cuda.synchronize()
        att = [events[2 * i].elapsed_time(events[2 * i + 1]) * 1e3 for i in range(len(layers))]
        log(f"  step {s}: attend kernel {np.mean(att):.1f} us per layer")
        for i, l in enumerate(layers):
            if l in check_layers:
                _check_layer(c, qs[l], inp[l], out[i], sel[i].cpu().numpy(), s + 1, f"{name} layer {l} step {s}")
    for l in layers:   # the tails now hold the appended tokens exactly
        for s in range(steps):
            assert torch.equal(inp[l]["k_tail"][inp[l]["n_rows"] + s], wl.new_token(0, "K", l, s))
    del inp
    torch.cuda.empty_cache()


def test_fullsize_llama64k_decode(ctx):
    # Layers 3 and 4 straddle a group boundary; both are checked at both steps.
    _decode_layers_fullsize(ctx, "llama64k", layers=[2, 3, 4], steps=2, check_layers=[3, 4])


def test_fullsize_qwen122k_decode(ctx):
    # GQA 7:1, r = 256, 15352 candidate chunks per head.
    _decode_layers_fullsize(ctx, "qwen122k", layers=[0, 27], steps=2, check_layers=[0, 27])


@pytest.mark.parametrize("name", ["batch8_g8", "batch8_g4", "batch8_g2", "batch8_g1"])
def test_fullsize_batch8_decode(ctx, name):
    # Batch 8 with per-sequence strides; G = 8 takes r = 1024 (two 512-column rank
    # chunks in the attend kernel), G = 1 takes r = 128.  Sequences 0 and 7 are checked.
    wl = make_workload(name, device=DEV)
    c = wl.cfg
    l, B = 1, c.batch
    log(f"{name}: batch {B}, T={c.T}, r={c.rank}, layer {l}")
    per = [_layer_inputs(wl, b, l, 1) for b in range(B)]
    st = {k: torch.stack([p[k] for p in per]).contiguous() for k in ("A_k", "Bt_k", "A_v", "Bt_v", "lm",
                                                                        "k_tail", "v_tail")}
    q = torch.stack([wl.query(b, l, 0) for b in range(B)]).contiguous()
    kn = torch.stack([wl.new_token(b, "K", l, 0) for b in range(B)]).contiguous()
    vn = torch.stack([wl.new_token(b, "V", l, 0) for b in range(B)]).contiguous()
    dec = xk.LayerDecoder(ctx, batch=B, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim,
                          T=c.T, chunk=c.chunk, top_k=c.top_k, n_sink=c.n_sink, n_local=c.n_local, r_k=c.rank,
                          r_v=c.rank, dtype=c.torch_dtype, device=DEV, max_gen=1)
    args = dec.args(n_gen=1, q=q, A_k=st["A_k"][0], Bt_k=st["Bt_k"][0], A_v=st["A_v"][0], Bt_v=st["Bt_v"][0],
                    landmarks=st["lm"], k_tail=st["k_tail"][0], v_tail=st["v_tail"][0], k_new=kn, v_new=vn,
                    bstride_A_k=st["A_k"].stride(0), bstride_Bt_k=st["Bt_k"].stride(0),
                    bstride_A_v=st["A_v"].stride(0), bstride_Bt_v=st["Bt_v"].stride(0),
                    bstride_lm=st["lm"].stride(0), bstride_tail=st["k_tail"].stride(0), bstride_new=kn.stride(0))
    out = dec.decode(args)
    torch.cuda.synchronize()
    sel = dec.sel.cpu().numpy()
    for b in (0, B - 1):
        x = per[b]
        x["A_k"], x["Bt_k"], x["A_v"], x["Bt_v"] = st["A_k"][b], st["Bt_k"][b], st["A_v"][b], st["Bt_v"][b]
        x["k_exact"][c.T], x["v_exact"][c.T] = f64(kn[b]), f64(vn[b])
        _check_layer(c, q[b], x, out[b], sel[b], 1, f"{name} sequence {b}")
        assert torch.equal(st["k_tail"][b, x["n_rows"]], kn[b])
    del per, st
    torch.cuda.empty_cache()


def test_fullsize_llama64k_compress_group(ctx):
    wl = make_workload("llama64k", device=DEV)
    c = wl.cfg
    g = 1   # the second group: its latent basis shares 70 % of its columns with group 0's
    Ks, Vs = wl.group_kv(0, "K", g), wl.group_kv(0, "V", g)
    outs = xk.compress(ctx, [Ks, Vs], r=c.rank, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim, chunk=c.chunk,
                       landmarks=[True, False], keep_vr64=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    t_s = np.sort(rng.choice(c.T, size=64, replace=False))
    for side, layers, o in (("K", Ks, outs[0]), ("V", Vs, outs[1])):
        st = o["stats"]
        Vr = f64(o["Vr64"])
        orth = np.abs(Vr.T @ Vr - np.eye(c.rank)).max()
        X_s = np.concatenate([f64(x[t_s]) for x in layers], axis=1)        # sampled rows of X
        A_ref = X_s @ Vr
        A_got = f64(o["A"][t_s])
        a_err = np.abs(A_got - A_ref).max() / np.abs(A_ref).max()
        lam = np.asarray(o["eigvals"], dtype=np.float64)[:c.rank]
        A_all = o["A"].double()
        energy = float((A_all * A_all).sum().item())
        e_err = abs(energy - lam.sum()) / lam.sum()
        log(f"  {side}: err_est {st['err_est']:.2e} rounds {st['rounds']} orth {orth:.1e} "
            f"A rows rel {a_err:.2e} energy rel {e_err:.2e}")
        assert st["err_est"] <= 1e-4
        assert orth <= 1e-10
        assert a_err <= 2 ** -7                  # bf16 storage of A (RNE) on top of float32 accumulation
        assert e_err <= 1e-2
        assert np.all(np.diff(lam) <= 0) and lam[-1] > 0
    # Landmarks of layer 1 of the group: every chunk, against the oracle on the same keys.
    ref = oracle.landmarks(f64(Ks[1]), c.n_kv_heads, c.head_dim, c.chunk, c.rope_theta)
    got = f64(outs[0]["landmarks"][1])
    lm_err = np.abs(got - ref).max() / np.abs(ref).max()
    log(f"  landmarks layer 1: max rel {lm_err:.2e}")
    assert lm_err <= 2 ** -7
    del outs, Ks, Vs
    torch.cuda.empty_cache()
