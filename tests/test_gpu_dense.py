"""Dense decode baseline and the RoPE row helper vs the float64 oracle.

The dense baseline attends one query position over every cached position (full
attention).  Its cache holds post-RoPE keys, as a standard cache does; the test
forms them on the GPU with ``rope_rows`` from the same pre-RoPE keys the oracle
receives, so the GPU side also carries the bf16 rounding of the rotated keys.
Bars: attention relative L2 <= 1e-2 and max abs <= 2e-2 (bf16 storage).
"""
import numpy as np
import pytest
import torch

import kv_cache_cross_amd as xk
import oracle
from parity_util import ATT_ABS_BF16, ATT_REL_BF16, attention_errors, f64
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


@pytest.mark.parametrize("dt,d,pos0", [(torch.float32, 128, 0), (torch.float32, 64, 122700),
                                       (torch.bfloat16, 128, 5), (torch.bfloat16, 128, 122800)])
def test_rope_rows(dt, d, pos0):
    log(f"rope_rows {dt} d={d} pos0={pos0}")
    rows, heads = 181, 3
    x = gaussian((rows, heads * d + 8), seed=7 + d, dtype=dt, device=DEV)[:, :heads * d]
    y = torch.zeros((rows, heads * d + 4), dtype=dt, device=DEV)
    xk.rope_rows(x, y, pos0, heads, d)
    torch.cuda.synchronize()
    ref = np.concatenate([oracle.rope(f64(x)[:, h * d:(h + 1) * d], pos0 + np.arange(rows))
                          for h in range(heads)], axis=1)
    got = f64(y)[:, :heads * d]
    # float32 output: cos/sin of the float64-reduced phase in float32; bf16 output: one
    # rounding to bf16 of a value that float32 arithmetic gets right to about 1e-6.
    bound = 2e-6 + (1e-6 if dt == torch.float32 else 2.0 ** -8) * np.abs(ref)
    assert np.all(np.abs(got - ref) <= bound)
    assert np.all(f64(y)[:, heads * d:] == 0.0)


def _dense_gpu(ctx, q, K_pre, V, n_ctx, q_pos, Hkv, pad=0):
    """q: batch x Hq x 128, K_pre, V: batch x n_ctx x d_kv (bf16 on the GPU)."""
    batch, Hq, d = q.shape
    d_kv = Hkv * d
    ld = d_kv + pad
    K = torch.zeros((batch, n_ctx, ld), dtype=torch.bfloat16, device=DEV)
    Vs = torch.zeros_like(K)
    for b in range(batch):
        xk.rope_rows(K_pre[b].contiguous(), K[b], 0, Hkv, d)
        Vs[b, :, :d_kv] = V[b]
    out = torch.full((batch, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    a = xk.dense_args(batch=batch, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, n_ctx=n_ctx, q_pos=q_pos,
                      dtype=xk.XKV_BF16, scale=1.0 / np.sqrt(d), rope_theta=10000.0, q=q, K=K, V=Vs,
                      ld_kv=ld, bstride_kv=n_ctx * ld, out=out)
    ws = torch.empty(xk.dense_ws_size(a) // 4, dtype=torch.float32, device=DEV)
    xk.dense_decode(ctx, a, ws)
    torch.cuda.synchronize()
    return f64(out)


@pytest.mark.parametrize("n_ctx,Hkv,grp,batch,pad", [(1, 1, 1, 1, 0), (255, 2, 4, 2, 0), (256, 2, 8, 1, 8),
                                                     (777, 2, 4, 2, 0), (4133, 8, 4, 1, 0),
                                                     (3000, 4, 7, 3, 16)])
def test_dense_decode(ctx, n_ctx, Hkv, grp, batch, pad):
    log(f"dense n_ctx={n_ctx} Hkv={Hkv} grp={grp} batch={batch} pad={pad}")
    d = 128
    q = gaussian((batch, Hkv * grp, d), seed=n_ctx + 1, dtype=torch.bfloat16, device=DEV)
    K = gaussian((batch, n_ctx, Hkv * d), seed=n_ctx + 2, dtype=torch.bfloat16, device=DEV)
    V = gaussian((batch, n_ctx, Hkv * d), seed=n_ctx + 3, dtype=torch.bfloat16, device=DEV)
    # Peaked scores on a few rows so the softmax is not flat.
    K[:, ::97] *= 4
    got = _dense_gpu(ctx, q, K, V, n_ctx, n_ctx - 1, Hkv, pad)
    for b in range(batch):
        ref = oracle.dense_decode(f64(q[b]), f64(K[b]), f64(V[b]), n_ctx - 1, Hkv)
        rel, mx = attention_errors(got[b], ref)
        log(f"  b={b} rel {rel:.2e} max abs {mx:.2e}")
        assert rel <= ATT_REL_BF16 and mx <= ATT_ABS_BF16


@pytest.mark.parametrize("name,batch", [("llama64k", 1), ("qwen122k", 1), ("batch8_g1", 8)])
def test_dense_decode_fullsize(ctx, name, batch):
    """Each workload's layer 0 with the first decode token appended (n_ctx = T + 1)."""
    wl = make_workload(name)
    c = wl.cfg
    log(f"dense full-size {name}: T={c.T} Hkv={c.n_kv_heads} Hq={c.n_q_heads} batch={batch}")
    n_ctx = c.T + 1
    K = torch.stack([torch.cat([wl.layer_kv(b, "K", 0), wl.new_token(b, "K", 0, 0)[None]]) for b in range(batch)])
    V = torch.stack([torch.cat([wl.layer_kv(b, "V", 0), wl.new_token(b, "V", 0, 0)[None]]) for b in range(batch)])
    q = torch.stack([wl.query(b, 0, 0) for b in range(batch)])
    got = _dense_gpu(ctx, q.to(DEV), K.to(DEV), V.to(DEV), n_ctx, c.T, c.n_kv_heads)
    for b in range(batch):
        ref = oracle.dense_decode(f64(q[b]), f64(K[b]), f64(V[b]), c.T, c.n_kv_heads)
        rel, mx = attention_errors(got[b], ref)
        log(f"  b={b} rel {rel:.2e} max abs {mx:.2e}")
        assert rel <= ATT_REL_BF16 and mx <= ATT_ABS_BF16
