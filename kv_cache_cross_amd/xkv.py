"""Thin Python layer over libxkv: allocates outputs and workspaces with torch
and passes pointers to the C ABI.  No arithmetic of the method happens here.
"""
from __future__ import annotations

import math

import torch

from . import _lib as L


def dtype_code(dt: torch.dtype) -> int:
    return L.XKV_BF16 if dt == torch.bfloat16 else L.XKV_F32


def compress(ctx: L.Context, sides, *, r: int, n_kv_heads: int, head_dim: int, chunk: int = 8,
             rope_theta: float = 10000.0, landmarks=None, oversample: int = -1, fp32_iters: int = 2,
             fp64_iters: int = 2, seed: int = 0, stream=None, ws: torch.Tensor | None = None,
             keep_vr64: bool = False, tol: float = 0.0, max_rounds: int = 0, allow_notconv: bool = False):
    """Factor every group side in ``sides`` (a list of lists of G layer tensors, T x d_kv).

    ``landmarks``: list of bools, one per side (True for key sides).  Returns a list of
    dicts with 'A' (T x r), 'Bt' (n x r, Bt = V_r), 'landmarks' (G x H_kv x T/chunk x d or
    None), 'Vr64' (float64 V_r when ``keep_vr64``) and 'eigvals' (numpy, r leading Ritz values).
    With ``allow_notconv`` an XKV_ENOTCONV return (every output written, the error estimate
    above ``tol``) is not raised; each side's stats then carry converged=False.
    """
    S = len(sides)
    G = len(sides[0])
    T, d_kv = sides[0][0].shape
    dt = sides[0][0].dtype
    dev = sides[0][0].device
    n = G * d_kv
    landmarks = landmarks or [False] * S
    desc = L.make_desc(T=T, G=G, d_kv=d_kv, r=r, dtype=dtype_code(dt), n_kv_heads=n_kv_heads,
                       head_dim=head_dim, chunk=chunk, rope_theta=rope_theta, oversample=oversample,
                       fp32_iters=fp32_iters, fp64_iters=fp64_iters, seed=seed, tol=tol, max_rounds=max_rounds)
    need = L.compress_ws_size(desc, S)
    if ws is None or ws.numel() * ws.element_size() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    outs, specs = [], []
    for s in range(S):
        o = {"A": torch.empty((T, r), dtype=dt, device=dev),
             "Bt": torch.empty((n, r), dtype=dt, device=dev),
             "landmarks": (torch.empty((G, n_kv_heads, T // chunk, head_dim), dtype=dt, device=dev)
                           if landmarks[s] else None),
             "Vr64": torch.empty((n, r), dtype=torch.float64, device=dev) if keep_vr64 else None}
        outs.append(o)
        specs.append({"layers": sides[s], **o})
    converged = True
    try:
        evals, stats = L.compress_sides(ctx, desc, specs, ws, stream)
    except L.XkvError as e:
        if not (allow_notconv and e.code == L.XKV_ENOTCONV):
            raise
        evals, stats = e.evals, e.stats
        converged = False
    for o, e, st in zip(outs, evals, stats):
        o["eigvals"] = e
        o["stats"] = dict(err_est=st[0], rel_gap=st[1], sweeps=int(st[2]), rounds=int(st[3]), energy=st[4],
                          converged=converged)
    return outs


class LayerDecoder:
    """Workspace and argument builder for SR decode of one layer (reusable across layers
    of the same shape). The workspace is sized for up to `max_gen` generated tokens."""

    def __init__(self, ctx: L.Context, *, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                 T: int, chunk: int, top_k: int, n_sink: int, n_local: int, r_k: int, r_v: int,
                 dtype: torch.dtype, device, rope_theta: float = 10000.0, scale: float | None = None,
                 max_gen: int = 64):
        self.ctx = ctx
        self.shape = dict(batch=batch, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, head_dim=head_dim, T=T,
                          chunk=chunk, top_k=top_k, n_sink=n_sink, n_local=n_local, r_k=r_k, r_v=r_v,
                          dtype=dtype_code(dtype), rope_theta=rope_theta,
                          scale=scale if scale is not None else 1.0 / math.sqrt(head_dim))
        self.device = device
        self.max_gen = max_gen
        self.out = torch.empty((batch, n_q_heads, head_dim), dtype=torch.float32, device=device)
        self.sel = torch.full((batch, n_kv_heads, max(top_k, 1)), -1, dtype=torch.int32, device=device)
        probe = L.sr_args(**self.shape, n_gen=max_gen, q=1, A_k=16, ld_A_k=r_k, Bt_k=16, ld_Bt_k=r_k,
                          A_v=16 if r_v else 0, ld_A_v=r_v, Bt_v=16 if r_v else 0, ld_Bt_v=r_v,
                          V_full=0 if r_v else 16, ld_V=n_kv_heads * head_dim, landmarks=16,
                          k_tail=16, v_tail=16, ld_tail=n_kv_heads * head_dim, out=16, sel=16)
        self.ws = torch.zeros(L.sr_ws_size(probe), dtype=torch.uint8, device=device)

    def args(self, *, n_gen: int, q, A_k, Bt_k, A_v=None, Bt_v=None, V_full=None, landmarks, k_tail, v_tail,
             k_new=None, v_new=None, bstride_A_k=0, bstride_Bt_k=0, bstride_A_v=0, bstride_Bt_v=0,
             bstride_V=0, bstride_lm=0, bstride_tail=0, bstride_new=0, ld_tail=None) -> L.SrArgs:
        """Tensors may be views (e.g. a layer's rows of Bt); their data pointers are used."""
        sh = self.shape
        if not 0 <= n_gen <= self.max_gen:
            raise ValueError(f"n_gen={n_gen} outside the workspace's range [0, {self.max_gen}]")
        d_kv = sh["n_kv_heads"] * sh["head_dim"]
        return L.sr_args(**sh, n_gen=n_gen, q=q, A_k=A_k, ld_A_k=A_k.stride(-2), bstride_A_k=bstride_A_k,
                         Bt_k=Bt_k, ld_Bt_k=Bt_k.stride(-2), bstride_Bt_k=bstride_Bt_k,
                         A_v=A_v, ld_A_v=A_v.stride(-2) if A_v is not None else 0, bstride_A_v=bstride_A_v,
                         Bt_v=Bt_v, ld_Bt_v=Bt_v.stride(-2) if Bt_v is not None else 0, bstride_Bt_v=bstride_Bt_v,
                         V_full=V_full, ld_V=V_full.stride(-2) if V_full is not None else d_kv, bstride_V=bstride_V,
                         landmarks=landmarks, bstride_lm=bstride_lm, k_tail=k_tail, v_tail=v_tail,
                         ld_tail=ld_tail if ld_tail is not None else k_tail.stride(-2), bstride_tail=bstride_tail,
                         k_new=k_new, v_new=v_new, bstride_new=bstride_new, out=self.out, sel=self.sel)

    def decode(self, args: L.SrArgs, stream=None):
        L.sr_decode(self.ctx, args, self.ws, stream)
        return self.out

    def select(self, args: L.SrArgs, stream=None):
        L.sr_select(self.ctx, args, self.ws, stream)

    def attend(self, args: L.SrArgs, stream=None):
        L.sr_attend(self.ctx, args, self.ws, stream)
        return self.out
