"""Synthetic low-rank-plus-noise KV caches shaped like the xKV workloads.

The xKV pages evaluate on Llama-3.1-8B-Instruct and Qwen2.5-7B-Instruct-1M
(xKV blog, Table 1) at 60k and 122k tokens (Fig. 7).  Trained weights and
benchmark data are not available, so every input here is drawn from a seeded
generator that keeps those models' KV shapes (layers, KV heads, head dim,
GQA ratio) and the pages' context lengths, and reproduces the premise the
method relies on: the layers' caches share a dominant low-rank subspace
(xKV blog, Fig. 2).

Recipe (one sequence ``b``, one side ``K`` or ``V``):

* a latent basis ``U`` (T x R) with i.i.d. N(0,1) entries is shared by the
  layers of one *latent block*; for the 64k Llama workload a block reuses the
  first ``floor(share*R)`` columns of the previous block's basis;
* each layer draws its own mixing matrix ``W_l`` (R x d_kv), N(0,1);
* ``K_l = U diag(s) W_l + sigma * N(0,1)`` with ``s_i = i**-0.8``;
* the value side uses independent draws of the same recipe;
* a decode step appends one token per layer: a fresh latent row pushed
  through the same ``diag(s) W_l`` plus noise;
* queries are i.i.d. N(0,1) per layer, head and step.

Values are produced in float32 and then rounded to the storage dtype
(bfloat16 round-to-nearest-even for the bf16 workloads).  Both the oracle and
the GPU path consume the same rounded bytes.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class XkvConfig:
    name: str
    n_layers: int
    group: int            # G, layers per compression group
    n_kv_heads: int
    head_dim: int
    n_q_heads: int
    T: int                # prefix (prefill) length
    rank: int             # r, the same for K and V
    latent_rank: int      # R of the generator
    sigma: float          # noise level of the generator
    share: float          # fraction of latent columns carried over between latent blocks
    latent_block: int     # layers that share one latent basis
    chunk: int
    top_k: int
    n_sink: int
    n_local: int
    decode_steps: int
    append: bool          # decode steps append a new (uncompressed) token
    batch: int
    dtype: str            # "fp32" or "bf16"
    rope_theta: float = 10000.0

    @property
    def d_kv(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def n(self) -> int:
        return self.group * self.d_kv

    @property
    def n_groups(self) -> int:
        return self.n_layers // self.group

    @property
    def n_chunks(self) -> int:
        return self.T // self.chunk

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


def _llama(**kw) -> XkvConfig:
    base = dict(n_layers=32, group=4, n_kv_heads=8, head_dim=128, n_q_heads=32,
                rank=512, latent_rank=768, sigma=0.02, share=0.0, latent_block=4,
                chunk=8, top_k=256, n_sink=4, n_local=64, append=True, batch=1,
                dtype="bf16")
    base.update(kw)
    return XkvConfig(**base)


CONFIGS = {
    # Tiny fp32 single group: X is 256 x 128, r = 16, one query head.
    "tiny": XkvConfig(name="tiny", n_layers=2, group=2, n_kv_heads=1, head_dim=64,
                      n_q_heads=1, T=256, rank=16, latent_rank=32, sigma=0.01, share=0.0,
                      latent_block=2, chunk=8, top_k=8, n_sink=4, n_local=16,
                      decode_steps=1, append=False, batch=1, dtype="fp32"),
    # Llama-3.1-8B-shaped single group at 16k tokens.
    "llama16k": _llama(name="llama16k", n_layers=4, T=16384, decode_steps=64),
    # Llama-3.1-8B-shaped full KV at 64k tokens, 8 groups of 4, 70 % latent sharing.
    "llama64k": _llama(name="llama64k", T=65536, share=0.7, decode_steps=128),
    # Qwen2.5-7B-shaped long context at 122880 tokens.
    "qwen122k": XkvConfig(name="qwen122k", n_layers=28, group=4, n_kv_heads=4, head_dim=128,
                          n_q_heads=28, T=122880, rank=256, latent_rank=384, sigma=0.02,
                          share=0.0, latent_block=4, chunk=8, top_k=384, n_sink=4,
                          n_local=64, decode_steps=128, append=True, batch=1, dtype="bf16"),
}
# Batched decode with a group-size sweep: one latent basis per 8 layers, so the
# data is the same for every G and only the factorisation changes.
for _g in (1, 2, 4, 8):
    CONFIGS[f"batch8_g{_g}"] = _llama(name=f"batch8_g{_g}", group=_g, rank=128 * _g,
                                      T=32768, batch=8, latent_block=8, decode_steps=64)


def config_by_name(name: str, **overrides) -> XkvConfig:
    cfg = CONFIGS[name]
    return replace(cfg, **overrides) if overrides else cfg


def _subseed(seed: int, *tag) -> int:
    h = hashlib.sha256(repr((int(seed),) + tuple(tag)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


class Workload:
    """Lazily generated inputs of one configuration on one device."""

    def __init__(self, cfg: XkvConfig, seed: int = 0, device="cpu"):
        self.cfg = cfg
        self.seed = seed
        self.device = torch.device(device)
        self._latent = {}
        self._s = torch.arange(1, cfg.latent_rank + 1, dtype=torch.float64).pow(-0.8).float().to(self.device)

    # -- random streams -------------------------------------------------
    def _randn(self, shape, *tag) -> torch.Tensor:
        g = torch.Generator(device=self.device)
        g.manual_seed(_subseed(self.seed, *tag))
        return torch.randn(shape, generator=g, device=self.device, dtype=torch.float32)

    def _block_of(self, layer: int) -> int:
        return layer // self.cfg.latent_block

    def _latent_cols(self, shape_rows, b, side, block, tag):
        """Latent rows for one block, carrying over shared columns from the previous block."""
        cfg = self.cfg
        m = int(cfg.share * cfg.latent_rank)
        if block == 0 or m == 0:
            return self._randn((shape_rows, cfg.latent_rank), tag, b, side, block)
        prev = self._latent_cols(shape_rows, b, side, block - 1, tag)
        fresh = self._randn((shape_rows, cfg.latent_rank - m), tag, b, side, block)
        return torch.cat([prev[:, :m], fresh], dim=1)

    def latent(self, b: int, side: str, block: int) -> torch.Tensor:
        key = (b, side, block)
        if key not in self._latent:
            self._latent[key] = self._latent_cols(self.cfg.T, b, side, block, "U")
        return self._latent[key]

    def mixing(self, b: int, side: str, layer: int) -> torch.Tensor:
        cfg = self.cfg
        W = self._randn((cfg.latent_rank, cfg.d_kv), "W", b, side, layer)
        return self._s[:, None] * W

    # -- public draws ---------------------------------------------------
    def layer_kv(self, b: int, side: str, layer: int) -> torch.Tensor:
        """Pre-RoPE K (side='K') or V (side='V') of one layer: T x d_kv, storage dtype."""
        cfg = self.cfg
        U = self.latent(b, side, self._block_of(layer))
        X = U @ self.mixing(b, side, layer)
        X += cfg.sigma * self._randn((cfg.T, cfg.d_kv), "N", b, side, layer)
        return X.to(cfg.torch_dtype)

    def group_kv(self, b: int, side: str, group: int):
        g = self.cfg.group
        return [self.layer_kv(b, side, group * g + i) for i in range(g)]

    def new_token(self, b: int, side: str, layer: int, step: int) -> torch.Tensor:
        """The token appended at decode step ``step`` (position T + step): d_kv, storage dtype."""
        cfg = self.cfg
        u = self._latent_cols(1, b, side, self._block_of(layer), ("u", step))
        x = u @ self.mixing(b, side, layer)
        x += cfg.sigma * self._randn((1, cfg.d_kv), "n", b, side, layer, step)
        return x[0].to(cfg.torch_dtype)

    def factor_cache(self, b: int, side: str, layer: int, r: int):
        """The generator's own rank-r factors of one layer's noise-free K or V: the first r
        latent columns U[:, :r] (T x r) and the matching rows of diag(s) W_l, transposed
        (d_kv x r), both in the storage dtype.  A stand-in compressed cache for decode tests
        that involves no factorisation.  Past the latent rank R the extra r - R columns are
        fresh N(0,1) columns with sigma-scaled N(0,1) mixing rows (the noise floor)."""
        cfg = self.cfg
        R = cfg.latent_rank
        U = self.latent(b, side, self._block_of(layer))
        A = U[:, :min(r, R)]
        Bt = self.mixing(b, side, layer)[:min(r, R)].t()
        if r > R:
            A = torch.cat([A, self._randn((cfg.T, r - R), "Ux", b, side, self._block_of(layer))], dim=1)
            Bt = torch.cat([Bt, cfg.sigma * self._randn((cfg.d_kv, r - R), "Wx", b, side, layer)], dim=1)
        return A.contiguous().to(cfg.torch_dtype), Bt.contiguous().to(cfg.torch_dtype)

    def query(self, b: int, layer: int, step: int) -> torch.Tensor:
        """Pre-RoPE query of one layer at one step: H_q x d, storage dtype."""
        cfg = self.cfg
        return self._randn((cfg.n_q_heads, cfg.head_dim), "q", b, layer, step).to(cfg.torch_dtype)


def gaussian(shape, seed: int, *, scale: float = 1.0, dtype=torch.float32, device="cpu") -> torch.Tensor:
    """Seeded N(0, scale^2) matrix in the storage dtype (unit-level test inputs)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(_subseed(seed, "gaussian", tuple(shape)))
    return (scale * torch.randn(tuple(shape), generator=g)).to(dtype).to(device)


def make_workload(name: str, seed: int = 0, device="cpu", **overrides) -> Workload:
    return Workload(config_by_name(name, **overrides), seed=seed, device=device)
