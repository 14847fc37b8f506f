#!/usr/bin/env python
"""Benchmark of the xKV hot path on one MI355X.

Workload (default, --config llama64k): the Llama-3.1-8B-shaped 64k-token cache --
32 layers in 8 groups of G=4, 8 KV heads x 128, 32 query heads, T=65536, rank 512
for K and V, bf16, batch 1, chunk 8, top-k 256 chunks + 4 sink + 64 local, 128
decode steps appending uncompressed tokens.  Other workloads: llama16k, qwen122k,
batch8_g1 / g2 / g4 / g8 (batch 8, T=32768, r = 128 G), tiny.  Inputs are
synthetic (synth/), generated on the GPU before timing.

One step = the whole hot path over the workload: compress every group side of every
sequence (Gram, subspace iteration, host Rayleigh-Ritz, projection, landmarks), then
the decode steps through every layer (append, landmark scores, top-k, rebuild +
attend + merge) for all sequences at once.  The JSON line reports:
  value    SR decode microseconds per decode step (all layers, all sequences), higher_is_better false
  sr_decode_GBps, compress_tokens_per_s, compress breakdown
  roofline         attend kernel vs HBM (union-of-rows algorithmic bytes / event-timed duration)
  roofline_gram    Gram kernel vs bf16 MFMA peak
  roofline_project projection kernel vs bf16 MFMA peak
  cpu_baseline     the float64 oracle on a bounded sample, on this host's cores
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0

# HBM traffic of one attend-kernel dispatch at this workload, from two rocprofv3 --pmc passes
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch, averaged over 64 dispatches), each scaled by
# what the same counter reads for a 1 GiB device-to-device copy (read 524304.4 KiB, written
# 1048576 KiB).  It stands only while the decode kernels' source is the one measured: the
# source's SHA-256 prefix is recorded and `traffic` is null when it differs.
ATTEND_TRAFFIC = {"src": "decode.hip", "src_sha256": "8c075953f7a77c2c", "fetch_kib": 17180.3, "write_kib": 2064.0,
                  "fetch_scale": 1048576.0 / 524304.4, "write_scale": 1.0}
# The same for one launch of the Gram kernel over the 16 group sides of the 64k workload
# (the mean of bench.py's two 16-side timing dispatches).  FETCH_SIZE counts what the L2
# caches request from the memory fabric, so the Infinity Cache's hits are included: it
# is the Gram's L2-miss traffic.
GRAM_TRAFFIC = {"src": "gram.hip", "src_sha256": "20860a837367a954", "fetch_kib": 51651792.8, "write_kib": 2180760.2,
                "fetch_scale": 1048576.0 / 524304.4, "write_scale": 1.0}


def traffic_bytes(t):
    import hashlib
    src = os.path.join(ROOT, "kv_cache_cross_amd", "csrc", t["src"])
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    if sha != t["src_sha256"]:
        return None
    return int((t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="llama64k")
    ap.add_argument("--decode-steps", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the dense baseline, the SR variants, the token fold and the rank diagnostics "
                         "(for counter runs that should see the main decode kernels only)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--sides-per-call", type=int, default=16,
                    help="group sides per compression call (the workspace is sized for one call)")
    ap.add_argument("--max-rounds", type=int, default=0,
                    help="Rayleigh-Ritz rounds before a side is reported unconverged (0: the library's 8)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB device to device (a plain copy "
                         "kernel of known size that scales memory counters)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build runs on one GPU only (asked for {args.gpus} GPUs, WORLD_SIZE={world}); "
              "the multi-GPU sharding of the path is described in DESIGN.md but not built.", file=sys.stderr)
        sys.exit(2)

    import kv_cache_cross_amd as xk
    from kv_cache_cross_amd import _lib as L
    from synth import make_workload

    wl = make_workload(args.config, seed=args.seed, device="cuda:0")
    c = wl.cfg
    D = args.decode_steps if args.decode_steps is not None else c.decode_steps
    if D < 1:
        raise SystemExit("bench.py: --decode-steps must be at least 1 (a step is compression + D decode steps)")
    B, Lyr, G, d_kv, T, r = c.batch, c.n_layers, c.group, c.d_kv, c.T, c.rank
    H, d, Hq, n, C_ch = c.n_kv_heads, c.head_dim, c.n_q_heads, c.n, c.n_chunks
    dt = c.torch_dtype
    esz = 2 if dt == torch.bfloat16 else 4
    dev = torch.device("cuda:0")
    # The library's rule for selecting the top-k inside the attend kernel (3 launches per layer
    # instead of 4): the matrix-core path (bf16, head dim 128, rank a multiple of 128), at most
    # 16384 candidates, and an attend grid (KV heads x 64-row splits x batch) within the
    # device's compute units.
    n_cand_h = -(-(T - c.n_local) // c.chunk)
    k_eff_h = min(c.top_k, n_cand_h)
    n_splits_h = -(-k_eff_h // (64 // c.chunk))
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    fused = (dt == torch.bfloat16 and d == 128 and r % 128 == 0 and 0 < k_eff_h and n_cand_h <= 16384
             and H * n_splits_h * B <= n_cu)
    attend_kernel = f"sr_attend_mfma_kernel<false, false, {(16 if n_cand_h <= 8192 else 32) if fused else 0}>"
    torch.cuda.set_device(dev)
    log(f"[bench] workload {c.name}: B={B} L={Lyr} G={G} H_kv={H} d={d} H_q={Hq} T={T} r={r} top_k={c.top_k} "
        f"decode steps={D}")

    # ---- inputs, resident in HBM before timing ----
    t0 = time.time()
    layers = {}
    for b in range(B):
        for s in "KV":
            for l in range(Lyr):
                layers[(b, s, l)] = wl.layer_kv(b, s, l)
        wl._latent.clear()
    q_all = torch.stack([torch.stack([torch.stack([wl.query(b, l, s) for b in range(B)]) for l in range(Lyr)])
                         for s in range(D)]).contiguous()                                  # D x L x B x Hq x d
    kn_all = vn_all = None
    if c.append:
        kn_all = torch.stack([torch.stack([torch.stack([wl.new_token(b, "K", l, s) for b in range(B)])
                                           for l in range(Lyr)]) for s in range(D)]).contiguous()
        vn_all = torch.stack([torch.stack([torch.stack([wl.new_token(b, "V", l, s) for b in range(B)])
                                           for l in range(Lyr)]) for s in range(D)]).contiguous()
    torch.cuda.synchronize()
    log(f"[bench] inputs generated in {time.time() - t0:.1f}s")

    ctx = xk.Context(0)
    n_groups = c.n_groups
    desc = L.make_desc(T=T, G=G, d_kv=d_kv, r=r, dtype=xk.dtype_code(dt), n_kv_heads=H, head_dim=d, chunk=c.chunk,
                       rope_theta=c.rope_theta, max_rounds=args.max_rounds)
    # Compressed cache: per group and side, all sequences in one tensor (the decode reads
    # them with batch strides).  One factorisation per sequence, group and side.
    A_out = {(g, s): torch.empty((B, T, r), dtype=dt, device=dev) for g in range(n_groups) for s in "KV"}
    Bt_out = {(g, s): torch.empty((B, n, r), dtype=dt, device=dev) for g in range(n_groups) for s in "KV"}
    lm_out = {g: torch.empty((B, G, H, C_ch, d), dtype=dt, device=dev) for g in range(n_groups)}
    sides = []
    for b in range(B):
        for g in range(n_groups):
            for s in "KV":
                sides.append({"layers": [layers[(b, s, g * G + i)] for i in range(G)], "A": A_out[(g, s)][b],
                              "Bt": Bt_out[(g, s)][b], "landmarks": lm_out[g][b] if s == "K" else None})
    S = len(sides)
    spc = min(S, args.sides_per_call)
    calls = [sides[i:i + spc] for i in range(0, S, spc)]
    cws = torch.empty(L.compress_ws_size(desc, spc), dtype=torch.uint8, device=dev)
    log(f"[bench] compress workspace {cws.numel() / 2**30:.2f} GiB; {S} group sides in {len(calls)} calls")

    # ---- decode buffers: exact tails, selections, outputs ----
    rows = list(range(c.n_sink)) + list(range(T - c.n_local, T))
    n_tail = len(rows) + (D if c.append else 0)
    k_tail = torch.zeros((Lyr, B, n_tail, d_kv), dtype=dt, device=dev)
    v_tail = torch.zeros_like(k_tail)
    for l in range(Lyr):
        for b in range(B):
            k_tail[l, b, :len(rows)] = layers[(b, "K", l)][rows]
            v_tail[l, b, :len(rows)] = layers[(b, "V", l)][rows]
    sel = torch.full((D, Lyr, B, H, c.top_k), -1, dtype=torch.int32, device=dev)
    out = torch.empty((Lyr, B, Hq, d), dtype=torch.float32, device=dev)

    def layer_args(dec_, s, l, out_t, sel_t, exact_values=False):
        g, li = divmod(l, G)
        AK, AV, BK, BV = A_out[(g, "K")], A_out[(g, "V")], Bt_out[(g, "K")], Bt_out[(g, "V")]
        lm = lm_out[g]
        kw = dict(n_gen=(s + 1) if c.append else 0, q=q_all[s, l], A_k=AK[0], Bt_k=BK[0, li * d_kv:(li + 1) * d_kv],
                  landmarks=lm[0, li], k_tail=k_tail[l, 0], v_tail=v_tail[l, 0],
                  k_new=kn_all[s, l] if c.append else None, v_new=vn_all[s, l] if c.append else None,
                  bstride_A_k=AK.stride(0), bstride_Bt_k=BK.stride(0), bstride_lm=lm.stride(0),
                  bstride_tail=k_tail.stride(1), bstride_new=d_kv)
        if exact_values:
            kw.update(V_full=layers[(0, "V", l)])
        else:
            kw.update(A_v=AV[0], Bt_v=BV[0, li * d_kv:(li + 1) * d_kv], bstride_A_v=AV.stride(0),
                      bstride_Bt_v=BV.stride(0))
        a = dec_.args(**kw)
        a.out = out_t.data_ptr()
        a.sel = sel_t.data_ptr()
        return a

    dec = xk.LayerDecoder(ctx, batch=B, n_q_heads=Hq, n_kv_heads=H, head_dim=d, T=T, chunk=c.chunk, top_k=c.top_k,
                          n_sink=c.n_sink, n_local=c.n_local, r_k=r, r_v=r, dtype=dt, device=dev,
                          rope_theta=c.rope_theta, max_gen=D if c.append else 0)
    step_args = [L.sr_args_array([layer_args(dec, s, l, out[l], sel[s, l]) for l in range(Lyr)]) for s in range(D)]
    # Attend timing: step s stamps the attend kernel of layer s mod L only (events on every
    # layer's dispatch would add ~5 us per layer to the step); over the D steps every layer
    # is sampled D / L times.
    t_layer = [s % Lyr for s in range(D)]
    events = []
    for s in range(D):
        evs = [None] * (2 * Lyr)
        evs[2 * t_layer[s]] = torch.cuda.Event(enable_timing=True)
        evs[2 * t_layer[s] + 1] = torch.cuda.Event(enable_timing=True)
        evs[2 * t_layer[s]].record()          # creates the underlying HIP events
        evs[2 * t_layer[s] + 1].record()
        events.append(evs)
    torch.cuda.synchronize()

    last_evals, last_stats, notconv = [], [], [0]

    def compress():
        evals, stats, nc = [], [], 0
        for part in calls:
            try:
                e, st = L.compress_sides(ctx, desc, part, cws)
            except L.XkvError as err:
                if err.code != L.XKV_ENOTCONV:
                    raise
                e, st, nc = err.evals, err.stats, nc + len(part)
            evals += e
            stats += st
        last_evals[:], last_stats[:], notconv[0] = evals, stats, nc

    def decode(timed):
        for s in range(D):
            L.sr_decode_layers(ctx, step_args[s], dec.ws, attend_events=events[s] if timed else None)

    # ---- warmup ----
    for w in range(args.warmup):
        compress()
        torch.cuda.synchronize()
        log(f"[bench] warm-up {w}: compression done")
        decode(False)
        torch.cuda.synchronize()
        log(f"[bench] warm-up {w}: decode done")
    torch.cuda.synchronize()

    # ---- timed steps ----
    t_comp, t_dec, attend_ms = [], [], []
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        a0 = time.perf_counter()
        compress()
        torch.cuda.synchronize()
        a1 = time.perf_counter()
        decode(True)
        torch.cuda.synchronize()
        a2 = time.perf_counter()
        t_comp.append(a1 - a0)
        t_dec.append(a2 - a1)
        log(f"[bench] timed step {len(t_comp) - 1}: compression {a1 - a0:.3f} s, decode {a2 - a1:.3f} s")
        attend_ms.append(np.array([events[s][2 * t_layer[s]].elapsed_time(events[s][2 * t_layer[s] + 1])
                                   for s in range(D)]))
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    stats = last_stats

    # ---- algorithmic bytes of the last step's decode (from its actual selections) ----
    n_cand = -(-(T - c.n_local) // c.chunk)
    sel_np = sel.cpu().numpy()

    def rows_of(cs):
        cs = np.asarray(cs)
        m = len(cs) * c.chunk
        m -= np.sum(np.clip(c.n_sink - cs * c.chunk, 0, c.chunk))     # sink rows are exact
        return m

    union_rows = np.zeros((D, Lyr))
    perhead_rows = np.zeros((D, Lyr))
    for s in range(D):
        for l in range(Lyr):
            for b in range(B):
                ch = sel_np[s, l, b]
                union_rows[s, l] += rows_of(np.unique(ch[ch >= 0]))
                perhead_rows[s, l] += sum(rows_of(ch[h][ch[h] >= 0]) for h in range(H))
    n_gen = np.arange(1, D + 1)[:, None] if c.append else np.zeros((D, 1))
    # Attend kernel: the gathered rows of A_k and A_v, the layer's B_k slice and the queries
    # (all sequences).
    attend_union = union_rows * r * esz * 2 + B * (d_kv * r * esz + Hq * d * esz)
    attend_perhead = perhead_rows * r * esz * 2 + B * (d_kv * r * esz + Hq * d * esz)
    # The rest of a layer's step: landmarks and queries (scoring), the appended token,
    # the exact tail rows (K and V), B_v (applied in the merge) and the output.
    tail_bytes = (c.n_sink + c.n_local + n_gen) * d_kv * esz * 2
    other_bytes = B * (H * n_cand * d * esz + Hq * d * esz + (2 * d_kv * esz * 2 if c.append else 0)
                       + tail_bytes + d_kv * r * esz + Hq * d * 4)
    decode_bytes_step = float(np.mean(np.sum(attend_union + other_bytes, axis=1)))
    att_ms = attend_ms[-1]                                     # D sampled launches, last step (matches sel)
    att_ms_all = float(np.mean(attend_ms))
    samp = (np.arange(D), np.array(t_layer, dtype=np.int64))
    achieved_att = float(np.sum(attend_union[samp]) / (np.sum(att_ms) * 1e-3) / 1e9)
    achieved_att_perhead = float(np.sum(attend_perhead[samp]) / (np.sum(att_ms) * 1e-3) / 1e9)

    dec_us = float(np.median(t_dec)) / D * 1e6
    comp_s = float(np.median(t_comp))
    sr_gbps = decode_bytes_step / (dec_us * 1e-6) / 1e9

    # ---- the same decode steps replayed from a HIP graph (one capture of all D steps; the
    # appends rewrite the same tail rows with the same values, so a replay repeats the
    # eager run exactly): the launch path's share of the step time ----
    graph = None
    if not args.no_extras:
        out_eager, sel_eager = out.clone(), sel.clone()
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gs):
            for s in range(D):
                L.sr_decode_layers(ctx, step_args[s], dec.ws)
        torch.cuda.synchronize()
        times, same = [], True
        for _ in range(max(args.steps, 2)):
            out.zero_()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / D * 1e3)
            same = same and bool(torch.equal(out, out_eager)) and bool(torch.equal(sel, sel_eager))
        graph = {"us_per_step": round(float(np.median(times)), 2), "replays_match_eager": same,
                 "launches_per_step": (3 if fused else 4) * Lyr}
        del g

    # ---- dense flash-decode baseline: the same queries over the full post-RoPE cache ----
    dense = dense_baseline(xk, ctx, c, layers, q_all, kn_all, vn_all, D, args.steps) if not args.no_extras else None
    # ---- the SR variants on the same cache (batch 1): xK-SR (values exact, on the GPU) and
    # full reconstruction (every candidate chunk selected) ----
    variants = {}
    if B == 1 and not args.no_extras:
        def run_variant(top_k, exact_values, steps):
            vdec = xk.LayerDecoder(ctx, batch=1, n_q_heads=Hq, n_kv_heads=H, head_dim=d, T=T, chunk=c.chunk,
                                   top_k=top_k, n_sink=c.n_sink, n_local=c.n_local, r_k=r,
                                   r_v=0 if exact_values else r, dtype=dt, device=dev, rope_theta=c.rope_theta,
                                   max_gen=D if c.append else 0)
            vsel = torch.full((Lyr, 1, H, top_k), -1, dtype=torch.int32, device=dev)
            vout = torch.empty((Lyr, 1, Hq, d), dtype=torch.float32, device=dev)
            sargs = [L.sr_args_array([layer_args(vdec, s_, l, vout[l], vsel[l], exact_values) for l in range(Lyr)])
                     for s_ in range(steps)]
            for s_ in range(steps):
                L.sr_decode_layers(ctx, sargs[s_], vdec.ws)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            times = []
            for _ in range(args.steps):
                e0.record()
                for s_ in range(steps):
                    L.sr_decode_layers(ctx, sargs[s_], vdec.ws)
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1) / steps * 1e3)
            return round(float(np.median(times)), 2)
        variants["xk_sr_us_per_step"] = run_variant(c.top_k, True, D)
        full_steps = min(D, 4)
        if n_cand // (64 // c.chunk) + 2 <= 1088:
            variants["full_reconstruction_us_per_step"] = run_variant(n_cand, False, full_steps)
            variants["full_reconstruction_steps"] = full_steps

    # ---- folding a turn's generated tokens into the compressed prefix: the D appended
    # rows of every layer projected onto each group side's stored basis (+ landmarks of
    # the new chunks), every side of sequence 0 ----
    append_rate = None
    if c.append and D % c.chunk == 0 and not args.no_extras:
        app_args, app_keep = [], []
        for g in range(n_groups):
            for s_ in "KV":
                src = kn_all if s_ == "K" else vn_all
                new = [src[:, g * G + li, 0].contiguous() for li in range(G)]
                A_new = torch.empty((D, r), dtype=dt, device=dev)
                lm_new = (torch.empty((G, H, D // c.chunk, d), dtype=dt, device=dev) if s_ == "K" else None)
                app_keep.append((new, A_new, lm_new))
                app_args.append(xk.append_args(layers=new, Bt=Bt_out[(g, s_)][0], A_new=A_new, pos0=T, r=r,
                                               n_kv_heads=H, head_dim=d, chunk=c.chunk, landmarks_new=lm_new))
        app_ws = torch.empty(max(xk.append_ws_size(a_) for a_ in app_args), dtype=torch.uint8, device=dev)
        for a_ in app_args:
            xk.compress_append(ctx, a_, app_ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            for a_ in app_args:
                xk.compress_append(ctx, a_, app_ws)
        e1.record()
        torch.cuda.synchronize()
        fold_us = e0.elapsed_time(e1) / 10 * 1e3
        append_rate = {"tokens": D, "sides": len(app_args), "us_per_fold": round(fold_us, 2),
                       "tokens_per_s": round(D / (fold_us * 1e-6), 1)}
        del app_args, app_keep, app_ws

    # ---- rank diagnostics (outside the timed region), sequence 0: the cumulative-eigenvalue
    # rank of every group side from its leading Ritz values and trace, and the full spectrum
    # of layer 0 (K and V, a compression at r = d_kv) for NER and the same rank per layer ----
    rank_diag = None
    if c.dtype == "bf16" and not args.no_extras:
        def frac_rank(ev, total):
            rs = xk.rank_stats(ev, total=total, frac=0.95)
            return rs["energy_rank"] / float(n) if rs["energy_rank"] > 0 else None
        grp = {s_: [frac_rank(last_evals[2 * g + i], stats[2 * g + i][4]) for g in range(n_groups)]
               for i, s_ in enumerate("KV")}
        single = xk.compress(ctx, [[layers[(0, "K", 0)]], [layers[(0, "V", 0)]]], r=d_kv, n_kv_heads=H, head_dim=d,
                             landmarks=[False, False])
        torch.cuda.synchronize()
        layer0 = {}
        for s_, o in zip("KV", single):
            rs = xk.rank_stats(o["eigvals"], total=o["stats"]["energy"], frac=0.95, complete=True)
            layer0[s_] = {"ner": round(rs["ner"], 5), "erank": round(rs["erank"], 2),
                          "rank95_frac": round(rs["energy_rank"] / float(d_kv), 4)}
        del single
        # Adaptive rank at the uniform budget (every side of sequence 0 at r): one more
        # compression at r_max = r + 128 gives each side's leading eigenvalues; ranks are
        # multiples of 128 in [r - 128, r + 128].
        adaptive = None
        if r > 128 and r + 128 <= n:
            seq0 = sides[:2 * n_groups]          # the sides are ordered by sequence, group, K / V
            wide = xk.compress(ctx, [sd["layers"] for sd in seq0], r=r + 128, n_kv_heads=H, head_dim=d,
                               landmarks=[False] * len(seq0), allow_notconv=True)
            torch.cuda.synchronize()
            tr = sum(o["stats"]["energy"] for o in wide)
            ranks_a, kept_a = xk.rank_allocate([o["eigvals"] for o in wide], len(seq0) * r, 128, r - 128, r + 128)
            kept_u = sum(float(np.sum(o["eigvals"][:r])) for o in wide)
            adaptive = {"budget": len(seq0) * r, "ranks": ranks_a, "sides": "K, V of each group of sequence 0",
                        "rel_err_uniform": round(math.sqrt(max(0.0, 1 - kept_u / tr)), 6),
                        "rel_err_adaptive": round(math.sqrt(max(0.0, 1 - kept_a / tr)), 6)}
            del wide
        rank_diag = {"group_rank95_frac": {k: [None if v is None else round(v, 4) for v in vs] for k, vs in grp.items()},
                     "layer0": layer0, "adaptive_rank": adaptive,
                     "note": "rank95_frac = rank holding 95 % of the eigenvalue sum / dimension; group sides "
                             f"of sequence 0 from the {r} leading Ritz values and trace(C) (None: beyond {r})"}

    # ---- Gram and projection kernels vs bf16 MFMA peak (the compression's GEMMs), one
    # batched Gram launch over the sides of one compression call; the projection of every
    # row of those sides onto their stored bases (the token-fold entry point with m = T and
    # no landmarks: one launch of the projection kernel per side, plus a small transpose) ----
    gsides = [sd["layers"] for sd in calls[0]]
    Sg = len(gsides)
    gram_out = torch.empty((Sg, n, n), dtype=torch.float64, device=dev)
    xk.gram(None, sides=gsides, out=gram_out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    xk.gram(None, sides=gsides, out=gram_out)
    e1.record()
    torch.cuda.synchronize()
    gram_ms = e0.elapsed_time(e1)
    gram_flops = Sg * float(n) * (n + 1) * T             # unique entries of C, 2T flops each
    del gram_out
    gram_tflops = gram_flops / (gram_ms * 1e-3) / 1e12
    proj_args = []
    proj_out = torch.empty((Sg, T, r), dtype=dt, device=dev)
    for i, sd in enumerate(calls[0]):
        proj_args.append(xk.append_args(layers=sd["layers"], Bt=sd["Bt"], A_new=proj_out[i], pos0=0, r=r))
    proj_ws = torch.empty(xk.append_ws_size(proj_args[0]), dtype=torch.uint8, device=dev)
    for a_ in proj_args:
        xk.compress_append(ctx, a_, proj_ws)
    torch.cuda.synchronize()
    e0.record()
    for a_ in proj_args:
        xk.compress_append(ctx, a_, proj_ws)
    e1.record()
    torch.cuda.synchronize()
    proj_ms = e0.elapsed_time(e1)
    proj_same = bool(torch.equal(proj_out[0], calls[0][0]["A"]))      # the same kernel as in compression
    del proj_out, proj_args, proj_ws
    proj_tflops = Sg * 2.0 * T * n * r / (proj_ms * 1e-3) / 1e12

    traffic = traffic_bytes(ATTEND_TRAFFIC) if (c.name == "llama64k" and D > 0) else None
    gram_traffic = traffic_bytes(GRAM_TRAFFIC) if c.name == "llama64k" else None
    algo_bytes_launch = float(np.mean(attend_union[samp]))
    shape = {"llama64k": "Llama-3.1-8B-shaped", "llama16k": "Llama-3.1-8B-shaped", "qwen122k": "Qwen2.5-7B-shaped",
             "tiny": "tiny"}.get(c.name, "Llama-3.1-8B-shaped")
    line = {
        "metric": "SR decode us/step + achieved HBM GB/s; KV compress tokens/s at 64k ctx",
        "value": round(dec_us, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_total / args.steps * 1e3, 2),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dt == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": f"{c.name}: {shape} KV, {Lyr} layers in groups of {G}, {H} KV heads x {d}, "
                               f"{Hq} q heads, T={T}, r={r} (K and V), xKV-SR, top-k {c.top_k} chunks of {c.chunk} "
                               f"+ {c.n_sink} sink + {c.n_local} local, {D} decode steps, batch {B}",
                   "T": T, "layers": Lyr, "group": G, "rank": r, "top_k": c.top_k, "decode_steps": D, "batch": B},
        "sr_decode_us_per_step": round(dec_us, 2),
        "sr_decode_graph": graph,
        "sr_decode_GBps": round(sr_gbps, 1),
        "sr_decode_bytes_per_step": int(decode_bytes_step),
        "compress_tokens_per_s": round(B * T / comp_s, 1),
        "compress_s": round(comp_s, 4),
        "compress_stats": {"err_est_max": float(max(st[0] for st in stats)), "sweeps": int(stats[0][2]),
                           "rounds": int(stats[0][3]), "sides": S, "calls": len(calls),
                           "sides_not_converged": notconv[0]},
        "roofline": {"bound": "hbm", "kernel": attend_kernel, "achieved": round(achieved_att, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved_att / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE)",
                     "algorithmic_bytes_per_launch": int(algo_bytes_launch),
                     "bytes": "union over KV heads of the gathered A_k and A_v rows + B_k slice + queries",
                     "achieved_per_head_sum": round(achieved_att_perhead, 1),
                     "avg_launch_us": round(att_ms_all * 1e3, 2),
                     "timed_launches": "one layer per decode step (layer = step mod layers), every timed step"},
        "roofline_gram": {"bound": "mfma", "kernel": "gram_bf16_kernel", "achieved": round(gram_tflops, 1),
                          "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(gram_tflops / BF16_PEAK_TFLOPS, 4),
                          "launch_ms": round(gram_ms, 3), "sides": Sg, "traffic": gram_traffic,
                          "traffic_unit": "L2-miss bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE)",
                          "unique_input_bytes": int(Sg * T * n * esz)},
        "roofline_project": {"bound": "mfma", "kernel": "project_tile_kernel", "achieved": round(proj_tflops, 1),
                             "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(proj_tflops / BF16_PEAK_TFLOPS, 4), "ms_all_sides": round(proj_ms, 3),
                             "sides": Sg, "flops": "2 T n r per side",
                             "timed": "one projection launch per side (+ a 2 MiB transpose of the basis each)",
                             "matches_compression_output": proj_same},
        "dense_baseline": dense,
        "sr_speedup_vs_dense": round(dense["us_per_step"] / dec_us, 3) if dense else None,
        "sr_variants": variants or None,
        "rank_diagnostics": rank_diag,
        "append_fold": append_rate,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(c, wl, layers, q_all, kn_all, vn_all, rows, D)
    print(json.dumps(line), flush=True)
    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {nbytes} bytes read, {nbytes} bytes written")
    ctx.close()


def dense_baseline(xk, ctx, c, layers, q_all, kn_all, vn_all, D, reps):
    """Full attention of the same queries over every cached position (post-RoPE keys, as a
    standard cache holds them, rotated on the GPU before timing), n_ctx = T + s + 1 at step s.
    Returns its time per decode step over all layers and its achieved HBM rate."""
    dev = q_all.device
    B, Lyr, T, d_kv, H, d, Hq = c.batch, c.n_layers, c.T, c.d_kv, c.n_kv_heads, c.head_dim, c.n_q_heads
    if c.torch_dtype != torch.bfloat16 or d != 128 or Hq // H > 8:
        return None
    n_max = T + (D if kn_all is not None else 0)
    dk = torch.empty((Lyr, B, n_max, d_kv), dtype=c.torch_dtype, device=dev)
    dv = torch.empty_like(dk)
    for l in range(Lyr):
        for b in range(B):
            xk.rope_rows(layers[(b, "K", l)], dk[l, b, :T], 0, H, d, c.rope_theta)
            dv[l, b, :T] = layers[(b, "V", l)]
            if kn_all is not None:
                xk.rope_rows(kn_all[:, l, b].contiguous(), dk[l, b, T:], T, H, d, c.rope_theta)
                dv[l, b, T:] = vn_all[:, l, b]
    out = torch.empty((Lyr, B, Hq, d), dtype=torch.float32, device=dev)
    n_ctx = [T + s + 1 if kn_all is not None else T for s in range(D)]
    args = [[xk.dense_args(batch=B, n_q_heads=Hq, n_kv_heads=H, head_dim=d, n_ctx=n_ctx[s], q_pos=n_ctx[s] - 1,
                           dtype=xk.XKV_BF16, scale=1.0 / math.sqrt(d), rope_theta=c.rope_theta, q=q_all[s, l],
                           K=dk[l], V=dv[l], ld_kv=d_kv, bstride_kv=n_max * d_kv, out=out[l])
             for l in range(Lyr)] for s in range(D)]
    ws = torch.empty(xk.dense_ws_size(args[-1][0]) // 4, dtype=torch.float32, device=dev)

    def run():
        for s in range(D):
            for l in range(Lyr):
                xk.dense_decode(ctx, args[s][l], ws)

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(reps):
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / D * 1e3)
    us = float(np.median(times))
    nbytes = float(np.mean([B * Lyr * (2 * n * d_kv * 2 + Hq * d * 2 + Hq * d * 4) for n in n_ctx]))
    del dk, dv
    return {"us_per_step": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4), "bytes_per_step": int(nbytes),
            "kernels": "dense_attend_kernel + dense_merge_kernel per layer"}


def cpu_baseline(c, wl, layers, q_all, kn_all, vn_all, rows, D):
    """The float64 oracle, as it stands, on a bounded sample of the same workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    f64 = lambda t: t.detach().double().cpu().numpy()
    # Decode sample: layers 0 and 1 at the first four decode steps, on a cache of the same
    # shapes that involves no GPU output: the generator's own rank-r factors and the
    # oracle's landmarks of the original keys.
    sample_layers, sample_steps = [0, 1], [s for s in range(4) if s < D]
    t_dec = 0.0
    for l in sample_layers:
        A_k, Bk = (f64(x) for x in wl.factor_cache(0, "K", l, c.rank))
        A_v, Bv = (f64(x) for x in wl.factor_cache(0, "V", l, c.rank))
        Bk, Bv = Bk.T, Bv.T
        Kl, Vl = layers[(0, "K", l)], layers[(0, "V", l)]
        lm = oracle.landmarks(f64(Kl), c.n_kv_heads, c.head_dim, c.chunk, c.rope_theta)
        k_ex = {t: f64(Kl[t]) for t in rows}
        v_ex = {t: f64(Vl[t]) for t in rows}
        for s in sample_steps:
            if c.append:
                k_ex[c.T + s] = f64(kn_all[s, l, 0])
                v_ex[c.T + s] = f64(vn_all[s, l, 0])
            q = f64(q_all[s, l, 0])
            t0 = time.perf_counter()
            oracle.sr_decode_layer(q, T=c.T, n_gen=(s + 1) if c.append else 0, n_kv_heads=c.n_kv_heads,
                                   chunk=c.chunk, top_k=c.top_k, n_sink=c.n_sink, n_local=c.n_local,
                                   landmarks_l=lm, A_k=A_k, B_k_l=Bk, A_v=A_v, B_v_l=Bv, k_exact=k_ex, v_exact=v_ex)
            t_dec += time.perf_counter() - t0
    per_layer_step = t_dec / (len(sample_layers) * len(sample_steps))
    us_per_step = per_layer_step * c.n_layers * c.batch * 1e6
    # Compression sample: the oracle's factorisation of one group side (K of group 0) on its
    # first 16384 tokens; the Gram/projection parts scale with T, the n x n eigensolve does not.
    T_s = min(16384, c.T)
    Ks = [f64(layers[(0, "K", i)][:T_s]) for i in range(c.group)]
    t0 = time.perf_counter()
    X = oracle.group_matrix(Ks)
    C_ = oracle.gram(X)
    t1 = time.perf_counter()
    lam, V = oracle.eig_desc(C_)
    t2 = time.perf_counter()
    A = X @ V[:, :c.rank]
    t3 = time.perf_counter()
    lm = oracle.landmarks(Ks[0], c.n_kv_heads, c.head_dim, c.chunk)
    t4 = time.perf_counter()
    scale = c.T / T_s
    side_s = (t1 - t0 + t3 - t2 + (t4 - t3) * c.group) * scale + (t2 - t1)
    n_sides = 2 * c.n_groups * c.batch
    comp_s = side_s * n_sides
    return {"value": round(us_per_step, 1), "unit": "us/step", "cores": int(cores), "kind": "oracle",
            "sample": f"SR decode of layers 0-1 at decode steps 0-{len(sample_steps) - 1} "
                      f"({len(sample_layers) * len(sample_steps)} layer-steps, on a stand-in cache of the same shapes), "
                      f"scaled x{c.n_layers} layers x{c.batch} sequences; compression of one group side on its first {T_s} tokens "
                      f"(Gram+projection+landmarks scaled x{scale:g} in T, eigensolve of n={c.n} once), "
                      f"scaled x{n_sides} sides",
            "compress_tokens_per_s": round(c.batch * c.T / comp_s, 2),
            "sample_seconds": round(t_dec + (t4 - t0), 2)}


if __name__ == "__main__":
    main()
