"""ctypes binding of libxkv (argument marshalling only).

Every computation runs in the HIP kernels of libxkv.so (or, for the
Rayleigh-Ritz eigensolve, in its plain-C host routine).  Torch tensors only
provide device memory and the stream.  There is no fallback: if the library
is missing or was built for another GPU, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libxkv.so")

XKV_OK, XKV_EINVAL, XKV_EUNSUPPORTED, XKV_EWORKSPACE, XKV_EHIP, XKV_ENUMERIC, XKV_ENOTCONV = 0, -1, -2, -3, -4, -5, -6
XKV_F32, XKV_BF16 = 0, 1
_CODES = {-1: "XKV_EINVAL", -2: "XKV_EUNSUPPORTED", -3: "XKV_EWORKSPACE", -4: "XKV_EHIP", -5: "XKV_ENUMERIC",
          -6: "XKV_ENOTCONV"}


class XkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_CODES.get(code, code)}: {msg}")
        self.code = code


class CompressDesc(C.Structure):
    _fields_ = [("T", C.c_int), ("G", C.c_int), ("d_kv", C.c_int), ("r", C.c_int), ("dtype", C.c_int),
                ("n_kv_heads", C.c_int), ("head_dim", C.c_int), ("chunk", C.c_int),
                ("rope_theta", C.c_double), ("oversample", C.c_int), ("fp32_iters", C.c_int),
                ("fp64_iters", C.c_int), ("seed", C.c_uint64), ("tol", C.c_double), ("max_rounds", C.c_int)]


class Side(C.Structure):
    _fields_ = [("layers", C.POINTER(C.c_void_p)), ("ld_layer", C.c_long), ("A", C.c_void_p),
                ("Bt", C.c_void_p), ("landmarks", C.c_void_p), ("eigvals", C.POINTER(C.c_double)),
                ("Vr64", C.c_void_p), ("stats", C.POINTER(C.c_double))]


class SrArgs(C.Structure):
    _fields_ = [("batch", C.c_int), ("n_q_heads", C.c_int), ("n_kv_heads", C.c_int), ("head_dim", C.c_int),
                ("T", C.c_int), ("n_gen", C.c_int), ("chunk", C.c_int), ("top_k", C.c_int),
                ("n_sink", C.c_int), ("n_local", C.c_int), ("r_k", C.c_int), ("r_v", C.c_int),
                ("dtype", C.c_int), ("scale", C.c_float), ("rope_theta", C.c_double),
                ("q", C.c_void_p),
                ("A_k", C.c_void_p), ("ld_A_k", C.c_long), ("bstride_A_k", C.c_long),
                ("Bt_k", C.c_void_p), ("ld_Bt_k", C.c_long), ("bstride_Bt_k", C.c_long),
                ("A_v", C.c_void_p), ("ld_A_v", C.c_long), ("bstride_A_v", C.c_long),
                ("Bt_v", C.c_void_p), ("ld_Bt_v", C.c_long), ("bstride_Bt_v", C.c_long),
                ("V_full", C.c_void_p), ("ld_V", C.c_long), ("bstride_V", C.c_long),
                ("landmarks", C.c_void_p), ("bstride_lm", C.c_long),
                ("k_tail", C.c_void_p), ("v_tail", C.c_void_p), ("ld_tail", C.c_long), ("bstride_tail", C.c_long),
                ("k_new", C.c_void_p), ("v_new", C.c_void_p), ("bstride_new", C.c_long),
                ("out", C.c_void_p), ("sel", C.c_void_p)]


class AppendArgs(C.Structure):
    _fields_ = [("m", C.c_int), ("pos0", C.c_long), ("G", C.c_int), ("d_kv", C.c_int), ("r", C.c_int),
                ("dtype", C.c_int), ("n_kv_heads", C.c_int), ("head_dim", C.c_int), ("chunk", C.c_int),
                ("rope_theta", C.c_double), ("layers", C.POINTER(C.c_void_p)), ("ld_layer", C.c_long),
                ("Bt", C.c_void_p), ("A_new", C.c_void_p), ("landmarks_new", C.c_void_p)]


class RankInfo(C.Structure):
    _fields_ = [("energy_rank", C.c_int), ("covered", C.c_double), ("numerical_rank", C.c_int),
                ("erank", C.c_double), ("ner", C.c_double)]


class DenseArgs(C.Structure):
    _fields_ = [("batch", C.c_int), ("n_q_heads", C.c_int), ("n_kv_heads", C.c_int), ("head_dim", C.c_int),
                ("n_ctx", C.c_long), ("q_pos", C.c_long), ("dtype", C.c_int), ("scale", C.c_float),
                ("rope_theta", C.c_double), ("q", C.c_void_p), ("K", C.c_void_p), ("V", C.c_void_p),
                ("ld_kv", C.c_long), ("bstride_kv", C.c_long), ("out", C.c_void_p)]


_lib = None


def lib():
    """The loaded libxkv (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(python -m kv_cache_cross_amd.build)")
        L = C.CDLL(LIB_PATH)
        vp, i, l, sz = C.c_void_p, C.c_int, C.c_long, C.c_size_t
        L.xkv_version.restype = i
        L.xkv_last_error.restype = C.c_char_p
        L.xkv_ctx_create.argtypes = [i, i, C.POINTER(vp)]
        L.xkv_ctx_destroy.argtypes = [vp]
        L.xkv_ctx_destroy.restype = None
        L.xkv_compress_ws_size.argtypes = [C.POINTER(CompressDesc), i, C.POINTER(sz)]
        L.xkv_compress_sides.argtypes = [vp, C.POINTER(CompressDesc), i, C.POINTER(Side), vp, sz, vp]
        L.xkv_compress_group.argtypes = [vp, C.POINTER(CompressDesc), C.POINTER(Side), vp, sz, vp]
        L.xkv_sr_ws_size.argtypes = [C.POINTER(SrArgs), C.POINTER(sz)]
        for name in ("xkv_sr_select", "xkv_sr_attend", "xkv_sr_decode"):
            getattr(L, name).argtypes = [vp, C.POINTER(SrArgs), vp, sz, vp]
        L.xkv_sr_decode_layers.argtypes = [vp, i, C.POINTER(SrArgs), vp, sz, vp, C.POINTER(vp)]
        L.xkv_sr_decode_layers_noalloc.argtypes = [vp, i, C.POINTER(SrArgs), vp]
        L.xkv_gram.argtypes = [C.POINTER(vp), i, l, i, i, i, i, vp, vp]
        L.xkv_topk.argtypes = [vp, i, i, l, i, vp, vp]
        L.xkv_host_eigh.argtypes = [i, vp, i, vp, vp]
        L.xkv_dense_ws_size.argtypes = [C.POINTER(DenseArgs), C.POINTER(sz)]
        L.xkv_dense_decode.argtypes = [vp, C.POINTER(DenseArgs), vp, sz, vp]
        L.xkv_rank_stats.argtypes = [C.POINTER(C.c_double), i, C.c_double, C.c_double, i, C.POINTER(RankInfo)]
        L.xkv_rank_allocate.argtypes = [vp, i, i, i, l, i, i, vp, vp]
        L.xkv_append_ws_size.argtypes = [C.POINTER(AppendArgs), C.POINTER(sz)]
        L.xkv_compress_append.argtypes = [vp, C.POINTER(AppendArgs), vp, sz, vp]
        L.xkv_rope_rows.argtypes = [vp, l, vp, l, i, l, i, i, C.c_double, i, vp]
        _lib = L
    return _lib


def _check(rc: int):
    if rc != XKV_OK:
        raise XkvError(rc, lib().xkv_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return XKV_BF16
    if t.dtype == torch.float32:
        return XKV_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


class Context:
    """Host-side resources of the library, bound to one HIP device."""

    def __init__(self, device: int = 0, host_threads: int = 0):
        self.handle = C.c_void_p()
        _check(lib().xkv_ctx_create(device, host_threads, C.byref(self.handle)))
        self.device = device

    def close(self):
        if self.handle:
            lib().xkv_ctx_destroy(self.handle)
            self.handle = C.c_void_p()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def make_desc(*, T, G, d_kv, r, dtype, n_kv_heads, head_dim, chunk=8, rope_theta=10000.0,
              oversample=-1, fp32_iters=2, fp64_iters=2, seed=0, tol=0.0, max_rounds=0) -> CompressDesc:
    return CompressDesc(T, G, d_kv, r, dtype, n_kv_heads, head_dim, chunk, rope_theta, oversample,
                        fp32_iters, fp64_iters, seed, tol, max_rounds)


def compress_ws_size(desc: CompressDesc, n_sides: int) -> int:
    n = C.c_size_t()
    _check(lib().xkv_compress_ws_size(C.byref(desc), n_sides, C.byref(n)))
    return n.value


def compress_sides(ctx: Context, desc: CompressDesc, sides, ws: torch.Tensor, stream=None):
    """sides: list of dicts with 'layers' (list of G tensors, T x d_kv), 'A' (T x r), 'Bt' (n x r),
    optional 'landmarks' (G x H_kv x T/chunk x d) and 'Vr64' (n x r float64).  Returns the r leading
    Ritz values per side and per-side stats (error estimate, relative gap, sweeps, rounds,
    trace of the Gram)."""
    S = len(sides)
    arr = (Side * S)()
    keep = []
    evals = [np.zeros(desc.r, dtype=np.float64) for _ in range(S)]
    stats = [np.zeros(5, dtype=np.float64) for _ in range(S)]
    for s, sd in enumerate(sides):
        layers = sd["layers"]
        ptrs = (C.c_void_p * len(layers))(*[t.data_ptr() for t in layers])
        keep.append(ptrs)
        arr[s].layers = C.cast(ptrs, C.POINTER(C.c_void_p))
        arr[s].ld_layer = layers[0].stride(0)
        arr[s].A = sd["A"].data_ptr()
        arr[s].Bt = sd["Bt"].data_ptr()
        arr[s].landmarks = sd["landmarks"].data_ptr() if sd.get("landmarks") is not None else None
        arr[s].eigvals = evals[s].ctypes.data_as(C.POINTER(C.c_double))
        arr[s].Vr64 = sd["Vr64"].data_ptr() if sd.get("Vr64") is not None else None
        arr[s].stats = stats[s].ctypes.data_as(C.POINTER(C.c_double))
    rc = lib().xkv_compress_sides(ctx.handle, C.byref(desc), S, arr, _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream))
    if rc != XKV_OK:
        err = XkvError(rc, lib().xkv_last_error().decode())
        if rc == XKV_ENOTCONV:   # every output is written; the caller may still use them
            err.evals, err.stats = evals, stats
        raise err
    return evals, stats


def sr_args(**kw) -> SrArgs:
    """Build an SrArgs from keyword arguments; tensors become device pointers."""
    a = SrArgs()
    for name, _ in SrArgs._fields_:
        if name not in kw:
            continue
        v = kw[name]
        if isinstance(v, torch.Tensor):
            v = v.data_ptr()
        setattr(a, name, v)
    return a


def sr_ws_size(args: SrArgs) -> int:
    n = C.c_size_t()
    _check(lib().xkv_sr_ws_size(C.byref(args), C.byref(n)))
    return n.value


def _sr_call(fn, ctx, args, ws, stream):
    _check(fn(ctx.handle, C.byref(args), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def sr_select(ctx, args, ws, stream=None):
    _sr_call(lib().xkv_sr_select, ctx, args, ws, stream)


def sr_attend(ctx, args, ws, stream=None):
    _sr_call(lib().xkv_sr_attend, ctx, args, ws, stream)


def sr_decode(ctx, args, ws, stream=None):
    _sr_call(lib().xkv_sr_decode, ctx, args, ws, stream)


def sr_args_array(args_list):
    """Pack SrArgs into a C array for sr_decode_layers."""
    arr = (SrArgs * len(args_list))()
    for i, a in enumerate(args_list):
        arr[i] = a
    return arr


def sr_decode_layers(ctx, arr, ws, stream=None, attend_events=None):
    """One decode step through len(arr) layers; arr from sr_args_array.  attend_events: optional
    list of 2*len(arr) torch.cuda.Event (enable_timing=True) or None, stamped at the start and end
    of each layer's attend kernel (a layer whose pair is None is not timed)."""
    ev = None
    if attend_events is not None:
        ev = (C.c_void_p * len(attend_events))(*[None if e is None else e.cuda_event for e in attend_events])
    _check(lib().xkv_sr_decode_layers(ctx.handle, len(arr), arr, _ptr(ws), ws.numel() * ws.element_size(),
                                      _stream(stream), ev))


SR_SCRATCH_BYTES = 64 << 20


def sr_decode_layers_noalloc(ctx, arr, stream=None):
    """One decode step through len(arr) layers with the library's own scratch (no
    workspace argument; calls on one GPU must not overlap)."""
    _check(lib().xkv_sr_decode_layers_noalloc(ctx.handle, len(arr), arr, _stream(stream)))


def gram(layers, stream=None, sides=None, out=None) -> torch.Tensor:
    """X^T X of the horizontally concatenated layers (float64, n x n) on the layers' device.
    With ``sides`` (a list of layer lists) all sides go in one launch and the result is
    n_sides x n x n."""
    groups = sides if sides is not None else [layers]
    S, G = len(groups), len(groups[0])
    T, d_kv = groups[0][0].shape
    n = G * d_kv
    if out is None:
        out = torch.empty((S, n, n), dtype=torch.float64, device=groups[0][0].device)
    ptrs = (C.c_void_p * (S * G))(*[t.data_ptr() for g in groups for t in g])
    _check(lib().xkv_gram(ptrs, S, groups[0][0].stride(0), T, G, d_kv, _dtype_code(groups[0][0]), _ptr(out),
                          _stream(stream)))
    return out if sides is not None else out[0]


def topk(scores: torch.Tensor, n_cand: int, k: int, stream=None) -> torch.Tensor:
    rows = scores.shape[0]
    sel = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
    _check(lib().xkv_topk(_ptr(scores), rows, n_cand, scores.stride(0), k, _ptr(sel), _stream(stream)))
    return sel


def host_eigh(H: np.ndarray, nvec: int):
    """Largest nvec eigenpairs of symmetric H with the library's plain-C solver (no GPU needed)."""
    H = np.ascontiguousarray(H, dtype=np.float64)
    n = H.shape[0]
    w = np.zeros(nvec)
    Z = np.zeros((n, nvec))
    _check(lib().xkv_host_eigh(n, H.ctypes.data, nvec, w.ctypes.data, Z.ctypes.data))
    return w, Z


def append_args(*, layers, Bt, A_new, pos0: int, r: int, n_kv_heads: int = 0, head_dim: int = 0,
                chunk: int = 0, rope_theta: float = 10000.0, landmarks_new=None):
    """AppendArgs for rows appended after a compressed prefix; `layers` are the G new-row
    tensors (m x d_kv each).  The pointer array is kept alive on the returned object."""
    m, d_kv = layers[0].shape
    ptrs = (C.c_void_p * len(layers))(*[x.data_ptr() for x in layers])
    a = AppendArgs(m=m, pos0=pos0, G=len(layers), d_kv=d_kv, r=r, dtype=_dtype_code(layers[0]),
                   n_kv_heads=n_kv_heads, head_dim=head_dim, chunk=chunk, rope_theta=rope_theta,
                   layers=C.cast(ptrs, C.POINTER(C.c_void_p)), ld_layer=layers[0].stride(0), Bt=Bt.data_ptr(),
                   A_new=A_new.data_ptr(), landmarks_new=landmarks_new.data_ptr() if landmarks_new is not None else None)
    a._keep = ptrs
    return a


def append_ws_size(args: AppendArgs) -> int:
    n = C.c_size_t()
    _check(lib().xkv_append_ws_size(C.byref(args), C.byref(n)))
    return n.value


def compress_append(ctx, args: AppendArgs, ws: torch.Tensor, stream=None):
    _check(lib().xkv_compress_append(ctx.handle, C.byref(args), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)))


def rank_stats(eigvals, total: float = 0.0, frac: float = 0.95, complete: bool = False) -> dict:
    """Rank diagnostics of a spectrum (host only): energy rank at `frac` of `total`
    (<= 0: the sum of the given values), covered fraction and, for a complete spectrum,
    numerical rank, effective rank and NER."""
    v = np.ascontiguousarray(np.asarray(eigvals, dtype=np.float64))
    out = RankInfo()
    _check(lib().xkv_rank_stats(v.ctypes.data_as(C.POINTER(C.c_double)), v.size, float(total), float(frac),
                                int(bool(complete)), C.byref(out)))
    return {name: getattr(out, name) for name, _ in RankInfo._fields_}


def rank_allocate(spectra, budget: int, granule: int, r_min: int, r_max: int):
    """Per-side ranks at a total budget (host only): returns (ranks, kept energy).
    `spectra`: one sequence of at least r_max leading eigenvalues per side, descending."""
    S = len(spectra)
    eig = np.ascontiguousarray(np.stack([np.asarray(x, dtype=np.float64)[:r_max] for x in spectra]))
    ranks = np.zeros(S, dtype=np.int32)
    kept = np.zeros(1, dtype=np.float64)
    _check(lib().xkv_rank_allocate(eig.ctypes.data, S, r_max, r_max, int(budget), granule, r_min, ranks.ctypes.data,
                                   kept.ctypes.data))
    return [int(x) for x in ranks], float(kept[0])


def dense_args(**kw) -> DenseArgs:
    """Build a DenseArgs from keyword arguments; tensors become device pointers."""
    a = DenseArgs()
    for name, _ in DenseArgs._fields_:
        if name in kw:
            v = kw[name]
            setattr(a, name, v.data_ptr() if isinstance(v, torch.Tensor) else v)
    return a


def dense_ws_size(args: DenseArgs) -> int:
    n = C.c_size_t()
    _check(lib().xkv_dense_ws_size(C.byref(args), C.byref(n)))
    return n.value


def dense_decode(ctx, args: DenseArgs, ws: torch.Tensor, stream=None):
    _check(lib().xkv_dense_decode(ctx.handle, C.byref(args), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)))


def rope_rows(x: torch.Tensor, y: torch.Tensor, pos0: int, n_heads: int, head_dim: int,
              rope_theta: float = 10000.0, stream=None):
    """y[row] = RoPE(x[row], pos0 + row) (rows x n_heads*head_dim; x and y may alias)."""
    if y.dtype != x.dtype or y.shape[0] < x.shape[0]:
        raise ValueError("rope_rows: y needs x's dtype and at least x's rows")
    _check(lib().xkv_rope_rows(_ptr(x), x.stride(0), _ptr(y), y.stride(0), x.shape[0], pos0, n_heads, head_dim,
                               rope_theta, _dtype_code(x), _stream(stream)))
