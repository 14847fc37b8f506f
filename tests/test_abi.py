"""The C ABI without a GPU: the library loads, exports every declared entry point,
rejects bad arguments before touching the device, and its host eigensolver
(used for the Rayleigh-Ritz step) is correct."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import kv_cache_cross_amd as xk
from kv_cache_cross_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "xkv.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(xkv_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 14
    lib = xk.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/xkv.h but not exported"
    assert lib.xkv_version() >= 100


def test_struct_layouts_match_header_order():
    # Field order of the ctypes mirrors follows the header's declaration order.
    src = open(HEADER).read()
    body = src[src.index("typedef struct {\n  int batch;"):src.index("} xkv_sr_args;")]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = re.findall(r"\*?\s*([a-zA-Z_][a-zA-Z0-9_]*)\s*[,;]", body)
    assert names == [f for f, _ in L.SrArgs._fields_]


def test_dense_struct_layout_matches_header_order():
    src = open(HEADER).read()
    end = src.index("} xkv_dense_args;")
    body = src[src.rindex("typedef struct {", 0, end):end]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = re.findall(r"\*?\s*([a-zA-Z_][a-zA-Z0-9_]*)\s*[,;]", body.replace("typedef struct {", ""))
    assert names == [f for f, _ in L.DenseArgs._fields_]


def test_dense_validation():
    base = dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, n_ctx=1000, q_pos=999, dtype=xk.XKV_BF16,
                scale=0.088, rope_theta=1e4, q=16, K=16, V=16, ld_kv=1024, bstride_kv=0, out=16)
    n = xk.dense_ws_size(xk.dense_args(**base))
    assert n >= 1 * 8 * 4 * 4 * 130 * 4
    for bad, code in [(dict(head_dim=64, ld_kv=512), L.XKV_EUNSUPPORTED), (dict(dtype=xk.XKV_F32), L.XKV_EUNSUPPORTED),
                      (dict(n_ctx=0), L.XKV_EINVAL), (dict(n_ctx=512 * 2048 + 1), L.XKV_EUNSUPPORTED),
                      (dict(n_q_heads=72), L.XKV_EUNSUPPORTED), (dict(K=8), L.XKV_EINVAL),
                      (dict(ld_kv=1000), L.XKV_EINVAL), (dict(V=0), L.XKV_EINVAL)]:
        with pytest.raises(xk.XkvError) as e:
            xk.dense_ws_size(xk.dense_args(**dict(base, **bad)))
        assert e.value.code == code, bad
    # Split size: the smallest multiple of 128 rows that keeps the grid at or under 512
    # blocks (64k context, 8 KV heads: 1152 rows, 57 splits).
    big = xk.dense_ws_size(xk.dense_args(**dict(base, n_ctx=65537)))
    assert big == 8 * 57 * 4 * 130 * 4
    lib = xk.lib()
    assert lib.xkv_dense_decode(None, C.byref(xk.dense_args(**base)), None, 0, None) == L.XKV_EINVAL
    assert lib.xkv_rope_rows(None, 128, None, 128, 4, 0, 1, 128, 1e4, xk.XKV_BF16, None) == L.XKV_EINVAL
    assert lib.xkv_rope_rows(16, 64, 16, 128, 4, 0, 1, 128, 1e4, xk.XKV_BF16, None) == L.XKV_EINVAL


def _desc(**kw):
    base = dict(T=256, G=2, d_kv=64, r=16, dtype=xk.XKV_F32, n_kv_heads=1, head_dim=64)
    base.update(kw)
    return xk.make_desc(**base)


def test_compress_ws_size_and_validation():
    n = xk.compress_ws_size(_desc(), 1)
    assert n > 0 and n % 256 == 0
    assert xk.compress_ws_size(_desc(), 4) > 3 * n
    for bad in [dict(r=0), dict(r=129), dict(d_kv=60, head_dim=60), dict(G=0), dict(T=0), dict(fp64_iters=0),
                dict(dtype=7), dict(n_kv_heads=2)]:
        with pytest.raises(xk.XkvError) as e:
            xk.compress_ws_size(_desc(**bad), 1)
        assert e.value.code == L.XKV_EINVAL, bad


def test_compress_rejects_null_context():
    d = _desc()
    sides = (L.Side * 1)()
    rc = xk.lib().xkv_compress_sides(None, C.byref(d), 1, sides, None, 0, None)
    assert rc == L.XKV_EINVAL
    assert b"ctx" in xk.lib().xkv_last_error()


def test_sr_ws_size_validation():
    base = dict(batch=1, n_q_heads=4, n_kv_heads=2, head_dim=128, T=64, n_gen=1, chunk=8, top_k=2, n_sink=4,
                n_local=16, r_k=128, r_v=128, dtype=xk.XKV_BF16, scale=0.1, rope_theta=1e4, q=16, A_k=16,
                ld_A_k=128, Bt_k=16, ld_Bt_k=128, A_v=16, ld_A_v=128, Bt_v=16, ld_Bt_v=128, landmarks=16,
                k_tail=16, v_tail=16, ld_tail=256, out=16, sel=16)
    assert xk.sr_ws_size(xk.sr_args(**base)) > 0
    for bad, code in [(dict(n_q_heads=5), L.XKV_EINVAL), (dict(head_dim=96), L.XKV_EUNSUPPORTED),
                      (dict(chunk=12), L.XKV_EUNSUPPORTED), (dict(T=60), L.XKV_EINVAL),
                      (dict(n_q_heads=36, n_kv_heads=2), L.XKV_EUNSUPPORTED), (dict(q=0), L.XKV_EINVAL),
                      (dict(n_sink=40, n_local=40), L.XKV_EINVAL), (dict(A_k=8), L.XKV_EINVAL)]:
        kw = dict(base, **bad)
        with pytest.raises(xk.XkvError) as e:
            xk.sr_ws_size(xk.sr_args(**kw))
        assert e.value.code == code, bad
    # Attend blocks per head: every chunk of a 64k prefix (1023 blocks of 64 rows plus
    # exact tiles) fits the matrix-core path's 1088; the value-space path stops at 257.
    full64k = dict(base, T=65536, n_local=64, top_k=1 << 20)
    assert xk.sr_ws_size(xk.sr_args(**full64k)) > 0
    for bad in (dict(full64k, T=65536 + 8 * 1024), dict(full64k, r_v=0, V_full=16, ld_V=256)):
        with pytest.raises(xk.XkvError) as e:
            xk.sr_ws_size(xk.sr_args(**bad))
        assert e.value.code == L.XKV_EUNSUPPORTED, bad


def test_topk_and_gram_validation():
    lib = xk.lib()
    assert lib.xkv_topk(None, 1, 10, 10, 2, None, None) == L.XKV_EINVAL
    assert lib.xkv_topk(16, 1, 40000, 40000, 2, 16, None) == L.XKV_EINVAL
    ptrs = (C.c_void_p * 1)(None)
    assert lib.xkv_gram(ptrs, 1, 64, 16, 1, 64, xk.XKV_F32, 16, None) == L.XKV_EINVAL


def test_ctx_create_rejects_bad_device():
    h = C.c_void_p()
    rc = xk.lib().xkv_ctx_create(-1, 0, C.byref(h))
    assert rc in (L.XKV_EINVAL, L.XKV_EHIP)


@pytest.mark.parametrize("n,nvec", [(1, 1), (2, 1), (3, 2), (7, 3), (60, 60), (200, 40), (768, 512)])
def test_host_eigh_matches_lapack(n, nvec):
    rng = np.random.default_rng(n)
    G = rng.standard_normal((n, n))
    H = (G * np.arange(1, n + 1) ** -0.8) @ G.T            # graded, PSD like Q^T C Q
    w, Z = xk.host_eigh(H, nvec)
    ref_w = np.linalg.eigvalsh(H)[::-1][:nvec]
    np.testing.assert_allclose(w, ref_w, rtol=1e-11, atol=1e-12 * ref_w[0])
    np.testing.assert_allclose(Z.T @ Z, np.eye(nvec), atol=1e-12)
    np.testing.assert_allclose(H @ Z, Z * w, atol=1e-11 * abs(ref_w[0]))


def test_host_eigh_clustered_and_degenerate():
    rng = np.random.default_rng(0)
    Q, _ = np.linalg.qr(rng.standard_normal((50, 50)))
    lam = np.concatenate([np.full(10, 5.0), 5.0 + 1e-12 * np.arange(10), np.linspace(1, 2, 30)])
    H = (Q * lam) @ Q.T
    w, Z = xk.host_eigh(H, 20)
    np.testing.assert_allclose(np.sort(w), np.sort(lam)[-20:], atol=1e-12)
    P = Z @ Z.T
    Pref = Q[:, :20] @ Q[:, :20].T
    np.testing.assert_allclose(P, Pref, atol=1e-9)


@pytest.mark.parametrize("order", ["tridiagonal_first", "dense_first"])
def test_host_eigh_skipped_reflectors(order):
    # A tridiagonal block with positive off-diagonals has nothing to reduce: its columns
    # are already e_1 below the subdiagonal, the reflector factor is 0 and the reduction
    # skips those steps, then takes its next column from the matrix again.
    rng = np.random.default_rng(5)
    nt, nd = 20, 30
    T = np.diag(rng.uniform(1, 2, nt)) + np.diag(rng.uniform(0.1, 0.5, nt - 1), 1)
    T = T + np.triu(T, 1).T
    G = rng.standard_normal((nd, nd))
    D = G @ G.T / nd
    Z0 = np.zeros((nt, nd))
    H = np.block([[T, Z0], [Z0.T, D]]) if order == "tridiagonal_first" else np.block([[D, Z0.T], [Z0, T]])
    w, Z = xk.host_eigh(H, 25)
    ref_w = np.linalg.eigvalsh(H)[::-1][:25]
    np.testing.assert_allclose(w, ref_w, rtol=1e-12, atol=1e-13 * ref_w[0])
    np.testing.assert_allclose(Z.T @ Z, np.eye(25), atol=1e-12)
    np.testing.assert_allclose(H @ Z, Z * w, atol=1e-11 * abs(ref_w[0]))


def test_host_eigh_rejects_non_finite():
    H = np.eye(300)
    H[7, 3] = np.nan
    with pytest.raises(xk.XkvError, match="not finite"):
        xk.host_eigh(H, 10)
    H = np.eye(40)
    H[39, 39] = np.inf
    with pytest.raises(xk.XkvError, match="not finite"):
        xk.host_eigh(H, 4)


def test_host_eigh_rejects_bad_args():
    with pytest.raises(xk.XkvError):
        xk.host_eigh(np.eye(4), 5)


def test_rank_info_layout_matches_header_order():
    src = open(HEADER).read()
    body = src[src.index("typedef struct {\n  int energy_rank;"):src.index("} xkv_rank_info;")]
    names = re.findall(r"\s([a-zA-Z_][a-zA-Z0-9_]*);", body)
    assert names == [f for f, _ in L.RankInfo._fields_]


def test_rank_stats_matches_oracle():
    # Host entry point (no GPU work) against the oracle on random, flat, spiked and
    # rank-deficient spectra, complete and partial.
    import oracle
    rng = np.random.default_rng(11)
    spectra = [rng.exponential(size=300) ** 4, np.ones(64), np.r_[1e3, np.full(99, 1e-3)],
               np.r_[rng.random(40) + 1.0, np.zeros(24)], np.geomspace(1.0, 1e-12, 200)]
    for lam in spectra:
        for frac in (0.5, 0.9, 0.95, 1.0):
            got = xk.rank_stats(lam, frac=frac, complete=True)
            assert got["energy_rank"] == oracle.energy_rank(lam, frac)
            assert got["numerical_rank"] == oracle.numerical_rank(lam)
            assert got["erank"] == pytest.approx(oracle.effective_rank(lam), rel=1e-12)
            assert got["ner"] == pytest.approx(oracle.ner(lam), rel=1e-12)
            assert got["covered"] == pytest.approx(1.0)
        # Leading part of the spectrum against the full total.
        top = np.sort(lam)[::-1][: len(lam) // 3]
        part = xk.rank_stats(top, total=lam.sum(), frac=0.6)
        assert part["energy_rank"] == oracle.energy_rank(top, 0.6, total=lam.sum())
        assert part["covered"] == pytest.approx(top.sum() / lam.sum())
        assert part["numerical_rank"] == -1 and np.isnan(part["ner"])
    with pytest.raises(xk.XkvError):
        xk.rank_stats(np.ones(4), frac=0.0)
    with pytest.raises(xk.XkvError):
        xk.rank_stats(np.ones(4), frac=1.5)


def test_append_args_layout_and_validation():
    src = open(HEADER).read()
    body = src[src.index("typedef struct {\n  int m;"):src.index("} xkv_append_args;")]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = re.findall(r"\*?\s*([a-zA-Z_][a-zA-Z0-9_]*)\s*[,;]", body)
    assert names == [f for f, _ in L.AppendArgs._fields_]
    ptrs = (C.c_void_p * 2)(16, 16)
    base = dict(m=64, pos0=128, G=2, d_kv=256, r=128, dtype=xk.XKV_BF16, n_kv_heads=2, head_dim=128, chunk=8,
                rope_theta=1e4, layers=C.cast(ptrs, C.POINTER(C.c_void_p)), ld_layer=256, Bt=16, A_new=16,
                landmarks_new=16)
    n = C.c_size_t()
    assert xk.lib().xkv_append_ws_size(C.byref(L.AppendArgs(**base)), C.byref(n)) == 0
    assert n.value >= 128 * 512 * 2
    for bad in (dict(m=0), dict(r=513), dict(d_kv=12), dict(m=60), dict(pos0=4), dict(ld_layer=250),
                dict(Bt=None), dict(dtype=7), dict(n_kv_heads=3)):
        assert xk.lib().xkv_append_ws_size(C.byref(L.AppendArgs(**dict(base, **bad))), C.byref(n)) == L.XKV_EINVAL, bad
    # Without landmarks, m and pos0 need not be multiples of chunk.
    assert xk.lib().xkv_append_ws_size(C.byref(L.AppendArgs(**dict(base, m=60, pos0=4, landmarks_new=None))),
                                       C.byref(n)) == 0
