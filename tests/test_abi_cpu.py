"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and rejects invalid arguments on the host before launching anything."""

import ctypes
import os

import pytest

from sparse_retrieval_memory_amd import _lib

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libmsa.so not built")
N = None


def test_exports_every_declared_symbol():
    lib = _lib.load()
    names = _lib.declared_symbols()
    assert {"msa_pool_chunks", "msa_route_scores", "msa_topk_docs", "msa_sparse_attn_decode",
            "msa_fetch_docs", "msa_gather_docs", "msa_append_router_rows", "msa_encode_router_keys",
            "msa_encode_workspace_bytes", "msa_store_delete", "msa_store_append",
            "msa_store_delete_workspace_bytes", "msa_route_scores_backward",
            "msa_route_backward_workspace_bytes", "msa_sparse_attn_backward",
            "msa_sparse_attn_backward_workspace_bytes", "msa_sparse_attn_forward",
            "msa_sparse_attn_backward_saved", "msa_sparse_attn_local_partial",
            "msa_sparse_attn_memory_merge", "msa_route_topk", "msa_route_topk_workspace_bytes"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(_lib.SIGNATURES) == set(names)
    assert lib.msa_version() == 100
    assert lib.msa_status_string(-3) == b"workspace too small"


def _code(name, *args):
    return _lib.raw(name, *args)


def test_route_validation():
    p = ctypes.c_void_p(16)
    E = _lib
    assert _code("msa_route_scores", p, 0, 4, 8, 128, p, N, 10, p, 2, N, p, N, p, 1 << 20, N) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_scores", p, 1, 0, 8, 128, p, N, 10, p, 2, N, p, N, p, 1 << 20, N) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_scores", N, 1, 4, 8, 128, p, N, 10, p, 2, N, p, N, p, 1 << 20, N) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_scores", p, 1, 4, 8, 64, p, N, 10, p, 2, N, p, N, p, 1 << 20, N) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_route_scores", p, 1, 4, 3, 128, p, N, 10, p, 2, N, p, N, p, 1 << 20, N) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_route_scores", ctypes.c_void_p(18), 1, 4, 8, 128, p, N, 10, p, 2, N, p, N, p, 1 << 20, N) \
        == E.MSA_ERR_INVALID_ARG                                   # misaligned
    need = _lib.load().msa_route_workspace_bytes(2, 4, 8, 128, 1000, 10)
    assert need >= 2 * 1000 * 4
    assert _code("msa_route_scores", p, 2, 4, 8, 128, p, N, 1000, p, 10, N, p, N, p, need - 1, N) == E.MSA_ERR_WORKSPACE
    assert b"workspace" in _lib.load().msa_last_error()
    # misaligned stored norms
    assert _code("msa_route_scores", p, 2, 4, 8, 128, p, ctypes.c_void_p(20), 1000, p, 10, N, p, N, p, need, N) \
        == E.MSA_ERR_INVALID_ARG
    assert _code("msa_krbar_inv_norms", p, 10, 8, 96, p, N) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_krbar_inv_norms", N, 10, 8, 128, p, N) == E.MSA_ERR_INVALID_ARG


def test_topk_validation():
    p = ctypes.c_void_p(16)
    E = _lib
    ws = 1 << 20
    assert _code("msa_topk_docs", p, 1, 10, 0, p, p, p, ws, N) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_topk_docs", p, 1, 10, 11, p, p, p, ws, N) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_topk_docs", p, 1, 5000, 2000, p, p, p, ws, N) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_topk_docs", p, 1, 10, 4, p, p, p, 0, N) == E.MSA_ERR_WORKSPACE


def test_pool_and_attention_validation():
    p = ctypes.c_void_p(16)
    E = _lib
    assert _code("msa_pool_chunks", p, p, p, p, p, 4, 100, 4, 8, 96, 64, 1e6, p, p, p, N) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_pool_chunks", p, p, p, p, p, 4, 100, 4, 8, 128, 0, 1e6, p, p, p, N) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_pool_chunks", p, p, p, p, p, 4, 100, 4, 8, 128, 64, 1.0, p, p, p, N) == E.MSA_ERR_INVALID_ARG
    # attention: Tq > Tl, Hq % Hkv, D
    args = lambda B=1, Tq=4, Hq=32, D=128, Tl=4, Hkv=8: (p, B, Tq, Hq, D, p, p, Tl, Hkv, p, p, 2048, 8, p, 0, 1e6,
                                                         0.1, p, N)
    assert _code("msa_sparse_attn_decode", *args(Tq=5)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_sparse_attn_decode", *args(Hq=30)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_sparse_attn_decode", *args(D=64)) == E.MSA_ERR_UNSUPPORTED
    fw = lambda lse=p, **kw: (lambda a: a[:18] + (lse,) + a[18:])(args(**kw))      # + lse before the stream
    assert _code("msa_sparse_attn_forward", *fw(Tq=5)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_sparse_attn_forward", *fw(lse=ctypes.c_void_p((1 << 20) + 2))) == E.MSA_ERR_INVALID_ARG
    # split attention: the local partial and the memory pass validate like the one-launch call
    assert _code("msa_sparse_attn_local_partial", p, 1, 5, 32, 128, p, p, 4, 8, 0, 1e6, 0.1, p, p, N) == \
        E.MSA_ERR_INVALID_ARG                                                        # Tq > Tl
    assert _code("msa_sparse_attn_local_partial", p, 1, 4, 32, 64, p, p, 4, 8, 0, 1e6, 0.1, p, p, N) == \
        E.MSA_ERR_UNSUPPORTED                                                        # D
    assert _code("msa_sparse_attn_local_partial", p, 1, 4, 32, 128, p, p, 4, 8, 0, 1e6, 0.1, p,
                 ctypes.c_void_p((1 << 20) + 4), N) == E.MSA_ERR_INVALID_ARG          # part_ml alignment
    mm = lambda Tq=4, part_ml=p, O=p: (p, 1, Tq, 32, 128, 4, 8, p, p, 2048, 8, p, 0, 1e6, 0.1, p, part_ml, O, N, N)
    assert _code("msa_sparse_attn_memory_merge", *mm(Tq=5)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_sparse_attn_memory_merge", *mm(O=N)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_sparse_attn_memory_merge", *mm(part_ml=ctypes.c_void_p((1 << 20) + 4))) == E.MSA_ERR_INVALID_ARG


def test_encode_validation():
    p = ctypes.c_void_p(16)
    E = _lib
    need = _lib.load().msa_encode_workspace_bytes(100, 2560)
    assert need >= 2 * 100 * 2560 * 2
    args = lambda dm=2560, H=8, D=128, chunk=64, ws=p, wsb=need, hid=p, n_chunks=100: (
        hid, 6400, dm, p, H, D, p, p, 4, n_chunks, chunk, p, ws, wsb, N)
    assert _code("msa_encode_router_keys", *args(dm=2500)) == E.MSA_ERR_UNSUPPORTED          # not a multiple of 32
    assert _code("msa_encode_router_keys", *args(dm=16384)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_encode_router_keys", *args(D=64)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_encode_router_keys", *args(H=3)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_encode_router_keys", *args(chunk=0)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_encode_router_keys", *args(hid=N)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_encode_router_keys", *args(wsb=need - 1)) == E.MSA_ERR_WORKSPACE
    assert _code("msa_encode_router_keys", *args(ws=N)) == E.MSA_ERR_WORKSPACE
    assert _code("msa_encode_router_keys", *args(hid=ctypes.c_void_p(24))) == E.MSA_ERR_INVALID_ARG


def test_store_update_validation():
    E = _lib
    p = ctypes.c_void_p(1 << 20)
    q = ctypes.c_void_p(1 << 30)                      # far from p: no overlap for these sizes
    near = ctypes.c_void_p((1 << 20) + 2048)          # inside p's first rows
    need = _lib.load().msa_store_delete_workspace_bytes(10)
    assert need >= 16
    dl = lambda n_docs=10, n_chunks=100, H=8, D=128, kr=p, kro=q, nrm=N, nrmo=N, keep=p, ws=p, wsb=need: (
        kr, nrm, p, n_docs, n_chunks, H, D, keep, kro, nrmo, p, p, p, ws, wsb, N)
    assert _code("msa_store_delete", *dl(n_docs=0)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_store_delete", *dl(keep=N)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_store_delete", *dl(D=64)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_store_delete", *dl(H=5)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_store_delete", *dl(kro=near)) == E.MSA_ERR_INVALID_ARG          # output overlaps the store
    assert _code("msa_store_delete", *dl(nrm=p)) == E.MSA_ERR_INVALID_ARG             # norms without an output
    assert _code("msa_store_delete", *dl(wsb=need - 1)) == E.MSA_ERR_WORKSPACE
    assert _code("msa_store_delete", *dl(ws=N)) == E.MSA_ERR_WORKSPACE
    ap = lambda n_docs=10, n_chunks=100, nnd=2, nnc=5, cap=105, dcap=12, new=q: (
        p, N, p, n_docs, n_chunks, 8, 128, new, p, nnd, nnc, cap, dcap, N)
    assert _code("msa_store_append", *ap(cap=104)) == E.MSA_ERR_INVALID_ARG           # chunk capacity
    assert _code("msa_store_append", *ap(dcap=11)) == E.MSA_ERR_INVALID_ARG           # document capacity
    assert _code("msa_store_append", *ap(nnd=-1)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_store_append", *ap(new=ctypes.c_void_p((1 << 20) + 100 * 2048))) == E.MSA_ERR_INVALID_ARG


def test_route_backward_validation():
    E = _lib
    p = ctypes.c_void_p(1 << 20)
    need = _lib.load().msa_route_backward_workspace_bytes(2, 16, 8, 128, 40)
    assert need > 2 * 40 * 8 * 4 * 2                  # at least the two per-(query, document, head) weight arrays
    assert _lib.load().msa_route_backward_workspace_bytes(0, 16, 8, 128, 40) == 0
    bw = lambda B=2, T=16, H=8, D=128, n_chunks=300, n_docs=40, q=p, cs=p, dd=p, dq=p, dk=p, sel=p, ws=p, wsb=need: (
        q, B, T, H, D, p, N, n_chunks, p, n_docs, N, cs, dd, dq, dk, sel, ws, wsb, N)
    assert _code("msa_route_scores_backward", *bw(B=0)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_scores_backward", *bw(T=0)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_scores_backward", *bw(n_docs=0)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_scores_backward", *bw(cs=N)) == E.MSA_ERR_INVALID_ARG         # chunk scores required
    assert _code("msa_route_scores_backward", *bw(dd=N)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_scores_backward", *bw(sel=N)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_scores_backward", *bw(D=64)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_route_scores_backward", *bw(H=3)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_route_scores_backward", *bw(T=8193)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_route_scores_backward", *bw(B=70000)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_scores_backward", *bw(dq=ctypes.c_void_p((1 << 20) + 4))) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_scores_backward", *bw(wsb=need - 1)) == E.MSA_ERR_WORKSPACE
    assert _code("msa_route_scores_backward", *bw(ws=N)) == E.MSA_ERR_WORKSPACE


def test_attention_backward_validation():
    E = _lib
    p = ctypes.c_void_p(1 << 20)
    need = _lib.load().msa_sparse_attn_backward_workspace_bytes(1, 100, 32, 128, 130, 8, 45)
    # split Q and dO, row-major and transposed (8 arrays of [Hq, 128 padded rows, D] bf16)
    assert need >= 8 * 32 * 128 * 128 * 2
    assert _lib.load().msa_sparse_attn_backward_workspace_bytes(1, 100, 32, 128, 99, 8, 45) == 0   # Tl < Tq
    bw = lambda B=1, Tq=100, Hq=32, D=128, Tl=130, Hkv=8, Mmax=45, km=p, dO=p, dq=p, dkm=p, ws=p, wsb=need: (
        p, B, Tq, Hq, D, p, p, Tl, Hkv, km, p, 2 * Hkv * 128, Mmax, p, 7, 1e6, 0.088, dO, dq, p, p, dkm, p, ws, wsb, N)
    assert _code("msa_sparse_attn_backward", *bw(Tl=99)) == E.MSA_ERR_INVALID_ARG          # Tl < Tq
    assert _code("msa_sparse_attn_backward", *bw(Hq=30)) == E.MSA_ERR_INVALID_ARG          # Hq % Hkv
    assert _code("msa_sparse_attn_backward", *bw(D=64)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_sparse_attn_backward", *bw(Hkv=32, Hq=32)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_sparse_attn_backward", *bw(dO=N)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_sparse_attn_backward", *bw(dkm=N)) == E.MSA_ERR_INVALID_ARG          # memory gradient missing
    assert _code("msa_sparse_attn_backward", *bw(dq=ctypes.c_void_p((1 << 20) + 8))) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_sparse_attn_backward", *bw(wsb=need - 1)) == E.MSA_ERR_WORKSPACE
    assert _code("msa_sparse_attn_backward", *bw(ws=N)) == E.MSA_ERR_WORKSPACE
    # the saved-statistics variant: O and lse together or not at all, O 16-byte aligned, lse 4-byte
    sv = lambda O=p, lse=p, **kw: (lambda a: a[:18] + (O, lse) + a[18:])(bw(**kw))
    assert _code("msa_sparse_attn_backward_saved", *sv(O=N)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_sparse_attn_backward_saved", *sv(lse=N)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_sparse_attn_backward_saved", *sv(O=ctypes.c_void_p((1 << 20) + 4))) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_sparse_attn_backward_saved", *sv(lse=ctypes.c_void_p((1 << 20) + 2))) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_sparse_attn_backward_saved", *sv(Tl=99)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_sparse_attn_backward_saved", *sv(wsb=need - 1)) == E.MSA_ERR_WORKSPACE


def test_append_router_rows_validation():
    p = ctypes.c_void_p(16)
    E = _lib
    args = lambda B=1, T0=4, H=8, D=128, n_ids=2, T_out=20, qr=p: (qr, B, T0, H, D, p, p, 10, p, n_ids, T_out, p, N, N,
                                                                    N)
    assert _code("msa_append_router_rows", *args(T_out=3)) == E.MSA_ERR_INVALID_ARG      # T_out < T0
    assert _code("msa_append_router_rows", *args(D=64)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_append_router_rows", *args(B=0)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_append_router_rows", *args(qr=N)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_append_router_rows", *args(qr=ctypes.c_void_p(24))) == E.MSA_ERR_INVALID_ARG


def test_fetch_validation_host_side():
    import numpy as np
    top = np.array([[0, 5]], dtype=np.int32)                       # 5 is out of range
    off = np.array([0, 2, 3, 4], dtype=np.int64)
    ml = np.zeros(1, dtype=np.int32)
    p = ctypes.c_void_p(16)
    rc = _code("msa_fetch_docs", top.ctypes.data, 1, 2, p, off.ctypes.data, 3, 8, 128, p, 16, ml.ctypes.data, N, N)
    assert rc == _lib.MSA_ERR_INVALID_ARG
    top = np.array([[0, 2]], dtype=np.int32)                       # needs 3 entries > Mmax 2
    rc = _code("msa_fetch_docs", top.ctypes.data, 1, 2, p, off.ctypes.data, 3, 8, 128, p, 2, ml.ctypes.data, N, N)
    assert rc == _lib.MSA_ERR_INVALID_ARG


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load()


def test_route_topk_validation():
    E = _lib
    p = ctypes.c_void_p(1 << 20)
    lib = _lib.load()
    need = lib.msa_route_topk_workspace_bytes(1, 128, 8, 128, 1000, 100, 16)
    assert need >= lib.msa_topk_workspace_bytes(1, 100, 16) + 4 * 1000        # chunk maxima + group maxima
    assert lib.msa_route_topk_workspace_bytes(1, 128, 8, 128, 1000, 100, 33) == 0
    rt = lambda k=16, H=8, D=128, n_docs=100, ws=p, wsb=need, ti=p: (
        p, 1, 128, H, D, p, N, 1000, p, n_docs, N, k, p, N, ti, p, ws, wsb, N)
    assert _code("msa_route_topk", *rt(k=33)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_route_topk", *rt(k=0)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_route_topk", *rt(k=16, n_docs=10)) == E.MSA_ERR_INVALID_ARG        # k > n_docs
    assert _code("msa_route_topk", *rt(H=3)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_route_topk", *rt(ti=N)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_topk", *rt(wsb=need - 1)) == E.MSA_ERR_WORKSPACE
    assert _code("msa_route_topk", *rt(ws=N)) == E.MSA_ERR_WORKSPACE


def test_route_scan_select_clear_validation():
    E = _lib
    p = ctypes.c_void_p(1 << 20)
    lib = _lib.load()
    need_scan = lib.msa_route_workspace_bytes(2, 64, 8, 128, 1000, 1)
    sc = lambda B=2, T=64, H=8, D=128, q=p, ws=p, wsb=need_scan, nrm=N: (q, B, T, H, D, p, nrm, 1000, ws, wsb, N)
    assert _code("msa_route_scan", *sc(B=0)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_scan", *sc(q=N)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_scan", *sc(D=64)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_route_scan", *sc(H=16)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_route_scan", *sc(wsb=need_scan - 1)) == E.MSA_ERR_WORKSPACE
    assert _code("msa_route_scan", *sc(nrm=ctypes.c_void_p(20))) == E.MSA_ERR_INVALID_ARG
    need_sel = lib.msa_route_topk_workspace_bytes(2, 1, 1, 128, 1000, 100, 16)
    sl = lambda B=2, k=16, n_docs=100, off=p, ti=p, ws=p, wsb=need_sel: (
        B, 1000, off, n_docs, N, k, p, N, ti, p, ws, wsb, N)
    assert _code("msa_route_select", *sl(k=33)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_route_select", *sl(k=-1)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_route_select", *sl(k=16, n_docs=10)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_select", *sl(ti=N)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_select", *sl(off=N)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_select", *sl(B=0)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_select", *sl(wsb=need_sel - 1)) == E.MSA_ERR_WORKSPACE
    # k = 0 needs only the chunk maxima and no top-k outputs: a short workspace is enough
    assert _code("msa_route_select", *sl(k=0, ti=N, wsb=need_scan - 1)) == E.MSA_ERR_WORKSPACE
    assert _code("msa_route_workspace_clear", N, 256, N) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_workspace_clear", p, 255, N) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_workspace_clear", ctypes.c_void_p(20), 256, N) == E.MSA_ERR_INVALID_ARG


def test_route_topk_noalloc_validation():
    """Invalid arguments and sizes beyond the fixed scratch are rejected on the host, before any
    device call (so these run without a GPU)."""
    E = _lib
    p = ctypes.c_void_p(1 << 20)
    lib = _lib.load()
    cap = 16 << 20
    rt = lambda B=1, T=128, k=16, H=8, n_chunks=1000, n_docs=100, ti=p: (
        p, B, T, H, 128, p, N, n_chunks, p, n_docs, N, k, p, N, ti, p, N)
    assert _code("msa_route_topk_noalloc", *rt(k=33)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_route_topk_noalloc", *rt(H=3)) == E.MSA_ERR_UNSUPPORTED
    assert _code("msa_route_topk_noalloc", *rt(ti=N)) == E.MSA_ERR_INVALID_ARG
    assert _code("msa_route_topk_noalloc", *rt(k=16, n_docs=10)) == E.MSA_ERR_INVALID_ARG
    # the largest store that fits at batch 1, and one chunk more
    n_docs = 200_000
    gm = (n_docs + 63) // 64 * 8
    fit = (cap - gm) // 4 // 64 * 64
    assert lib.msa_route_topk_workspace_bytes(1, 128, 8, 128, fit, n_docs, 16) <= cap
    over = fit + 64 * 4
    assert lib.msa_route_topk_workspace_bytes(1, 128, 8, 128, over, n_docs, 16) > cap
    assert _code("msa_route_topk_noalloc", *rt(n_chunks=over, n_docs=n_docs)) == E.MSA_ERR_WORKSPACE
    assert b"scratch" in lib.msa_last_error()
    assert _code("msa_route_topk_noalloc", *rt(B=4, n_chunks=fit, n_docs=n_docs)) == E.MSA_ERR_WORKSPACE
