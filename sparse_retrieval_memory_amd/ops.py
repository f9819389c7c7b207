"""Torch-tensor wrappers with the C ABI's names (argument marshalling only).

Every step runs in libmsa's HIP kernels; PyTorch only provides device memory,
pinned host memory and streams.  bf16 tensors may be ``torch.bfloat16`` or
``int16``/``uint16`` views of the bits.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib

_ws_cache = {}


def _p(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _bf16(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.element_size() != 2 or t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must be a bf16 tensor (or its 16-bit bits), got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def workspace(nbytes: int, device, tag: str = "route") -> torch.Tensor:
    """A cached device scratch buffer of at least nbytes (one per device and tag),
    zero-filled when allocated (the routing calls need a zero workspace on their
    first use and hand it back zeroed).

    Calls on one stream reuse it in order; callers that run on several streams
    at once pass their own buffers instead."""
    key = (torch.device(device), tag)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max((int(nbytes) + 255) // 256 * 256, 256), dtype=torch.uint8, device=key[0])
        _ws_cache[key] = buf
    return buf


def route_workspace_clear(ws, stream=None):
    """msa_route_workspace_clear: zero a routing workspace with a kernel."""
    _lib.call("msa_route_workspace_clear", _p(ws), ws.numel() * ws.element_size() // 4 * 4, _stream(stream))


def pool_chunks(K, V, Kr, doc_tok_off, doc_chunk_off, n_chunks: int, chunk_len: int = 64,
                rope_base: float = 1.0e6, out: Optional[Tuple] = None, stream=None):
    """msa_pool_chunks: returns (Kbar, Vbar, Krbar) bf16 [n_chunks, H, D]."""
    for t, n in ((K, "K"), (V, "V"), (Kr, "Kr")):
        _bf16(t, n); _dev(t, n)
    n_tok, H, D = K.shape
    n_docs = doc_tok_off.numel() - 1
    if out is None:
        out = tuple(torch.empty((n_chunks, H, D), dtype=K.dtype, device=K.device) for _ in range(3))
    Kb, Vb, Rb = out
    _lib.call("msa_pool_chunks", _p(K), _p(V), _p(Kr), _p(doc_tok_off), _p(doc_chunk_off), n_docs, n_tok,
              n_chunks, H, D, chunk_len, float(rope_base), _p(Kb), _p(Vb), _p(Rb), _stream(stream))
    return Kb, Vb, Rb


def encode_workspace_bytes(n_chunks: int, d_model: int) -> int:
    return int(_lib.load().msa_encode_workspace_bytes(n_chunks, d_model))


def encode_router_keys(hidden, W, doc_tok_off, doc_chunk_off, n_chunks: int, H: int, chunk_len: int = 64,
                       out=None, ws=None, stream=None):
    """msa_encode_router_keys: Krbar bf16 [n_chunks, H, D] from hidden [n_tok, d_model] and W [H*D, d_model]."""
    _bf16(hidden, "hidden"); _bf16(W, "W"); _dev(hidden, "hidden"); _dev(W, "W")
    n_tok, dm = hidden.shape
    HD = W.shape[0]
    if W.shape[1] != dm or HD % H:
        raise ValueError(f"W must be [H*D, d_model], got {tuple(W.shape)} for d_model={dm}, H={H}")
    D = HD // H
    n_docs = doc_tok_off.numel() - 1
    if out is None:
        out = torch.empty((n_chunks, H, D), dtype=hidden.dtype, device=hidden.device)
    need = encode_workspace_bytes(n_chunks, dm)
    if ws is None:
        ws = workspace(need, hidden.device, "encode")
    _lib.call("msa_encode_router_keys", _p(hidden), n_tok, dm, _p(W), H, D, _p(doc_tok_off), _p(doc_chunk_off),
              n_docs, n_chunks, chunk_len, _p(out), _p(ws), ws.numel() * ws.element_size(), _stream(stream))
    return out


def store_delete(Krbar, doc_chunk_off, keep, inv_norm=None, out=None, stream=None):
    """msa_store_delete: (Krbar_out, inv_norm_out or None, doc_chunk_off_out, new_id, counts) with the deleted
    documents removed; the outputs are sized like the inputs, the first counts[1] rows / counts[0] + 1 offsets
    are the updated store (counts is a device int64 [2])."""
    _bf16(Krbar, "Krbar"); _dev(Krbar, "Krbar")
    n_chunks, H, D = Krbar.shape
    n_docs = doc_chunk_off.numel() - 1
    if keep.dtype != torch.uint8 or keep.numel() != n_docs:
        raise ValueError("keep must be uint8 [n_docs]")
    dev = Krbar.device
    if out is None:
        out = (torch.empty_like(Krbar), None if inv_norm is None else torch.empty_like(inv_norm),
               torch.empty_like(doc_chunk_off), torch.empty(n_docs, dtype=torch.int32, device=dev),
               torch.empty(2, dtype=torch.int64, device=dev))
    kr_o, nrm_o, off_o, ids, counts = out
    ws = workspace(int(_lib.load().msa_store_delete_workspace_bytes(n_docs)), dev, "store")
    _lib.call("msa_store_delete", _p(Krbar), _p(inv_norm), _p(doc_chunk_off), n_docs, n_chunks, H, D, _p(keep),
              _p(kr_o), _p(nrm_o), _p(off_o), _p(ids), _p(counts), _p(ws), ws.numel(), _stream(stream))
    return kr_o, nrm_o, off_o, ids, counts


def store_append(Krbar, doc_chunk_off, n_docs: int, n_chunks: int, new_Krbar, new_doc_chunk_off, inv_norm=None,
                 stream=None):
    """msa_store_append: append documents in place.  Krbar [capacity, H, D] and doc_chunk_off [doc_capacity + 1]
    hold n_docs documents / n_chunks chunks; returns the new (n_docs, n_chunks)."""
    _bf16(Krbar, "Krbar"); _bf16(new_Krbar, "new_Krbar"); _dev(Krbar, "Krbar")
    cap, H, D = Krbar.shape
    n_new_docs = new_doc_chunk_off.numel() - 1
    n_new_chunks = new_Krbar.shape[0]
    _lib.call("msa_store_append", _p(Krbar), _p(inv_norm), _p(doc_chunk_off), n_docs, n_chunks, H, D, _p(new_Krbar),
              _p(new_doc_chunk_off), n_new_docs, n_new_chunks, cap, doc_chunk_off.numel() - 1, _stream(stream))
    return n_docs + n_new_docs, n_chunks + n_new_chunks


def route_workspace_bytes(B, T, H, D, n_chunks, n_docs) -> int:
    return int(_lib.load().msa_route_workspace_bytes(B, T, H, D, n_chunks, n_docs))


def krbar_inv_norms(Krbar, out=None, stream=None):
    """msa_krbar_inv_norms: fp32 [n_chunks, H] reciprocal norms of a routing-key store."""
    _bf16(Krbar, "Krbar"); _dev(Krbar, "Krbar")
    n_chunks, H, D = Krbar.shape
    if out is None:
        out = torch.empty((n_chunks, H), dtype=torch.float32, device=Krbar.device)
    _lib.call("msa_krbar_inv_norms", _p(Krbar), n_chunks, H, D, _p(out), _stream(stream))
    return out


def route_scores(Qr, Krbar, doc_chunk_off, doc_exclude=None, want_chunk_scores: bool = False,
                 doc_scores=None, chunk_scores=None, ws=None, krbar_inv_norm=None, stream=None):
    """msa_route_scores: doc_scores fp32 [B, n_docs] (and chunk_scores [B, n_chunks])."""
    _bf16(Qr, "Qr"); _bf16(Krbar, "Krbar"); _dev(Qr, "Qr")
    B, T, H, D = Qr.shape
    n_chunks = Krbar.shape[0]
    n_docs = doc_chunk_off.numel() - 1
    dev = Qr.device
    if doc_scores is None:
        doc_scores = torch.empty((B, n_docs), dtype=torch.float32, device=dev)
    if want_chunk_scores and chunk_scores is None:
        chunk_scores = torch.empty((B, n_chunks), dtype=torch.float32, device=dev)
    need = route_workspace_bytes(B, T, H, D, n_chunks, n_docs)
    if ws is None:
        ws = workspace(need, dev)
    if doc_exclude is not None:
        assert doc_exclude.dtype in (torch.uint8, torch.bool) and doc_exclude.shape == (B, n_docs)
        doc_exclude = doc_exclude.contiguous()
    if krbar_inv_norm is not None:
        assert krbar_inv_norm.dtype == torch.float32 and krbar_inv_norm.shape == (n_chunks, H)
    _lib.call("msa_route_scores", _p(Qr), B, T, H, D, _p(Krbar), _p(krbar_inv_norm), n_chunks, _p(doc_chunk_off), n_docs,
              _p(doc_exclude), _p(doc_scores), _p(chunk_scores), _p(ws), ws.numel(), _stream(stream))
    if chunk_scores is not None:
        return doc_scores, chunk_scores
    return doc_scores


def route_topk_workspace_bytes(B, T, H, D, n_chunks, n_docs, k) -> int:
    return int(_lib.load().msa_route_topk_workspace_bytes(B, T, H, D, n_chunks, n_docs, k))


def route_topk(Qr, Krbar, doc_chunk_off, k: int, doc_exclude=None, krbar_inv_norm=None, doc_scores=None,
               top_idx=None, top_scores=None, ws=None, stream=None):
    """msa_route_topk: (doc_scores fp32 [B, n_docs], top_idx int32 [B, k], top_scores fp32 [B, k])."""
    _bf16(Qr, "Qr"); _bf16(Krbar, "Krbar"); _dev(Qr, "Qr")
    B, T, H, D = Qr.shape
    n_chunks = Krbar.shape[0]
    n_docs = doc_chunk_off.numel() - 1
    dev = Qr.device
    if doc_scores is None:
        doc_scores = torch.empty((B, n_docs), dtype=torch.float32, device=dev)
    if top_idx is None:
        top_idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    if top_scores is None:
        top_scores = torch.empty((B, k), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(route_topk_workspace_bytes(B, T, H, D, n_chunks, n_docs, k), dev, "route-topk")
    if doc_exclude is not None:
        assert doc_exclude.dtype in (torch.uint8, torch.bool) and doc_exclude.shape == (B, n_docs)
        doc_exclude = doc_exclude.contiguous()
    if krbar_inv_norm is not None:
        assert krbar_inv_norm.dtype == torch.float32 and krbar_inv_norm.shape == (n_chunks, H)
    _lib.call("msa_route_topk", _p(Qr), B, T, H, D, _p(Krbar), _p(krbar_inv_norm), n_chunks, _p(doc_chunk_off), n_docs,
              _p(doc_exclude), k, _p(doc_scores), None, _p(top_idx), _p(top_scores), _p(ws), ws.numel(),
              _stream(stream))
    return doc_scores, top_idx, top_scores


def route_topk_noalloc(Qr, Krbar, doc_chunk_off, k: int, doc_exclude=None, krbar_inv_norm=None, doc_scores=None,
                       top_idx=None, top_scores=None, stream=None):
    """msa_route_topk_noalloc: msa_route_topk with the library's fixed scratch array as workspace."""
    _bf16(Qr, "Qr"); _bf16(Krbar, "Krbar"); _dev(Qr, "Qr")
    B, T, H, D = Qr.shape
    n_chunks = Krbar.shape[0]
    n_docs = doc_chunk_off.numel() - 1
    dev = Qr.device
    if doc_scores is None:
        doc_scores = torch.empty((B, n_docs), dtype=torch.float32, device=dev)
    if top_idx is None:
        top_idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    if top_scores is None:
        top_scores = torch.empty((B, k), dtype=torch.float32, device=dev)
    if doc_exclude is not None:
        assert doc_exclude.dtype in (torch.uint8, torch.bool) and doc_exclude.shape == (B, n_docs)
        doc_exclude = doc_exclude.contiguous()
    _lib.call("msa_route_topk_noalloc", _p(Qr), B, T, H, D, _p(Krbar), _p(krbar_inv_norm), n_chunks,
              _p(doc_chunk_off), n_docs, _p(doc_exclude), k, _p(doc_scores), None, _p(top_idx), _p(top_scores),
              _stream(stream))
    return doc_scores, top_idx, top_scores


def route_scan(Qr, Krbar, ws, krbar_inv_norm=None, stream=None):
    """msa_route_scan: the scan only; the chunk maxima stay in ``ws`` for route_select."""
    _bf16(Qr, "Qr"); _bf16(Krbar, "Krbar"); _dev(Qr, "Qr")
    B, T, H, D = Qr.shape
    n_chunks = Krbar.shape[0]
    if krbar_inv_norm is not None:
        assert krbar_inv_norm.dtype == torch.float32 and krbar_inv_norm.shape == (n_chunks, H)
    _lib.call("msa_route_scan", _p(Qr), B, T, H, D, _p(Krbar), _p(krbar_inv_norm), n_chunks, _p(ws), ws.numel(),
              _stream(stream))


def route_select(B, n_chunks, doc_chunk_off, k: int, ws, doc_exclude=None, doc_scores=None, chunk_scores=None,
                 top_idx=None, top_scores=None, stream=None):
    """msa_route_select: document max (+ top-k for k >= 1) from the chunk maxima route_scan left in ``ws``.
    Returns doc_scores, or (doc_scores, top_idx, top_scores) for k >= 1."""
    n_docs = doc_chunk_off.numel() - 1
    dev = doc_chunk_off.device
    if doc_scores is None:
        doc_scores = torch.empty((B, n_docs), dtype=torch.float32, device=dev)
    if k > 0:
        if top_idx is None:
            top_idx = torch.empty((B, k), dtype=torch.int32, device=dev)
        if top_scores is None:
            top_scores = torch.empty((B, k), dtype=torch.float32, device=dev)
    if doc_exclude is not None:
        assert doc_exclude.dtype in (torch.uint8, torch.bool) and doc_exclude.shape == (B, n_docs)
        doc_exclude = doc_exclude.contiguous()
    _lib.call("msa_route_select", B, n_chunks, _p(doc_chunk_off), n_docs, _p(doc_exclude), k, _p(doc_scores),
              _p(chunk_scores), _p(top_idx), _p(top_scores), _p(ws), ws.numel(), _stream(stream))
    return (doc_scores, top_idx, top_scores) if k > 0 else doc_scores


def route_backward_workspace_bytes(B, T, H, D, n_docs) -> int:
    return int(_lib.load().msa_route_backward_workspace_bytes(B, T, H, D, n_docs))


def route_scores_backward(Qr, Krbar, doc_chunk_off, chunk_scores, d_doc_scores, doc_exclude=None,
                          krbar_inv_norm=None, dQr=None, dKsel=None, sel=None, ws=None, stream=None):
    """msa_route_scores_backward: (dQr fp32 [B, T, H, D], dKsel fp32 [B, n_docs, H, D], sel int32 [B, n_docs, 2])."""
    _bf16(Qr, "Qr"); _bf16(Krbar, "Krbar"); _dev(Qr, "Qr")
    B, T, H, D = Qr.shape
    n_chunks = Krbar.shape[0]
    n_docs = doc_chunk_off.numel() - 1
    dev = Qr.device
    assert chunk_scores.dtype == torch.float32 and chunk_scores.shape == (B, n_chunks) and chunk_scores.is_contiguous()
    assert d_doc_scores.dtype == torch.float32 and d_doc_scores.shape == (B, n_docs) and d_doc_scores.is_contiguous()
    if dQr is None:
        dQr = torch.empty((B, T, H, D), dtype=torch.float32, device=dev)
    if dKsel is None:
        dKsel = torch.empty((B, n_docs, H, D), dtype=torch.float32, device=dev)
    if sel is None:
        sel = torch.empty((B, n_docs, 2), dtype=torch.int32, device=dev)
    if doc_exclude is not None:
        assert doc_exclude.dtype in (torch.uint8, torch.bool) and doc_exclude.shape == (B, n_docs)
        doc_exclude = doc_exclude.contiguous()
    if krbar_inv_norm is not None:
        assert krbar_inv_norm.dtype == torch.float32 and krbar_inv_norm.shape == (n_chunks, H)
    need = route_backward_workspace_bytes(B, T, H, D, n_docs)
    if ws is None:
        ws = workspace(need, dev, "route_bwd")
    _lib.call("msa_route_scores_backward", _p(Qr), B, T, H, D, _p(Krbar), _p(krbar_inv_norm), n_chunks,
              _p(doc_chunk_off), n_docs, _p(doc_exclude), _p(chunk_scores), _p(d_doc_scores), _p(dQr), _p(dKsel),
              _p(sel), _p(ws), ws.numel(), _stream(stream))
    return dQr, dKsel, sel


def topk_workspace_bytes(B, n_docs, k) -> int:
    return int(_lib.load().msa_topk_workspace_bytes(B, n_docs, k))


def topk_docs(doc_scores, k: int, top_idx=None, top_scores=None, ws=None, stream=None):
    """msa_topk_docs: (top_idx int32 [B, k], top_scores fp32 [B, k])."""
    _dev(doc_scores, "doc_scores")
    assert doc_scores.dtype == torch.float32 and doc_scores.is_contiguous()
    B, n_docs = doc_scores.shape
    dev = doc_scores.device
    if top_idx is None:
        top_idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    if top_scores is None:
        top_scores = torch.empty((B, k), dtype=torch.float32, device=dev)
    need = topk_workspace_bytes(B, n_docs, k)
    if ws is None:
        ws = workspace(need, dev, "topk")
    _lib.call("msa_topk_docs", _p(doc_scores), B, n_docs, k, _p(top_idx), _p(top_scores), _p(ws), ws.numel(),
              _stream(stream))
    return top_idx, top_scores


def fetch_docs(top_idx_host, host_store, doc_chunk_off_host, staging, Mmax: int, side_stream=None,
               done_event=None) -> torch.Tensor:
    """msa_fetch_docs: host-driven copies of the selected docs into staging; returns mem_len (host int32)."""
    assert top_idx_host.device.type == "cpu" and top_idx_host.dtype == torch.int32
    assert doc_chunk_off_host.device.type == "cpu" and doc_chunk_off_host.dtype == torch.int64
    top_idx_host = top_idx_host.contiguous()
    B, k = top_idx_host.shape
    n_docs = doc_chunk_off_host.numel() - 1
    H, D = host_store.shape[-2], host_store.shape[-1]
    mem_len = torch.empty(B, dtype=torch.int32)
    side = side_stream if side_stream is not None else torch.cuda.current_stream()
    if done_event is not None and not done_event.cuda_event:
        # torch creates the underlying event on its first record: create it here so the
        # library can record it after the copies (an absent event would order nothing)
        done_event.record(side)
    ev = ctypes.c_void_p(0 if done_event is None else done_event.cuda_event)
    _lib.call("msa_fetch_docs", _p(top_idx_host), B, k, _p(host_store), _p(doc_chunk_off_host), n_docs, H, D,
              _p(staging), Mmax, _p(mem_len), ctypes.c_void_p(side.cuda_stream), ev)
    return mem_len


def gather_docs(top_idx, host_store, doc_chunk_off, staging, Mmax: int, mem_len=None, stream=None):
    """msa_gather_docs: device-side assembly; returns mem_len (device int32 [B])."""
    B, k = top_idx.shape
    n_docs = doc_chunk_off.numel() - 1
    H, D = host_store.shape[-2], host_store.shape[-1]
    if mem_len is None:
        mem_len = torch.empty(B, dtype=torch.int32, device=top_idx.device)
    _lib.call("msa_gather_docs", _p(top_idx), B, k, _p(host_store), _p(doc_chunk_off), n_docs, H, D,
              _p(staging), Mmax, _p(mem_len), _stream(stream))
    return mem_len


def append_router_rows(Qr, Krbar, doc_chunk_off, ids, T_out: int, rows=None, n_rows=None, doc_exclude=None,
                       stream=None):
    """msa_append_router_rows: the next interleave round's router rows bf16 [B, T_out, H, D].

    Also marks ``ids`` in ``doc_exclude`` (uint8 [B, n_docs]) when given; returns (rows, n_rows)."""
    _bf16(Qr, "Qr"); _bf16(Krbar, "Krbar"); _dev(Qr, "Qr")
    B, T0, H, D = Qr.shape
    n_docs = doc_chunk_off.numel() - 1
    assert ids.dtype == torch.int32 and ids.is_cuda and ids.shape[0] == B
    ids = ids.contiguous()
    if rows is None:
        rows = torch.empty((B, T_out, H, D), dtype=Qr.dtype, device=Qr.device)
    if n_rows is None:
        n_rows = torch.empty(B, dtype=torch.int32, device=Qr.device)
    if doc_exclude is not None:
        assert doc_exclude.dtype == torch.uint8 and doc_exclude.shape == (B, n_docs) and doc_exclude.is_contiguous()
    _lib.call("msa_append_router_rows", _p(Qr), B, T0, H, D, _p(Krbar), _p(doc_chunk_off), n_docs, _p(ids),
              ids.shape[1], T_out, _p(rows), _p(n_rows), _p(doc_exclude), _stream(stream))
    return rows, n_rows


def sparse_attn_decode(Q, Kloc, Vloc, Kmem, Vmem, mem_entry_stride: int, Mmax: int, mem_len,
                       rope_offset: int, rope_base: float = 1.0e6, scale: Optional[float] = None,
                       out=None, stream=None):
    """msa_sparse_attn_decode: O fp32 [B, Tq, Hq, D]."""
    _bf16(Q, "Q"); _bf16(Kloc, "Kloc"); _bf16(Vloc, "Vloc")
    B, Tq, Hq, D = Q.shape
    _, Tl, Hkv, _ = Kloc.shape
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty((B, Tq, Hq, D), dtype=torch.float32, device=Q.device)
    kp = Kmem.data_ptr() if Kmem is not None else 0
    vp = Vmem.data_ptr() if Vmem is not None else 0
    _lib.call("msa_sparse_attn_decode", _p(Q), B, Tq, Hq, D, _p(Kloc), _p(Vloc), Tl, Hkv, ctypes.c_void_p(kp),
              ctypes.c_void_p(vp), mem_entry_stride, Mmax, _p(mem_len), rope_offset, float(rope_base),
              float(scale), _p(out), _stream(stream))
    return out


def sparse_attn_forward(Q, Kloc, Vloc, Kmem, Vmem, mem_entry_stride: int, Mmax: int, mem_len,
                        rope_offset: int, rope_base: float = 1.0e6, scale: Optional[float] = None,
                        out=None, lse=None, stream=None):
    """msa_sparse_attn_forward: (O fp32 [B, Tq, Hq, D], lse fp32 [B, Tq, Hq], natural log)."""
    _bf16(Q, "Q"); _bf16(Kloc, "Kloc"); _bf16(Vloc, "Vloc")
    B, Tq, Hq, D = Q.shape
    _, Tl, Hkv, _ = Kloc.shape
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty((B, Tq, Hq, D), dtype=torch.float32, device=Q.device)
    if lse is None:
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=Q.device)
    assert lse.dtype == torch.float32 and lse.shape == (B, Tq, Hq) and lse.is_contiguous()
    kp = Kmem.data_ptr() if Kmem is not None else 0
    vp = Vmem.data_ptr() if Vmem is not None else 0
    _lib.call("msa_sparse_attn_forward", _p(Q), B, Tq, Hq, D, _p(Kloc), _p(Vloc), Tl, Hkv, ctypes.c_void_p(kp),
              ctypes.c_void_p(vp), mem_entry_stride, Mmax, _p(mem_len), rope_offset, float(rope_base),
              float(scale), _p(out), _p(lse), _stream(stream))
    return out, lse


def sparse_attn_local_partial(Q, Kloc, Vloc, rope_offset: int, rope_base: float = 1.0e6,
                              scale: Optional[float] = None, part=None, stream=None):
    """msa_sparse_attn_local_partial: the local-key half of the attention; returns
    part = (part_O fp32 [B, Tq, Hq, D], part_ml fp32 [B, Tq, Hq, 2])."""
    _bf16(Q, "Q"); _bf16(Kloc, "Kloc"); _bf16(Vloc, "Vloc")
    B, Tq, Hq, D = Q.shape
    _, Tl, Hkv, _ = Kloc.shape
    if scale is None:
        scale = D ** -0.5
    if part is None:
        part = (torch.empty((B, Tq, Hq, D), dtype=torch.float32, device=Q.device),
                torch.empty((B, Tq, Hq, 2), dtype=torch.float32, device=Q.device))
    _lib.call("msa_sparse_attn_local_partial", _p(Q), B, Tq, Hq, D, _p(Kloc), _p(Vloc), Tl, Hkv, rope_offset,
              float(rope_base), float(scale), _p(part[0]), _p(part[1]), _stream(stream))
    return part


def sparse_attn_memory_merge(Q, Tl: int, Hkv: int, Kmem, Vmem, mem_entry_stride: int, Mmax: int, mem_len,
                             rope_offset: int, part, rope_base: float = 1.0e6, scale: Optional[float] = None,
                             out=None, lse=None, stream=None):
    """msa_sparse_attn_memory_merge: the memory half merged with ``part``; O fp32 [B, Tq, Hq, D]
    (and the log-sum-exp into ``lse`` when given)."""
    _bf16(Q, "Q")
    B, Tq, Hq, D = Q.shape
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty((B, Tq, Hq, D), dtype=torch.float32, device=Q.device)
    kp = Kmem.data_ptr() if Kmem is not None else 0
    vp = Vmem.data_ptr() if Vmem is not None else 0
    _lib.call("msa_sparse_attn_memory_merge", _p(Q), B, Tq, Hq, D, Tl, Hkv, ctypes.c_void_p(kp), ctypes.c_void_p(vp),
              mem_entry_stride, Mmax, _p(mem_len), rope_offset, float(rope_base), float(scale), _p(part[0]),
              _p(part[1]), _p(out), ctypes.c_void_p(lse.data_ptr() if lse is not None else 0), _stream(stream))
    return out


def attn_backward_workspace_bytes(B, Tq, Hq, D, Tl, Hkv, Mmax) -> int:
    return int(_lib.load().msa_sparse_attn_backward_workspace_bytes(B, Tq, Hq, D, Tl, Hkv, Mmax))


def sparse_attn_backward(Q, Kloc, Vloc, Kmem, Vmem, mem_entry_stride: int, Mmax: int, mem_len, rope_offset: int,
                         dO, rope_base: float = 1.0e6, scale: Optional[float] = None, out=None, ws=None,
                         stream=None, O=None, lse=None):
    """msa_sparse_attn_backward: (dQ [B, Tq, Hq, D], dKloc, dVloc [B, Tl, Hkv, D], dKmem, dVmem [B, Mmax, Hkv, D]),
    all fp32.  With the forward's output O and log-sum-exp lse (sparse_attn_forward), calls
    msa_sparse_attn_backward_saved, which reuses them instead of recomputing the softmax statistics."""
    _bf16(Q, "Q"); _bf16(Kloc, "Kloc"); _bf16(Vloc, "Vloc")
    B, Tq, Hq, D = Q.shape
    _, Tl, Hkv, _ = Kloc.shape
    assert dO.dtype == torch.float32 and dO.shape == (B, Tq, Hq, D) and dO.is_contiguous()
    if scale is None:
        scale = D ** -0.5
    dev = Q.device
    if out is None:
        f = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)
        out = (f(B, Tq, Hq, D), f(B, Tl, Hkv, D), f(B, Tl, Hkv, D), f(B, max(Mmax, 1), Hkv, D),
               f(B, max(Mmax, 1), Hkv, D))
    need = attn_backward_workspace_bytes(B, Tq, Hq, D, Tl, Hkv, Mmax)
    if ws is None:
        ws = workspace(need, dev, "attn_bwd")
    kp = Kmem.data_ptr() if Kmem is not None else 0
    vp = Vmem.data_ptr() if Vmem is not None else 0
    if O is None and lse is None:
        _lib.call("msa_sparse_attn_backward", _p(Q), B, Tq, Hq, D, _p(Kloc), _p(Vloc), Tl, Hkv,
                  ctypes.c_void_p(kp), ctypes.c_void_p(vp), mem_entry_stride, Mmax, _p(mem_len), rope_offset,
                  float(rope_base), float(scale), _p(dO), _p(out[0]), _p(out[1]), _p(out[2]), _p(out[3]),
                  _p(out[4]), _p(ws), ws.numel(), _stream(stream))
        return out
    assert O is not None and lse is not None, "O and lse are given together"
    assert O.dtype == torch.float32 and O.shape == (B, Tq, Hq, D) and O.is_contiguous()
    assert lse.dtype == torch.float32 and lse.shape == (B, Tq, Hq) and lse.is_contiguous()
    _lib.call("msa_sparse_attn_backward_saved", _p(Q), B, Tq, Hq, D, _p(Kloc), _p(Vloc), Tl, Hkv,
              ctypes.c_void_p(kp), ctypes.c_void_p(vp), mem_entry_stride, Mmax, _p(mem_len), rope_offset,
              float(rope_base), float(scale), _p(dO), _p(O), _p(lse), _p(out[0]), _p(out[1]), _p(out[2]),
              _p(out[3]), _p(out[4]), _p(ws), ws.numel(), _stream(stream))
    return out
