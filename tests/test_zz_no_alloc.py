"""msa_route_topk_noalloc (the routing + top-k call with its workspace in a fixed array inside the
library) through the C ABI, against msa_route_topk with a caller workspace: two calls in a row, the
second with a smaller store, batch and k, and a third at the 100M-token layer's full size."""

import ctypes
import sys

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O
from sparse_retrieval_memory_amd import _lib, ops
from synth import splitmix as sm
from synth import workloads as C
from synth import native
from tests.parity import SCORE_TOL, check_topk, dev_bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def announce(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _case(B, T, n_docs, seed, H=8):
    r = np.random.default_rng(seed)
    lens = r.integers(1, 9, n_docs)
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    G = int(off[-1])
    Qr = sm.normal_bf16(seed, sm.TID_QR, 0, 0, B * T * H * 128).reshape(B, T, H, 128)
    Kr = sm.normal_bf16(seed, sm.TID_KRBAR, 0, 0, G * H * 128).reshape(G, H, 128)
    excl = (r.random((B, n_docs)) < 0.03).astype(np.uint8)
    return Qr, Kr, off, excl


def _noalloc(q, kr, offd, k, ex=None, nrm=None):
    B, T, H, D = q.shape
    G, n_docs = kr.shape[0], offd.numel() - 1
    doc = torch.empty((B, n_docs), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, k), dtype=torch.int32, device=DEV)
    sc = torch.empty((B, k), dtype=torch.float32, device=DEV)
    p = lambda t: ctypes.c_void_p(0 if t is None else t.data_ptr())
    _lib.call("msa_route_topk_noalloc", p(q), B, T, H, D, p(kr), p(nrm), G, p(offd), n_docs, p(ex), k, p(doc), None,
              p(idx), p(sc), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return doc, idx, sc


def _same(a, b):
    for x, y in zip(a, b):
        assert np.array_equal(x.cpu().numpy().view(np.uint32), y.cpu().numpy().view(np.uint32))


def test_noalloc_matches_route_topk_two_calls():
    for i, (B, T, n_docs, k, stored) in enumerate([(3, 100, 4000, 16, True), (1, 20, 700, 4, False)]):
        announce("noalloc", i, B, T, n_docs, k)
        Qr, Kr, off, excl = _case(B, T, n_docs, seed=900 + i)
        q, kr, offd = dev_bits(Qr), dev_bits(Kr), torch.from_numpy(off).to(DEV)
        ex = torch.from_numpy(excl).to(DEV)
        nrm = ops.krbar_inv_norms(kr) if stored else None
        got = _noalloc(q, kr, offd, k, ex, nrm)
        ref = ops.route_topk(q, kr, offd, k, doc_exclude=ex, krbar_inv_norm=nrm)
        torch.cuda.synchronize()
        _same(got, ref)
        _, ref_doc = O.route(O.bf16_to_f64(Qr), O.bf16_to_f64(Kr), off, excl.astype(bool))
        fin = np.isfinite(ref_doc)
        assert np.abs(got[0].cpu().numpy()[fin] - ref_doc[fin]).max() <= SCORE_TOL
        for b in range(B):
            check_topk(got[1].cpu().numpy()[b], ref_doc[b], k)


def test_noalloc_100M_layer_then_small():
    """A full 100M-token routing layer (1.66M chunks, 6.7 MB of scratch), then a small call."""
    w = C.workload("100M-18layer")
    announce("noalloc 100M layer")
    kr = torch.empty((w.n_chunks, w.H, w.D), dtype=torch.int16, device=DEV)
    native.fill_normal_bf16_device(kr, w.seed, sm.TID_KRBAR, 2, 0)
    for g, row in C.pooled_plants(w, 2).items():
        kr[g].copy_(dev_bits(row))
    q = dev_bits(C.queries(w, 2)["Qr"])
    offd = torch.from_numpy(w.doc_chunk_off).to(DEV)
    nrm = ops.krbar_inv_norms(kr)
    got = _noalloc(q, kr, offd, w.k, None, nrm)
    ref = ops.route_topk(q, kr, offd, w.k, krbar_inv_norm=nrm)
    torch.cuda.synchronize()
    _same(got, ref)
    assert set(d for _, d in C.planted_docs(w, 2)) <= set(got[1].cpu().numpy()[0].tolist())
    del kr, nrm
    Qr, Kr, off, excl = _case(2, 33, 300, seed=950)
    q, kr, offd = dev_bits(Qr), dev_bits(Kr), torch.from_numpy(off).to(DEV)
    got = _noalloc(q, kr, offd, 8)
    ref = ops.route_topk(q, kr, offd, 8)
    torch.cuda.synchronize()
    _same(got, ref)
