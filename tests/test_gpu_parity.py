"""GPU parity: every kernel through the C ABI against the fp64 oracle, on the
same seeded inputs, at sizes that span several tiles and a ragged tail, plus
the edge cases (1-chunk documents, k = 1, k = n_docs, single query token,
empty memory).  Rules P1-P4 are in tests/parity.py."""

import sys

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O
from sparse_retrieval_memory_amd import ops
from synth import workloads as C
from synth import native
from synth import splitmix as sm

from tests.parity import (ATT_GRAD_OBS, ATT_TOL, SCORE_TOL, bf16_ulp_diff, check_topk, dev_bits, encoded_keys_ok, grads_ok,
                          host_bits, pooled_k_ok, pooled_k_scales, rel_rows, route_grad_bounds, route_near_ties)

# lse of the GPU forward against the oracle: scores carry ~2^-16 of sum_d |q_d k_d| * scale
# (about 1e-4 for N(0,1) rows at D = 128), so the log-sum-exp is within 1e-3 absolute
LSE_TOL = 1e-3

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def announce(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def f64(bits):
    return O.bf16_to_f64(bits)


# ------------------------------------------------------------------ generator
def test_device_generator_matches_host():
    for (seed, tid, layer, start, n) in [(1, 3, 0, 0, 4096), (7, 11, 5, 12345, 100003), (2, 9, 17, 2**33 + 5, 777)]:
        announce("fill", seed, tid, layer, start, n)
        out = torch.empty(n, dtype=torch.int16, device=DEV)
        native.fill_normal_bf16_device(out, seed, tid, layer, start)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), sm.normal_bf16(seed, tid, layer, start, n))


# -------------------------------------------------------------------- routing
def _route_case(B, T, H, n_docs, seed, lens=None):
    r = np.random.default_rng(seed)
    if lens is None:
        lens = r.integers(1, 7, n_docs)                  # chunks per document, includes 1-chunk docs
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    G = int(off[-1])
    Qr = sm.normal_bf16(seed, sm.TID_QR, 0, 0, B * T * H * 128).reshape(B, T, H, 128)
    Kr = sm.normal_bf16(seed, sm.TID_KRBAR, 0, 0, G * H * 128).reshape(G, H, 128)
    return Qr, Kr, off


def _run_route(Qr, Kr, off, exclude=None, stored_norms=False):
    kr = dev_bits(Kr)
    nrm = ops.krbar_inv_norms(kr) if stored_norms else None
    doc, ch = ops.route_scores(dev_bits(Qr), kr, torch.from_numpy(off).to(DEV),
                               None if exclude is None else torch.from_numpy(exclude.astype(np.uint8)).to(DEV),
                               want_chunk_scores=True, krbar_inv_norm=nrm)
    torch.cuda.synchronize()
    return doc.cpu().numpy().astype(np.float64), ch.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("B,T,H", [(1, 1, 8), (1, 2, 8), (1, 7, 8), (1, 15, 8), (3, 5, 8), (2, 3, 4), (1, 9, 1),
                                   (1, 16, 8), (1, 17, 8), (1, 32, 8), (1, 33, 8), (1, 64, 8), (1, 100, 8),
                                   (1, 128, 8), (1, 130, 8), (2, 64, 8), (5, 40, 8), (3, 20, 2), (1, 48, 4),
                                   (1, 260, 8)])
def test_route_scores_match_oracle(B, T, H):
    announce("route", B, T, H)
    Qr, Kr, off = _route_case(B, T, H, n_docs=337, seed=100 + B * 1000 + T * 10 + H)
    doc, ch = _run_route(Qr, Kr, off)
    ref_ch, ref_doc = O.route(f64(Qr), f64(Kr), off)
    assert np.abs(ch - ref_ch).max() <= SCORE_TOL
    assert np.abs(doc - ref_doc).max() <= SCORE_TOL


@pytest.mark.parametrize("B,T,H", [(1, 128, 8), (1, 16, 8), (1, 130, 8), (2, 64, 8), (5, 40, 4), (1, 260, 8),
                                   (16, 64, 8), (1, 3, 8)])
def test_route_with_stored_norms_matches_oracle(B, T, H):
    announce("route-stored-norms", B, T, H)
    Qr, Kr, off = _route_case(B, T, H, n_docs=401, seed=7 + B * 100 + T + H)
    doc, ch = _run_route(Qr, Kr, off, stored_norms=True)
    ref_ch, ref_doc = O.route(f64(Qr), f64(Kr), off)
    assert np.abs(ch - ref_ch).max() <= SCORE_TOL
    assert np.abs(doc - ref_doc).max() <= SCORE_TOL


def test_krbar_inv_norms_match_oracle():
    Qr, Kr, off = _route_case(1, 1, 8, n_docs=200, seed=3)
    Kr = Kr.copy()
    Kr[5, 3] = 0
    announce("krbar-norms")
    n = ops.krbar_inv_norms(dev_bits(Kr)).cpu().numpy().astype(np.float64)
    ref_n = np.linalg.norm(f64(Kr), axis=-1)
    ref = np.divide(1.0, ref_n, out=np.zeros_like(ref_n), where=ref_n > 0)
    assert n[5, 3] == 0.0
    assert np.abs(n - ref).max() <= 1e-6 * np.abs(ref).max()


def test_route_exclusion_and_zero_vectors():
    Qr, Kr, off = _route_case(2, 40, 8, n_docs=97, seed=5)
    Kr = Kr.copy(); Qr = Qr.copy()
    Kr[3, 2] = 0                       # zero head in a chunk -> cosine 0 for that head
    Qr[1, 7, 5] = 0                    # zero query head
    excl = np.zeros((2, 97), bool); excl[0, [1, 50]] = True; excl[1, 96] = True
    announce("route-exclude")
    ref_ch, ref_doc = O.route(f64(Qr), f64(Kr), off, excl)
    for stored in (False, True):
        doc, ch = _run_route(Qr, Kr, off, excl, stored_norms=stored)
        assert np.all(doc[excl] == -np.inf)
        assert np.abs(doc[~excl] - ref_doc[~excl]).max() <= SCORE_TOL
        assert np.abs(ch - ref_ch).max() <= SCORE_TOL


def test_route_few_rows_exclusion():
    Qr, Kr, off = _route_case(1, 3, 8, n_docs=50, seed=6)
    excl = np.zeros((1, 50), bool); excl[0, ::7] = True
    announce("route-few-rows-exclude")
    doc, _ = _run_route(Qr, Kr, off, excl)
    _, ref_doc = O.route(f64(Qr), f64(Kr), off, excl)
    assert np.all(doc[excl] == -np.inf)
    assert np.abs(doc[~excl] - ref_doc[~excl]).max() <= SCORE_TOL


def test_route_deterministic():
    Qr, Kr, off = _route_case(1, 128, 8, n_docs=3000, seed=8)
    announce("route-determinism")
    for stored in (False, True):
        a, _ = _run_route(Qr, Kr, off, stored_norms=stored)
        b, _ = _run_route(Qr, Kr, off, stored_norms=stored)
        assert np.array_equal(a.view(np.uint64), b.view(np.uint64))


def test_route_empty_documents_match_oracle():
    """Documents without chunks (leading, several in a row, in the middle, trailing) score -inf and
    the others keep their own chunks' maximum: msa_route_scores (with and without stored norms),
    msa_route_topk and msa_route_scan + msa_route_select against the oracle, with exclusions."""
    r = np.random.default_rng(41)
    lens = r.integers(1, 5, 300)
    lens[[0, 7, 8, 9, 150, 297, 298, 299]] = 0
    B = 2
    Qr, Kr, off = _route_case(B, 40, 8, 300, seed=41, lens=lens)
    excl = np.zeros((B, 300), bool); excl[0, [3, 8, 200]] = True
    empty = lens == 0
    announce("route-empty-docs")
    ref_ch, ref_doc = O.route(f64(Qr), f64(Kr), off, excl)
    assert np.all(ref_doc[:, empty] == -np.inf)
    fin = np.isfinite(ref_doc)
    for stored in (False, True):
        doc, ch = _run_route(Qr, Kr, off, excl, stored_norms=stored)
        assert np.array_equal(np.isfinite(doc), fin)
        assert np.abs(doc[fin] - ref_doc[fin]).max() <= SCORE_TOL
        assert np.abs(ch - ref_ch).max() <= SCORE_TOL
    q, kr, offd = dev_bits(Qr), dev_bits(Kr), torch.from_numpy(off).to(DEV)
    ex = torch.from_numpy(excl.astype(np.uint8)).to(DEV)
    k = 16
    d1, i1, s1 = ops.route_topk(q, kr, offd, k, doc_exclude=ex)
    ws = ops.workspace(ops.route_topk_workspace_bytes(B, 40, 8, 128, len(Kr), 300, k), DEV, "test-empty")
    ops.route_scan(q, kr, ws)
    d2, i2, s2 = ops.route_select(B, len(Kr), offd, k, ws, doc_exclude=ex)
    torch.cuda.synchronize()
    assert np.array_equal(d1.cpu().numpy().view(np.uint32), d2.cpu().numpy().view(np.uint32))
    assert np.array_equal(i1.cpu().numpy(), i2.cpu().numpy())
    gi = i1.cpu().numpy()
    for b in range(B):
        check_topk(gi[b], ref_doc[b], k)
        assert not np.any(empty[gi[b]]) and not np.any(excl[b, gi[b]])
    # more documents requested than have chunks: the rest are -inf documents, lowest ids first
    lens2 = np.array([0, 2, 0, 1, 0, 0, 3, 0])
    Qr2, Kr2, off2 = _route_case(1, 5, 8, 8, seed=42, lens=lens2)
    _, ref2 = O.route(f64(Qr2), f64(Kr2), off2)
    _, i3, s3 = ops.route_topk(dev_bits(Qr2), dev_bits(Kr2), torch.from_numpy(off2).to(DEV), 6)
    ridx, rsc = O.topk(ref2, 6)
    assert list(i3.cpu().numpy()[0]) == list(ridx[0])
    assert np.all(s3.cpu().numpy()[0][3:] == -np.inf)


def test_route_long_documents_match_oracle():
    """Groups of 64 documents whose chunk ranges span more than one pass of the document-max
    workgroup (a 1,500-chunk document, several of 300-700 chunks, single-chunk and empty ones):
    document scores, chunk scores and top-k against the oracle, and the workspace handed back zeroed."""
    r = np.random.default_rng(43)
    n_docs = 200
    lens = r.integers(0, 3, n_docs)
    lens[[5, 70, 71, 140]] = [1500, 700, 333, 513]
    lens[[64, 65, 127, 199]] = 0
    B, T, k = 2, 48, 8
    Qr, Kr, off = _route_case(B, T, 8, n_docs, seed=43, lens=lens)
    announce("route-long-docs", int(lens.sum()))
    ref_ch, ref_doc = O.route(f64(Qr), f64(Kr), off)
    fin = np.isfinite(ref_doc)
    q, kr, offd = dev_bits(Qr), dev_bits(Kr), torch.from_numpy(off).to(DEV)
    ws = torch.zeros(ops.route_topk_workspace_bytes(B, T, 8, 128, len(Kr), n_docs, k), dtype=torch.uint8, device=DEV)
    ops.route_scan(q, kr, ws)
    ch = torch.empty((B, len(Kr)), dtype=torch.float32, device=DEV)
    doc, idx, _ = ops.route_select(B, len(Kr), offd, k, ws, chunk_scores=ch)
    torch.cuda.synchronize()
    doc = doc.cpu().numpy()
    assert np.array_equal(np.isfinite(doc), fin)
    assert np.abs(doc[fin] - ref_doc[fin]).max() <= SCORE_TOL
    assert np.abs(ch.cpu().numpy() - ref_ch).max() <= SCORE_TOL
    for bb in range(B):
        check_topk(idx.cpu().numpy()[bb], ref_doc[bb], k)
    assert int(ws.count_nonzero().item()) == 0


def test_route_workspace_reuse_across_sizes():
    """One routing workspace reused by calls of different sizes (batch, chunks, documents, k) in a
    row, without clearing: every call's outputs are bit-identical to the same call on a fresh
    zero workspace (each call hands the workspace back zeroed)."""
    cases = [(2, 40, 3000, 16), (1, 128, 400, 4), (3, 20, 1200, 8), (1, 7, 5000, 32), (2, 64, 50, 1)]
    max_bytes = max(ops.route_topk_workspace_bytes(B, T, 8, 128, 4 * n, n, k) for B, T, n, k in cases)
    shared = torch.zeros(max_bytes, dtype=torch.uint8, device=DEV)
    for i, (B, T, n_docs, k) in enumerate(cases):
        announce("route-workspace-reuse", B, T, n_docs, k)
        Qr, Kr, off = _route_case(B, T, 8, n_docs, seed=500 + i)
        q, kr, offd = dev_bits(Qr), dev_bits(Kr), torch.from_numpy(off).to(DEV)
        nrm = ops.krbar_inv_norms(kr)
        fresh = torch.zeros_like(shared)
        a = ops.route_topk(q, kr, offd, k, krbar_inv_norm=nrm, ws=shared)
        b = ops.route_topk(q, kr, offd, k, krbar_inv_norm=nrm, ws=fresh)
        c = ops.route_scores(q, kr, offd, krbar_inv_norm=nrm, ws=shared)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y)
        assert torch.equal(a[0], c)
        assert int(shared.count_nonzero().item()) == 0 and int(fresh.count_nonzero().item()) == 0
        _, ref_doc = O.route(f64(Qr), f64(Kr), off)
        assert np.abs(c.cpu().numpy() - ref_doc).max() <= SCORE_TOL
        for bb in range(B):
            check_topk(a[1].cpu().numpy()[bb], ref_doc[bb], k)


def test_route_scan_select_equal_one_call():
    """msa_route_scan + msa_route_select(k) == msa_route_topk and scan + select(0) == msa_route_scores,
    bit for bit (scores, chunk scores, ids), over a multi-row-block batch with exclusions."""
    B, T, n_docs, k = 4, 96, 2500, 16
    Qr, Kr, off = _route_case(B, T, 8, n_docs, seed=77)
    q, kr, offd = dev_bits(Qr), dev_bits(Kr), torch.from_numpy(off).to(DEV)
    nrm = ops.krbar_inv_norms(kr)
    excl = (np.random.default_rng(77).random((B, n_docs)) < 0.05).astype(np.uint8)
    ex = torch.from_numpy(excl).to(DEV)
    announce("route-scan-select")
    G = len(Kr)
    d1, i1, s1 = ops.route_topk(q, kr, offd, k, doc_exclude=ex, krbar_inv_norm=nrm)
    d0, c0 = ops.route_scores(q, kr, offd, doc_exclude=ex, krbar_inv_norm=nrm, want_chunk_scores=True)
    ws = ops.workspace(ops.route_topk_workspace_bytes(B, T, 8, 128, G, n_docs, k), DEV, "test-scan-select")
    ops.route_scan(q, kr, ws, krbar_inv_norm=nrm)
    d2, i2, s2 = ops.route_select(B, G, offd, k, ws, doc_exclude=ex)
    ops.route_scan(q, kr, ws, krbar_inv_norm=nrm)
    c3 = torch.empty((B, G), dtype=torch.float32, device=DEV)
    d3 = ops.route_select(B, G, offd, 0, ws, doc_exclude=ex, chunk_scores=c3)
    torch.cuda.synchronize()
    bits = lambda t: t.cpu().numpy().view(np.uint32)
    assert np.array_equal(bits(d1), bits(d2)) and np.array_equal(bits(d0), bits(d3))
    assert np.array_equal(bits(d0), bits(d1))
    assert np.array_equal(bits(c0), bits(c3))
    assert torch.equal(i1, i2) and np.array_equal(bits(s1), bits(s2))


# ---------------------------------------------------------------------- top-k
# ---------------------------------------------------------- routing backward
def _run_route_backward(Qr, Kr, off, dDoc, exclude=None, stored_norms=False, score_off=None):
    """Forward on the GPU for the chunk scores, then the backward.  score_off: offsets for the
    forward call when ``off`` has empty documents (chunk scores do not depend on the offsets)."""
    kr = dev_bits(Kr)
    nrm = ops.krbar_inv_norms(kr) if stored_norms else None
    q = dev_bits(Qr)
    fo = off if score_off is None else score_off
    _, ch = ops.route_scores(q, kr, torch.from_numpy(fo).to(DEV), want_chunk_scores=True, krbar_inv_norm=nrm)
    ex = None if exclude is None else torch.from_numpy(exclude.astype(np.uint8)).to(DEV)
    dQ, dK, sel = ops.route_scores_backward(q, kr, torch.from_numpy(off).to(DEV), ch,
                                            torch.from_numpy(dDoc.astype(np.float32)).to(DEV), doc_exclude=ex,
                                            krbar_inv_norm=nrm)
    torch.cuda.synchronize()
    return dQ.cpu().numpy(), dK.cpu().numpy(), sel.cpu().numpy()


def _check_route_backward(Qr, Kr, off, dDoc, exclude=None, stored_norms=False, score_off=None):
    q64, k64 = f64(Qr), f64(Kr)
    dDoc = dDoc.astype(np.float32).copy()
    dDoc[route_near_ties(q64, k64, off)] = 0.0          # P6: near ties get no gradient on either side
    dQ, dK, sel = _run_route_backward(Qr, Kr, off, dDoc, exclude, stored_norms, score_off)
    rQ, rK, rsel = O.route_backward(q64, k64, off, dDoc.astype(np.float64), exclude)
    assert np.array_equal(sel, rsel), f"selection differs at {np.argwhere(sel != rsel)[:5].tolist()}"
    sQ, sK = route_grad_bounds(q64, k64, dDoc, rsel)
    grads_ok(dK, rK, sK, "dK")
    grads_ok(dQ, rQ, sQ, "dQr")
    return sel


@pytest.mark.parametrize("B,T,H,n_docs", [(1, 1, 8, 50), (1, 7, 8, 337), (2, 40, 4, 1500), (1, 130, 8, 3000),
                                          (3, 5, 2, 700), (1, 33, 1, 2100), (16, 64, 8, 300), (1, 300, 8, 200),
                                          (2, 128, 8, 1100)])
def test_route_backward_matches_oracle(B, T, H, n_docs):
    announce("route-backward", B, T, H, n_docs)
    Qr, Kr, off = _route_case(B, T, H, n_docs, seed=300 + B * 1000 + T * 10 + H)
    dDoc = np.random.default_rng(n_docs).standard_normal((B, n_docs))
    sel = _check_route_backward(Qr, Kr, off, dDoc, stored_norms=(T > 20))
    assert (sel[..., 0] >= 0).mean() > 0.9


def test_route_backward_special_cases():
    """Exclusion, zero upstream gradients, zero query / key heads, empty documents, exact
    duplicate chunks and tokens (first maximiser), and a sparse upstream gradient."""
    B, T, H = 2, 45, 8
    r = np.random.default_rng(11)
    lens = r.integers(1, 7, 260)
    lens[[3, 100, 259]] = 0                               # empty documents
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    G = int(off[-1])
    Qr = sm.normal_bf16(11, sm.TID_QR, 0, 0, B * T * H * 128).reshape(B, T, H, 128).copy()
    Kr = sm.normal_bf16(11, sm.TID_KRBAR, 0, 0, G * H * 128).reshape(G, H, 128).copy()
    Qr[0, 9, 2] = 0                                       # zero query head
    Qr[1, :, 6] = 0                                       # a head that is zero for every token of query 1
    Kr[off[10], 4] = 0                                    # zero key head
    d = next(i for i in range(260) if lens[i] >= 3)
    Kr[off[d] + 2] = Kr[off[d]]                           # duplicate chunk inside a document
    Qr[0, 30] = Qr[0, 12]                                 # duplicate token rows
    excl = np.zeros((B, 260), bool)
    excl[0, [1, 7, 50]] = True
    excl[1, 200:210] = True
    dDoc = r.standard_normal((B, 260))
    dDoc[0, 20:40] = 0.0
    # the forward needs no empty documents: chunk scores depend only on the chunks
    score_off = np.concatenate([[0], np.cumsum(lens[lens > 0])]).astype(np.int64)
    announce("route-backward-special")
    for stored in (False, True):
        sel = _check_route_backward(Qr, Kr, off, dDoc, excl, stored, score_off)
        assert np.all(sel[excl] == -1) and np.all(sel[:, [3, 100, 259]] == -1) and np.all(sel[0, 20:40] == -1)
    # sparse upstream gradient: only each query's 16 best documents (a top-k loss)
    sparse = np.zeros_like(dDoc)
    top = np.argsort(-O.route(f64(Qr), f64(Kr), score_off)[1], axis=1)[:, :16]
    ids = np.flatnonzero(lens > 0)                        # score_off's documents -> off's documents
    for b in range(B):
        sparse[b, ids[top[b]]] = r.standard_normal(16)
    announce("route-backward-sparse")
    sel = _check_route_backward(Qr, Kr, off, sparse, None, True, score_off)
    assert (sel[..., 0] >= 0).sum() <= 2 * 16


@pytest.mark.parametrize("B,T,stored", [(4, 12, True), (4, 8, False)])
def test_route_backward_many_groups_per_workgroup(B, T, stored):
    """H = 8 with several groups of 32 documents per workgroup of the persistent selection kernel
    (9,001 documents over 4 queries: ~4 groups each, a partial last group), so the copies issued
    one group ahead and the chunk ids copied two groups ahead are exercised, with and without
    stored key norms."""
    n_docs = 9001
    announce("route-backward-many-groups", B, T, stored, n_docs)
    lens = np.random.default_rng(T).integers(1, 3, n_docs)
    Qr, Kr, off = _route_case(B, T, 8, n_docs, seed=1700 + T, lens=lens)
    dDoc = np.random.default_rng(T + 1).standard_normal((B, n_docs))
    excl = np.zeros((B, n_docs), bool)
    excl[1, ::97] = True
    sel = _check_route_backward(Qr, Kr, off, dDoc, excl, stored_norms=stored)
    assert (sel[..., 0] >= 0).mean() > 0.9


@pytest.mark.parametrize("B,T,H,n_docs", [(1, 8192, 8, 90), (2, 600, 8, 700), (1, 8192, 2, 40)])
def test_route_backward_long_queries(B, T, H, n_docs):
    """The longest router queries the call accepts (T = 8192: 256 token tiles, the router rows
    no longer resident in the H = 8 kernel) and a ragged long case."""
    announce("route-backward-long", B, T, H, n_docs)
    Qr, Kr, off = _route_case(B, T, H, n_docs, seed=900 + T + H)
    dDoc = np.random.default_rng(T).standard_normal((B, n_docs))
    sel = _check_route_backward(Qr, Kr, off, dDoc, stored_norms=True)
    assert (sel[..., 0] >= 0).mean() > 0.8


def test_route_backward_deterministic():
    Qr, Kr, off = _route_case(1, 16, 8, n_docs=5000, seed=21)   # ~300 documents per token: several pieces
    dDoc = np.random.default_rng(2).standard_normal((1, 5000))
    announce("route-backward-determinism")
    a = _run_route_backward(Qr, Kr, off, dDoc, stored_norms=True)
    b = _run_route_backward(Qr, Kr, off, dDoc, stored_norms=True)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


@pytest.mark.parametrize("B,T,n_docs,k,norms", [(1, 128, 3000, 16, True), (1, 128, 3000, 16, False), (2, 40, 1500, 5, True),
                                                (3, 7, 700, 1, True), (1, 33, 130, 32, False), (16, 64, 300, 16, True),
                                                (1, 128, 64, 32, True)])
def test_route_topk_matches_separate_calls(B, T, n_docs, k, norms):
    """msa_route_topk (document max and group maxima in one pass) gives exactly what
    msa_route_scores followed by msa_topk_docs gives, with excluded documents."""
    announce("route-topk", B, T, n_docs, k, norms)
    Qr, Kr, off = _route_case(B, T, 8, n_docs=n_docs, seed=B * 31 + T + k)
    q, kr, offd = dev_bits(Qr), dev_bits(Kr), torch.from_numpy(off).to(DEV)
    excl = np.zeros((B, n_docs), np.uint8); excl[:, 3::11] = 1
    ex = torch.from_numpy(excl).to(DEV)
    nrm = ops.krbar_inv_norms(kr) if norms else None
    d1, i1, s1 = ops.route_topk(q, kr, offd, k, doc_exclude=ex, krbar_inv_norm=nrm)
    d2 = ops.route_scores(q, kr, offd, doc_exclude=ex, krbar_inv_norm=nrm)
    i2, s2 = ops.topk_docs(d2, k)
    torch.cuda.synchronize()
    assert np.array_equal(d1.cpu().numpy().view(np.uint32), d2.cpu().numpy().view(np.uint32))
    assert np.array_equal(i1.cpu().numpy(), i2.cpu().numpy())
    assert np.array_equal(s1.cpu().numpy().view(np.uint32), s2.cpu().numpy().view(np.uint32))
    ref_idx, ref_sc = O.topk(d1.cpu().numpy().astype(np.float64), k)
    assert np.array_equal(i1.cpu().numpy(), ref_idx)


@pytest.mark.parametrize("B,n,k", [(1, 64, 4), (1, 1000, 16), (16, 20000, 16), (1, 200000, 16), (4, 20000, 8),
                                   (1, 7, 7), (3, 5, 1), (2, 4097, 1024), (1, 2049, 2), (2, 100, 100),
                                   (1, 70000, 32), (2, 40000, 17), (3, 33000, 5), (1, 32768, 16), (1, 32769, 3),
                                   (2, 513, 33), (1, 1, 1)])
def test_topk_matches_oracle(B, n, k):
    announce("topk", B, n, k)
    r = np.random.default_rng(B * 7 + n + k)
    s = r.standard_normal((B, n)).astype(np.float32)
    s[:, ::5] = np.round(s[:, ::5], 1)                       # ties
    if n > 10:
        s[0, 3] = -np.inf
    idx, sc = ops.topk_docs(torch.from_numpy(s).to(DEV), k)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy(); sc = sc.cpu().numpy()
    ref_idx, ref_sc = O.topk(s.astype(np.float64), k)
    # the scores are exact fp32 inputs: selection and order must be identical
    assert np.array_equal(idx, ref_idx)
    assert np.array_equal(sc.astype(np.float64), ref_sc)


@pytest.mark.parametrize("pattern", ["ascending", "descending", "constant", "one_block", "sparse_finite"])
@pytest.mark.parametrize("n,k", [(200000, 16), (20000, 8), (3000, 4), (1000, 16), (130, 16)])
def test_topk_score_layouts(pattern, n, k):
    """Layouts that defeat the per-wave thresholds (the best keys packed into one wave's share, ties everywhere)."""
    announce("topk layout", pattern, n, k)
    r = np.random.default_rng(n + k)
    if pattern == "ascending":
        s = np.linspace(-1.0, 1.0, n, dtype=np.float32)
    elif pattern == "descending":
        s = np.linspace(1.0, -1.0, n, dtype=np.float32)
    elif pattern == "constant":
        s = np.full(n, 0.25, dtype=np.float32)
    elif pattern == "one_block":                            # the top documents all inside one 64-document group run
        s = r.standard_normal(n).astype(np.float32) * 0.01
        m = min(40 * k, n - n // 3)
        s[n // 3: n // 3 + m] = 1.0 + r.random(m).astype(np.float32)
    else:                                                   # nearly everything excluded
        s = np.full(n, -np.inf, dtype=np.float32)
        s[r.choice(n, min(n, k + 3), replace=False)] = r.standard_normal(min(n, k + 3)).astype(np.float32)
    s = s[None]
    idx, sc = ops.topk_docs(torch.from_numpy(s).to(DEV), k)
    torch.cuda.synchronize()
    ref_idx, ref_sc = O.topk(s.astype(np.float64), k)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    assert np.array_equal(sc.cpu().numpy().astype(np.float64), ref_sc)


@pytest.mark.parametrize("n_s", [255, 256, 1023, 1024])
@pytest.mark.parametrize("within", ["constant", "one_doc"])
def test_topk_short_list_boundaries(n_s, within):
    """The filtered path's short lists at their size limits (200,000 documents, k = 16).

    Documents score -1 except: document 0 scores 0.5 (the smallest of the 16 waves'
    maxima, so the first threshold is its key), and n_s groups spread over the other
    waves' shares score 1.0 — every document of the group ("constant": the second list
    then holds the 15 best groups' 64 documents + 1 = 961 keys) or its first document
    only ("one_doc": 16 keys).  The first list holds n_s + 1 keys: 256 (ranked), 257
    and 1,024 (reduced by waves), 1,025 (overflow: selection over every group maximum)."""
    announce("topk list", n_s, within)
    n, k = 200000, 16
    n_groups = (n + 63) // 64
    per = (n_groups + 15) // 16
    s = np.full(n, -1.0, dtype=np.float32)
    s[0] = 0.5
    groups = np.unique(np.linspace(per, n_groups - 1, n_s).astype(np.int64))
    assert len(groups) == n_s
    for g in groups:
        if within == "constant":
            s[g * 64: min(n, g * 64 + 64)] = 1.0
        else:
            s[g * 64] = 1.0
    s = s[None]
    idx, sc = ops.topk_docs(torch.from_numpy(s).to(DEV), k)
    torch.cuda.synchronize()
    ref_idx, ref_sc = O.topk(s.astype(np.float64), k)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    assert np.array_equal(sc.cpu().numpy().astype(np.float64), ref_sc)


# ---------------------------------------------------------------------- pool
@pytest.mark.parametrize("H,lens", [(8, [1, 63, 64, 65, 130, 512, 7, 200]), (4, [64, 3, 129]), (16, [70, 1]),
                                    (2, [300, 5, 64])])
def test_pool_matches_oracle(H, lens):
    announce("pool", H, lens)
    w = C.workload("tiny-32K", n_docs=len(lens), length_law="custom", custom_lengths=tuple(lens), H=H)
    K = C.raw_block(w, "K", 0, w.n_tok); V = C.raw_block(w, "V", 0, w.n_tok); Kr = C.raw_block(w, "Kr", 0, w.n_tok)
    Kb, Vb, Rb = ops.pool_chunks(dev_bits(K), dev_bits(V), dev_bits(Kr), torch.from_numpy(w.doc_tok_off).to(DEV),
                                 torch.from_numpy(w.doc_chunk_off).to(DEV), w.n_chunks, 64, w.rope_base)
    torch.cuda.synchronize()
    rK, rV, rR, off = O.pool(f64(K), f64(V), f64(Kr), w.doc_len, 64, w.rope_base)
    assert bf16_ulp_diff(host_bits(Vb), O.f64_to_bf16_bits(rV)).max() <= 1
    assert bf16_ulp_diff(host_bits(Rb), O.f64_to_bf16_bits(rR)).max() <= 1
    assert pooled_k_ok(host_bits(Kb), rK, *pooled_k_scales(f64(K), w.doc_len, 64))


@pytest.mark.parametrize("chunk,lens", [(1, [5, 1, 3]), (100, [100, 101, 250, 37, 1]), (256, [600, 256, 1, 70]),
                                        (1024, [1500, 1024, 3]), (33, [99, 34, 2])])
def test_pool_chunk_lengths_match_oracle(chunk, lens):
    """Chunk lengths other than 64: one token per chunk, chunks of several 64-token rotation blocks
    with a ragged last block, the 1024 maximum, and lengths that do not divide 64."""
    announce("pool-chunk", chunk, lens)
    w = C.workload("tiny-32K", n_docs=len(lens), length_law="custom", custom_lengths=tuple(lens), chunk=chunk)
    K = C.raw_block(w, "K", 0, w.n_tok); V = C.raw_block(w, "V", 0, w.n_tok); Kr = C.raw_block(w, "Kr", 0, w.n_tok)
    Kb, Vb, Rb = ops.pool_chunks(dev_bits(K), dev_bits(V), dev_bits(Kr), torch.from_numpy(w.doc_tok_off).to(DEV),
                                 torch.from_numpy(w.doc_chunk_off).to(DEV), w.n_chunks, chunk, w.rope_base)
    torch.cuda.synchronize()
    rK, rV, rR, off = O.pool(f64(K), f64(V), f64(Kr), w.doc_len, chunk, w.rope_base)
    assert Kb.shape[0] == off[-1]
    assert bf16_ulp_diff(host_bits(Vb), O.f64_to_bf16_bits(rV)).max() <= 1
    assert bf16_ulp_diff(host_bits(Rb), O.f64_to_bf16_bits(rR)).max() <= 1
    assert pooled_k_ok(host_bits(Kb), rK, *pooled_k_scales(f64(K), w.doc_len, chunk))


def test_pool_slab_with_offset_bases():
    # a slab of documents 3..5 of a corpus: offsets rebased by the caller's first row
    lens = [100, 64, 1, 300, 65, 2]
    w = C.workload("tiny-32K", n_docs=6, length_law="custom", custom_lengths=tuple(lens))
    K = C.raw_block(w, "K", 0, w.n_tok); V = C.raw_block(w, "V", 0, w.n_tok); Kr = C.raw_block(w, "Kr", 0, w.n_tok)
    t0, t1 = int(w.doc_tok_off[3]), int(w.doc_tok_off[6])
    c0, c1 = int(w.doc_chunk_off[3]), int(w.doc_chunk_off[6])
    announce("pool-slab")
    Kb, Vb, Rb = ops.pool_chunks(dev_bits(K[t0:t1]), dev_bits(V[t0:t1]), dev_bits(Kr[t0:t1]),
                                 torch.from_numpy(w.doc_tok_off[3:]).to(DEV),
                                 torch.from_numpy(w.doc_chunk_off[3:]).to(DEV), c1 - c0, 64, w.rope_base)
    torch.cuda.synchronize()
    rK, rV, rR, off = O.pool(f64(K), f64(V), f64(Kr), w.doc_len, 64, w.rope_base)
    assert bf16_ulp_diff(host_bits(Vb), O.f64_to_bf16_bits(rV[c0:c1])).max() <= 1
    assert bf16_ulp_diff(host_bits(Rb), O.f64_to_bf16_bits(rR[c0:c1])).max() <= 1
    m, n = pooled_k_scales(f64(K), w.doc_len, 64)
    assert pooled_k_ok(host_bits(Kb), rK[c0:c1], m[c0:c1], n[c0:c1])


# ------------------------------------------------------- router-key encoding
def _encode_case(lens, dm, H, chunk, seed, first_doc=0):
    """Encode documents first_doc.. of a corpus with the given lengths; returns gpu bits, oracle, magnitude."""
    r = np.random.default_rng(seed)
    n_tok = sum(lens)
    hid = O.f64_to_bf16_bits(r.standard_normal((n_tok, dm)))
    W = O.f64_to_bf16_bits(r.standard_normal((H * 128, dm)))
    tok_off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    ch_off = O.chunk_offsets(lens, chunk)
    t0, c0 = int(tok_off[first_doc]), int(ch_off[first_doc])
    n_chunks = int(ch_off[-1]) - c0
    out = ops.encode_router_keys(dev_bits(hid[t0:]), dev_bits(W), torch.from_numpy(tok_off[first_doc:]).to(DEV),
                                 torch.from_numpy(ch_off[first_doc:]).to(DEV), n_chunks, H, chunk)
    torch.cuda.synchronize()
    ref, _ = O.encode_router_keys(O.bf16_to_f64(hid), O.bf16_to_f64(W), lens, chunk, H, 128)
    # per element sum_k |mean hidden_k| |W_nk| of the exact chunk means (the error scale of P5)
    hf = O.bf16_to_f64(hid)
    means = np.stack([hf[int(tok_off[d]) + j * chunk: int(tok_off[d]) + min((j + 1) * chunk, lens[d])].mean(axis=0)
                      for d in range(len(lens)) for j in range(int(ch_off[d + 1] - ch_off[d]))])
    mag = (np.abs(means) @ np.abs(O.bf16_to_f64(W)).T).reshape(ref.shape)
    return host_bits(out), ref[c0:], mag[c0:]


@pytest.mark.parametrize("lens,dm,H,chunk", [([1, 63, 64, 65, 130, 300, 7, 2000, 64], 2560, 8, 64),
                                             ([5, 3, 200], 64, 1, 64), ([100, 33, 257], 96, 2, 32),
                                             ([64] * 300, 256, 4, 64), ([700, 1, 1024], 128, 16, 100)])
def test_encode_router_keys_matches_oracle(lens, dm, H, chunk):
    announce("encode", len(lens), dm, H, chunk)
    gpu, ref, mag = _encode_case(lens, dm, H, chunk, seed=dm + H + chunk)
    assert gpu.shape == ref.shape
    assert encoded_keys_ok(gpu, ref, mag)
    # most elements are exactly the oracle's rounded value
    assert (bf16_ulp_diff(gpu, O.f64_to_bf16_bits(ref)) == 0).mean() > 0.9


def test_encode_slab_with_offset_bases():
    announce("encode-slab")
    gpu, ref, mag = _encode_case([90, 64, 1, 300, 65, 2, 129], 512, 8, 64, seed=7, first_doc=3)
    assert encoded_keys_ok(gpu, ref, mag)


# ------------------------------------------------------------ store updates
def _random_store(n_docs, H, seed, max_chunks=9):
    r = np.random.default_rng(seed)
    counts = r.integers(1, max_chunks + 1, n_docs)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    rows = O.f64_to_bf16_bits(r.standard_normal((int(off[-1]), H, 128)))
    return rows, off, r


@pytest.mark.parametrize("n_docs,H,pattern", [(50, 8, "random"), (1, 8, "all"), (1, 8, "none"), (300, 4, "none"),
                                              (300, 4, "all"), (2000, 8, "random"), (7, 16, "ends")])
def test_store_delete_bit_exact(n_docs, H, pattern):
    announce("store-delete", n_docs, H, pattern)
    rows, off, r = _random_store(n_docs, H, seed=n_docs + H)
    keep = {"random": r.random(n_docs) < 0.6, "all": np.ones(n_docs, bool), "none": np.zeros(n_docs, bool),
            "ends": np.array([0, 1, 1, 0, 1, 1, 0], bool)}[pattern]
    kr = dev_bits(rows)
    nrm = ops.krbar_inv_norms(kr)
    kr_o, nrm_o, off_o, ids, counts = ops.store_delete(kr, torch.from_numpy(off).to(DEV),
                                                       torch.from_numpy(keep.astype(np.uint8)).to(DEV), inv_norm=nrm)
    torch.cuda.synchronize()
    ref_rows, ref_off, ref_ids = O.store_delete(rows, off, keep)
    ref_nrm, _, _ = O.store_delete(nrm.cpu().numpy(), off, keep)
    nd, nc = (int(x) for x in counts.cpu())
    assert (nd, nc) == (len(ref_off) - 1, len(ref_rows))
    assert np.array_equal(host_bits(kr_o)[:nc], ref_rows)
    assert np.array_equal(nrm_o.cpu().numpy()[:nc], ref_nrm)
    assert np.array_equal(off_o.cpu().numpy()[:nd + 1], ref_off)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)


def test_store_append_then_delete_round_trip():
    announce("store-append")
    rows, off, r = _random_store(40, 8, seed=11)
    new_rows, new_off, _ = _random_store(9, 8, seed=12)
    cap_c, cap_d = len(rows) + len(new_rows) + 5, 40 + 9 + 3
    kr = torch.zeros((cap_c, 8, 128), dtype=torch.int16, device=DEV)
    kr[:len(rows)] = dev_bits(rows)
    nrm = torch.zeros((cap_c, 8), dtype=torch.float32, device=DEV)
    nrm[:len(rows)] = ops.krbar_inv_norms(kr[:len(rows)])
    offd = torch.zeros(cap_d + 1, dtype=torch.int64, device=DEV)
    offd[:41] = torch.from_numpy(off)
    nd, nc = ops.store_append(kr, offd, 40, len(rows), dev_bits(new_rows), torch.from_numpy(new_off).to(DEV),
                              inv_norm=nrm)
    torch.cuda.synchronize()
    ref_rows, ref_off = O.store_append(rows, off, new_rows, new_off)
    assert (nd, nc) == (49, len(ref_rows))
    assert np.array_equal(host_bits(kr)[:nc], ref_rows)
    assert np.array_equal(offd.cpu().numpy()[:nd + 1], ref_off)
    # the appended chunks' norms are the ones a scratch build computes
    scratch = ops.krbar_inv_norms(kr[:nc].contiguous())
    assert torch.equal(nrm[:nc], scratch)
    # deleting the appended documents gives the original store back
    keep = np.r_[np.ones(40, bool), np.zeros(9, bool)]
    kr_o, nrm_o, off_o, ids, counts = ops.store_delete(kr[:nc].contiguous(), offd[:nd + 1].contiguous(),
                                                       torch.from_numpy(keep.astype(np.uint8)).to(DEV),
                                                       inv_norm=nrm[:nc].contiguous())
    torch.cuda.synchronize()
    assert [int(x) for x in counts.cpu()] == [40, len(rows)]
    assert np.array_equal(host_bits(kr_o)[:len(rows)], rows)
    assert np.array_equal(off_o.cpu().numpy()[:41], off)


# ------------------------------------------------------------------ attention
@pytest.mark.parametrize("B,Tq,Tl,M,offset", [(1, 32, 32, 32, 4), (1, 1, 128, 262, 16), (1, 128, 128, 262, 16),
                                              (2, 64, 64, 133, 16), (1, 5, 9, 0, 0), (1, 17, 40, 1, 3),
                                              (3, 16, 16, 70, 8), (1, 128, 128, 448, 16),
                                              (1, 64, 200, 40, 7), (2, 1, 300, 5, 2),
                                              # 32-row tiles with 5-8, 14-16 and 17 key tiles over 8 waves
                                              (1, 128, 128, 128, 16), (1, 96, 96, 416, 16), (1, 32, 128, 400, 9),
                                              # <= 4 rows, Mmax + Tl <= 512, Tl <= 128: the few-row kernel
                                              (1, 1, 128, 133, 16), (1, 3, 100, 50, 7), (2, 4, 4, 0, 0),
                                              (1, 1, 1, 1, 0), (1, 2, 128, 384, 16), (3, 1, 64, 77, 5)])
def test_attention_matches_oracle(B, Tq, Tl, M, offset):
    announce("attn", B, Tq, Tl, M, offset)
    seed = B * 1000 + Tq + M
    Hq, Hkv, D = 32, 8, 128
    Q = sm.normal_bf16(seed, sm.TID_Q, 0, 0, B * Tq * Hq * D).reshape(B, Tq, Hq, D)
    Kl = sm.normal_bf16(seed, sm.TID_KLOC, 0, 0, B * Tl * Hkv * D).reshape(B, Tl, Hkv, D)
    Vl = sm.normal_bf16(seed, sm.TID_VLOC, 0, 0, B * Tl * Hkv * D).reshape(B, Tl, Hkv, D)
    Mmax = max(M, 1)
    st = sm.normal_bf16(seed, sm.TID_KBAR, 0, 0, B * Mmax * 2 * Hkv * D).reshape(B, Mmax, 2, Hkv, D)
    mem_len = np.array([max(M - 3 * b, 0) for b in range(B)], dtype=np.int32)
    stg = dev_bits(st)
    O_gpu = ops.sparse_attn_decode(dev_bits(Q), dev_bits(Kl), dev_bits(Vl), stg, stg[:, :, 1], 2 * Hkv * D, Mmax,
                                   torch.from_numpy(mem_len).to(DEV), offset, 1e6)
    torch.cuda.synchronize()
    o = O_gpu.cpu().numpy()
    for b in range(B):
        m = int(mem_len[b])
        ref = O.attend(f64(Q[b]), f64(Kl[b]), f64(Vl[b]), f64(st[b, :m, 0]), f64(st[b, :m, 1]), offset, 1e6,
                       D ** -0.5)
        assert rel_rows(o[b], ref) <= ATT_TOL
        assert rel_rows(o[b], ref) <= 1e-4          # fp32 path: far inside the bf16 budget


@pytest.mark.parametrize("B,Tq,Tl,M,offset,Hq,Hkv", [(1, 32, 32, 32, 4, 32, 8), (1, 1, 128, 262, 16, 32, 8),
                                                     (1, 128, 128, 262, 16, 32, 8), (2, 64, 64, 133, 16, 32, 8),
                                                     (1, 5, 9, 0, 0, 32, 8), (2, 1, 300, 5, 2, 32, 8),
                                                     (1, 100, 130, 45, 7, 32, 8), (1, 40, 50, 20, 5, 16, 2),
                                                     (1, 300, 1000, 700, 16, 32, 8)])
def test_attention_split_matches_fused_and_oracle(B, Tq, Tl, M, offset, Hq, Hkv):
    """msa_sparse_attn_local_partial on a side stream, then msa_sparse_attn_memory_merge after an
    event: O against the oracle and against the one-launch kernel, lse against the oracle."""
    announce("attn-split", B, Tq, Tl, M, offset, Hq, Hkv)
    Q, Kl, Vl, st, mem_len, _, Mmax = _attn_bwd_case(B, Tq, Tl, M, offset, Hq, Hkv, seed=B * 700 + Tq + M)
    stg = dev_bits(st)
    q, kl, vl = dev_bits(Q), dev_bits(Kl), dev_bits(Vl)
    ml = torch.from_numpy(mem_len).to(DEV)
    side = torch.cuda.Stream()
    ev = torch.cuda.Event()
    side.wait_stream(torch.cuda.current_stream())               # inputs are ready
    with torch.cuda.stream(side):
        part = ops.sparse_attn_local_partial(q, kl, vl, offset, 1e6, stream=side)
        ev.record(side)
    torch.cuda.current_stream().wait_event(ev)
    lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=DEV)
    o = ops.sparse_attn_memory_merge(q, Tl, Hkv, stg, stg[:, :, 1], 2 * Hkv * 128, Mmax, ml, offset, part, 1e6, lse=lse)
    fused = ops.sparse_attn_decode(q, kl, vl, stg, stg[:, :, 1], 2 * Hkv * 128, Mmax, ml, offset, 1e6)
    torch.cuda.synchronize()
    o, lse, fused = o.cpu().numpy(), lse.cpu().numpy(), fused.cpu().numpy()
    assert rel_rows(o, fused) <= 1e-5                            # same sums in another order
    worst = 0.0
    for b in range(B):
        m = int(mem_len[b])
        ref = O.attend(f64(Q[b]), f64(Kl[b]), f64(Vl[b]), f64(st[b, :m, 0]), f64(st[b, :m, 1]), offset, 1e6,
                       128 ** -0.5)
        assert rel_rows(o[b], ref) <= 1e-4
        ref_lse = O.attend_lse(f64(Q[b]), f64(Kl[b]), f64(st[b, :m, 0]), offset, 1e6, 128 ** -0.5)
        worst = max(worst, float(np.abs(lse[b] - ref_lse).max()))
    assert worst <= LSE_TOL


def _random_attn_shapes(n=24, seed=20261204):
    """Seeded shapes across both attention kernels: 1-4 query rows (the few-row kernel when the
    keys fit) and up to 200 (the matrix-core kernel), local lengths past the 128-position table,
    memory lengths from none to several hundred entries, and four GQA ratios."""
    rng = np.random.default_rng(seed)
    heads = [(32, 8), (16, 2), (8, 8), (32, 4)]
    out = []
    for i in range(n):
        Tq = int(rng.choice([1, 2, 4])) if i % 3 == 0 else int(rng.integers(1, 201))
        Tl = Tq + int(rng.integers(0, 301))
        M = int(rng.choice([0, int(rng.integers(1, 33)), int(rng.integers(33, 401))]))
        Hq, Hkv = heads[i % len(heads)]
        out.append((int(rng.integers(1, 3)), Tq, Tl, M, int(rng.integers(0, 33)), Hq, Hkv))
    return out


@pytest.mark.parametrize("B,Tq,Tl,M,offset,Hq,Hkv", _random_attn_shapes())
def test_attention_random_shapes_match_oracle(B, Tq, Tl, M, offset, Hq, Hkv):
    """msa_sparse_attn_decode and msa_sparse_attn_forward (O and log-sum-exp) against the oracle; the
    two-launch split (local partial + memory merge) against the one-launch forward."""
    announce("attn-random", B, Tq, Tl, M, offset, Hq, Hkv)
    Q, Kl, Vl, st, mem_len, _, Mmax = _attn_bwd_case(B, Tq, Tl, M, offset, Hq, Hkv, seed=B * 911 + Tq * 7 + M)
    stg = dev_bits(st)
    args = (dev_bits(Q), dev_bits(Kl), dev_bits(Vl), stg, stg[:, :, 1], 2 * Hkv * 128, Mmax,
            torch.from_numpy(mem_len).to(DEV), offset)
    o_dec = ops.sparse_attn_decode(*args, 1e6)
    o_fwd, lse = ops.sparse_attn_forward(*args, rope_base=1e6)
    # the same attention in two launches: local-key partial, then the memory pass merging with it
    part = ops.sparse_attn_local_partial(args[0], args[1], args[2], offset, 1e6)
    o_split = ops.sparse_attn_memory_merge(args[0], Tl, Hkv, stg, stg[:, :, 1], 2 * Hkv * 128, Mmax, args[7], offset,
                                           part, 1e6)
    torch.cuda.synchronize()
    o_dec, o_fwd, lse = o_dec.cpu().numpy(), o_fwd.cpu().numpy(), lse.cpu().numpy()
    assert rel_rows(o_split.cpu().numpy(), o_fwd) <= 1e-5      # same sums in another order
    for b in range(B):
        m = int(mem_len[b])
        ref = O.attend(f64(Q[b]), f64(Kl[b]), f64(Vl[b]), f64(st[b, :m, 0]), f64(st[b, :m, 1]), offset, 1e6,
                       128 ** -0.5)
        assert rel_rows(o_dec[b], ref) <= 1e-4
        assert rel_rows(o_fwd[b], ref) <= 1e-4
        ref_lse = O.attend_lse(f64(Q[b]), f64(Kl[b]), f64(st[b, :m, 0]), offset, 1e6, 128 ** -0.5)
        assert float(np.abs(lse[b] - ref_lse).max()) <= LSE_TOL


# ------------------------------------------------------ attention backward
def _attn_bwd_case(B, Tq, Tl, M, offset, Hq=32, Hkv=8, seed=0):
    D = 128
    Q = sm.normal_bf16(seed, sm.TID_Q, 1, 0, B * Tq * Hq * D).reshape(B, Tq, Hq, D)
    Kl = sm.normal_bf16(seed, sm.TID_KLOC, 1, 0, B * Tl * Hkv * D).reshape(B, Tl, Hkv, D)
    Vl = sm.normal_bf16(seed, sm.TID_VLOC, 1, 0, B * Tl * Hkv * D).reshape(B, Tl, Hkv, D)
    Mmax = max(M, 1)
    st = sm.normal_bf16(seed, sm.TID_KBAR, 1, 0, B * Mmax * 2 * Hkv * D).reshape(B, Mmax, 2, Hkv, D)
    mem_len = np.array([max(M - 3 * b, 0) for b in range(B)], dtype=np.int32)
    dO = np.random.default_rng(seed).standard_normal((B, Tq, Hq, D)).astype(np.float32)
    return Q, Kl, Vl, st, mem_len, dO, Mmax


def _run_attn_bwd(Q, Kl, Vl, st, mem_len, dO, Mmax, offset, saved=False):
    """The backward on the GPU; saved=True first runs the forward with its log-sum-exp and
    hands (O, lse) to msa_sparse_attn_backward_saved."""
    stg = dev_bits(st)
    args = (dev_bits(Q), dev_bits(Kl), dev_bits(Vl), stg, stg[:, :, 1], 2 * st.shape[-2] * 128, Mmax,
            torch.from_numpy(mem_len).to(DEV), offset)
    kw = {}
    if saved:
        o, lse = ops.sparse_attn_forward(*args, rope_base=1e6)
        kw = dict(O=o, lse=lse)
    out = ops.sparse_attn_backward(*args, torch.from_numpy(dO).to(DEV), rope_base=1e6, **kw)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


@pytest.mark.parametrize("B,Tq,Tl,M,offset,Hq,Hkv", [(1, 32, 32, 32, 4, 32, 8), (1, 1, 128, 262, 16, 32, 8),
                                                     (1, 128, 128, 262, 16, 32, 8), (2, 64, 64, 133, 16, 32, 8),
                                                     (1, 5, 9, 0, 0, 32, 8), (1, 17, 40, 1, 3, 32, 8),
                                                     (3, 16, 16, 70, 8, 32, 8), (2, 1, 300, 5, 2, 32, 8),
                                                     (1, 100, 130, 45, 7, 32, 8), (1, 40, 50, 20, 5, 16, 2),
                                                     (1, 33, 33, 10, 0, 8, 8)])
@pytest.mark.parametrize("saved", [False, True])
def test_attention_backward_matches_oracle(B, Tq, Tl, M, offset, Hq, Hkv, saved):
    """saved=True: msa_sparse_attn_backward_saved with the GPU forward's O and log-sum-exp."""
    announce("attn-backward", B, Tq, Tl, M, offset, Hq, Hkv, "saved" if saved else "recomputed")
    Q, Kl, Vl, st, mem_len, dO, Mmax = _attn_bwd_case(B, Tq, Tl, M, offset, Hq, Hkv, seed=B * 1000 + Tq + M)
    dQ, dKl, dVl, dKm, dVm = _run_attn_bwd(Q, Kl, Vl, st, mem_len, dO, Mmax, offset, saved=saved)
    worst = 0.0
    for b in range(B):
        m = int(mem_len[b])
        ref = O.attend_backward(f64(Q[b]), f64(Kl[b]), f64(Vl[b]), f64(st[b, :m, 0]), f64(st[b, :m, 1]), offset,
                                1e6, 128 ** -0.5, dO[b].astype(np.float64))
        got = (dQ[b], dKl[b], dVl[b], dKm[b, :m], dVm[b, :m])
        for name, x, y in zip(("dQ", "dKloc", "dVloc", "dKmem", "dVmem"), got, ref):
            if y.size:
                e = rel_rows(x, y)
                worst = max(worst, e)
                assert e <= ATT_TOL, f"{name} b={b}: {e}"
        assert np.all(dKm[b, m:] == 0) and np.all(dVm[b, m:] == 0)
    print("worst per-row relative error", worst, flush=True)
    assert worst <= ATT_GRAD_OBS


@pytest.mark.parametrize("B,Tq,Tl,M,offset,Hq,Hkv", [(1, 128, 128, 262, 16, 32, 8), (2, 64, 64, 133, 16, 32, 8),
                                                     (1, 1, 128, 262, 16, 32, 8), (1, 5, 9, 0, 0, 32, 8),
                                                     (1, 100, 130, 45, 7, 32, 8), (1, 40, 50, 20, 5, 16, 2),
                                                     (1, 2, 64, 30, 3, 16, 2), (2, 4, 100, 300, 9, 8, 8)])
def test_attention_forward_lse_matches_oracle(B, Tq, Tl, M, offset, Hq, Hkv):
    """msa_sparse_attn_forward: O as msa_sparse_attn_decode, and each row's natural log-sum-exp."""
    announce("attn-forward-lse", B, Tq, Tl, M, offset, Hq, Hkv)
    Q, Kl, Vl, st, mem_len, _, Mmax = _attn_bwd_case(B, Tq, Tl, M, offset, Hq, Hkv, seed=B * 500 + Tq + M)
    stg = dev_bits(st)
    args = (dev_bits(Q), dev_bits(Kl), dev_bits(Vl), stg, stg[:, :, 1], 2 * Hkv * 128, Mmax,
            torch.from_numpy(mem_len).to(DEV), offset)
    o, lse = ops.sparse_attn_forward(*args, rope_base=1e6)
    o_dec = ops.sparse_attn_decode(*args, rope_base=1e6)
    torch.cuda.synchronize()
    o, lse, o_dec = o.cpu().numpy(), lse.cpu().numpy(), o_dec.cpu().numpy()
    assert np.array_equal(o.view(np.uint32), o_dec.view(np.uint32))       # same kernel, same output
    worst = 0.0
    for b in range(B):
        m = int(mem_len[b])
        ref = O.attend_lse(f64(Q[b]), f64(Kl[b]), f64(st[b, :m, 0]), offset, 1e6, 128 ** -0.5)
        worst = max(worst, float(np.abs(lse[b] - ref).max()))
        ref_o = O.attend(f64(Q[b]), f64(Kl[b]), f64(Vl[b]), f64(st[b, :m, 0]), f64(st[b, :m, 1]), offset, 1e6,
                         128 ** -0.5)
        assert rel_rows(o[b], ref_o) <= ATT_TOL
    print("worst lse error", worst, flush=True)
    assert worst <= LSE_TOL


@pytest.mark.parametrize("B,Tq,Tl,M,offset", [(1, 512, 1024, 700, 16), (2, 300, 300, 0, 0), (1, 1, 2000, 950, 8)])
def test_attention_backward_long(B, Tq, Tl, M, offset):
    """Many row and key tiles: long local contexts, large memories, no memory, a single row."""
    announce("attn-backward-long", B, Tq, Tl, M, offset)
    Q, Kl, Vl, st, mem_len, dO, Mmax = _attn_bwd_case(B, Tq, Tl, M, offset, seed=7 * Tq + M)
    dQ, dKl, dVl, dKm, dVm = _run_attn_bwd(Q, Kl, Vl, st, mem_len, dO, Mmax, offset)
    worst = 0.0
    for b in range(B):
        m = int(mem_len[b])
        ref = O.attend_backward(f64(Q[b]), f64(Kl[b]), f64(Vl[b]), f64(st[b, :m, 0]), f64(st[b, :m, 1]), offset,
                                1e6, 128 ** -0.5, dO[b].astype(np.float64))
        for x, y in zip((dQ[b], dKl[b], dVl[b], dKm[b, :m], dVm[b, :m]), ref):
            if y.size:
                worst = max(worst, rel_rows(x, y))
    print("worst per-row relative error", worst, flush=True)
    assert worst <= ATT_GRAD_OBS


def test_attention_backward_deterministic():
    Q, Kl, Vl, st, mem_len, dO, Mmax = _attn_bwd_case(2, 128, 128, 262, 16, seed=5)
    announce("attn-backward-determinism")
    a = _run_attn_bwd(Q, Kl, Vl, st, mem_len, dO, Mmax, 16)
    b = _run_attn_bwd(Q, Kl, Vl, st, mem_len, dO, Mmax, 16)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


# ---------------------------------------------------------------- assembly
def test_fetch_and_gather_assemble_rank_order():
    announce("fetch/gather")
    H, D = 8, 128
    lens = np.array([3, 1, 5, 2, 4, 1, 6], dtype=np.int64)
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    G = int(off[-1])
    store_np = sm.normal_bf16(9, sm.TID_KBAR, 0, 0, G * 2 * H * D).reshape(G, 2, H, D)
    store = torch.from_numpy(store_np.view(np.int16)).pin_memory()
    top = np.array([[2, 3, 0], [6, 1, 4]], dtype=np.int32)     # 2,3 adjacent -> one copy
    Mmax = 12
    staging = torch.zeros((2, Mmax, 2, H, D), dtype=torch.int16, device=DEV)
    side = torch.cuda.Stream()
    ev = torch.cuda.Event()
    ml = ops.fetch_docs(torch.from_numpy(top), store, torch.from_numpy(off), staging, Mmax, side, ev)
    assert ev.cuda_event, "the completion event must exist so that it orders the copies"
    ev.synchronize()
    st = host_bits(staging)
    for b in range(2):
        chunks = O.assemble(top[b], off)
        assert ml[b] == len(chunks)
        assert np.array_equal(st[b, :len(chunks)], store_np[chunks])
    staging2 = torch.zeros_like(staging)
    ml2 = ops.gather_docs(torch.from_numpy(top).to(DEV), store, torch.from_numpy(off).to(DEV), staging2, Mmax)
    torch.cuda.synchronize()
    assert np.array_equal(ml2.cpu().numpy(), ml.numpy())
    assert np.array_equal(host_bits(staging2), st)


# ------------------------------------------------------------- end to end
def test_tiny_corpus_end_to_end_step():
    """Pool raw K/V/Kr, route, top-k, fetch from pinned host, attend (Tq = T and Tq = 1)."""
    w = C.workload("tiny-32K")
    announce("tiny-32K e2e", w.describe())
    K = C.raw_block(w, "K", 0, w.n_tok); V = C.raw_block(w, "V", 0, w.n_tok); Kr = C.raw_block(w, "Kr", 0, w.n_tok)
    q = C.queries(w)
    tok_off = torch.from_numpy(w.doc_tok_off).to(DEV); ch_off = torch.from_numpy(w.doc_chunk_off).to(DEV)
    Kb, Vb, Rb = ops.pool_chunks(dev_bits(K), dev_bits(V), dev_bits(Kr), tok_off, ch_off, w.n_chunks, 64, w.rope_base)
    doc = ops.route_scores(dev_bits(q["Qr"]), Rb, ch_off)
    idx, sc = ops.topk_docs(doc, w.k)
    store = torch.stack([Kb, Vb], dim=1).cpu().pin_memory()          # [G, 2, H, D] host tier
    Mmax = int(w.doc_n_chunks.max()) * w.k
    staging = torch.zeros((1, Mmax, 2, w.H, w.D), dtype=torch.int16, device=DEV)
    ml = ops.fetch_docs(idx.cpu(), store, torch.from_numpy(w.doc_chunk_off), staging, Mmax)
    ml_dev = ml.to(DEV)
    outs = {}
    for Tq in (w.Tq, 1):
        Qx = dev_bits(q["Q"][:, -Tq:])
        outs[Tq] = ops.sparse_attn_decode(Qx, dev_bits(q["Kloc"]), dev_bits(q["Vloc"]), staging, staging[:, :, 1],
                                          2 * w.H * w.D, Mmax, ml_dev, w.k, w.rope_base)
    torch.cuda.synchronize()
    # oracle pipeline, independently from raw inputs
    rK, rV, rR, off = O.pool(f64(K), f64(V), f64(Kr), w.doc_len, 64, w.rope_base)
    rK, rV, rR = O.round_bf16(rK), O.round_bf16(rV), O.round_bf16(rR)
    _, ref_doc = O.route(f64(q["Qr"]), rR, off)
    assert np.abs(doc.cpu().numpy() - ref_doc).max() <= 1e-4       # pooled stores may differ by 1 ulp
    gi = idx.cpu().numpy()[0]
    check_topk(gi, ref_doc[0], w.k)
    (_, needle), = C.planted_docs(w)
    assert gi[0] == needle
    mem = O.assemble(gi, off)
    for Tq, o in outs.items():
        ref = O.attend(f64(q["Q"][0, -Tq:]), f64(q["Kloc"][0]), f64(q["Vloc"][0]), rK[mem], rV[mem], w.k,
                       w.rope_base, w.D ** -0.5)
        assert rel_rows(o.cpu().numpy()[0], ref) <= ATT_TOL
