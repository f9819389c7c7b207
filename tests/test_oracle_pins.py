"""Pins for the oracle: closed forms, hand-worked examples, invariants, library
routines in special cases and brute force on tiny inputs.

Each test pins the oracle to something other than itself, chosen so that a
plausible slip (a dropped term, a sign, a transposed operand, a wrong axis or
index) fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import bruteforce as bf
from oracle import msa_oracle as O
from synth import splitmix as sm

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))
BASE = 1.0e6


def rng(seed=0):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- bf16 round
def test_round_bf16_ties_and_known_values():
    one = 1.0
    assert O.round_bf16(one + 2 ** -8) == 1.0                    # tie -> even (1.0)
    assert O.round_bf16(one + 3 * 2 ** -8) == 1.0 + 2 ** -6      # tie -> even (mantissa 2)
    assert O.round_bf16(one + 2 ** -8 + 2 ** -20) == 1.0 + 2 ** -7
    assert O.round_bf16(-(one + 2 ** -8)) == -1.0
    assert O.round_bf16(0.0) == 0.0


def test_round_bf16_matches_independent_generator_rounding():
    # synth rounds through round-to-odd float32; oracle rounds the frexp mantissa
    x = rng(1).standard_normal(200000) * np.exp(rng(2).uniform(-20, 20, 200000))
    a = O.f64_to_bf16_bits(x)
    b = sm.f64_to_bf16_bits(x)
    assert np.array_equal(a, b)


# ----------------------------------------------------------------------- RoPE
def test_rope_golden():
    g = GOLD["rope_d4"]
    for c in g["cases"]:
        got = O.rope(np.array(c["x"], float), c["pos"], g["base"])
        np.testing.assert_allclose(got, c["expect"], rtol=0, atol=1e-14)


def test_rope_identity_norm_composition_relativity():
    x = rng(3).standard_normal((5, 128))
    np.testing.assert_array_equal(O.rope(x, 0, BASE), x)
    y = O.rope(x, np.arange(5) * 97, BASE)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    np.testing.assert_allclose(O.rope(O.rope(x, 17, BASE), 40, BASE), O.rope(x, 57, BASE), atol=1e-12)
    q, k = x[0], x[1]
    d1 = O.rope(q, 300, BASE) @ O.rope(k, 120, BASE)
    d2 = O.rope(q, 1300, BASE) @ O.rope(k, 1120, BASE)
    assert abs(d1 - d2) < 1e-10
    # pairing: dimension i only mixes with i + D/2
    e = np.zeros(128); e[5] = 1.0
    r = O.rope(e, 11, BASE)
    assert set(np.flatnonzero(np.abs(r) > 1e-15)) <= {5, 69}


def test_rope_bruteforce():
    x = rng(4).standard_normal((3, 16))
    for p in (0, 1, 9, 1234):
        for row in x:
            np.testing.assert_allclose(O.rope(row, p, BASE), bf.rope_vec(list(row), p, BASE), atol=1e-13)


# -------------------------------------------------------------------- pooling
def test_pool_golden_partial_chunk():
    g = GOLD["pool_partial_chunk"]
    K = np.array(g["K"], float); V = np.array(g["V"], float)
    Kb, Vb, Rb, off = O.pool(K, V, V, g["doc_len"], g["chunk"], g["base"])
    np.testing.assert_allclose(Vb, g["expect_V"], atol=1e-15)
    np.testing.assert_allclose(Rb, g["expect_V"], atol=1e-15)
    np.testing.assert_allclose(Kb, g["expect_K"], atol=1e-15)
    assert list(off) == [0, 2, 3]


def test_pool_constant_mean_linearity_avgpool():
    r = rng(5)
    L = [130, 64, 1, 200]
    n = sum(L)
    V = r.standard_normal((n, 2, 8)); Kr = r.standard_normal((n, 2, 8)); K = r.standard_normal((n, 2, 8))
    # constant chunk -> that constant
    Vc = np.broadcast_to(np.arange(16.0).reshape(1, 2, 8), (n, 2, 8))
    _, Vb, _, off = O.pool(K, Vc, Kr, L, 64, BASE)
    assert np.all(Vb == np.arange(16.0).reshape(1, 2, 8))
    # chunk >= doc length -> per-document mean
    _, Vb, Rb, off = O.pool(K, V, Kr, L, 512, BASE)
    t = np.concatenate([[0], np.cumsum(L)])
    for d in range(len(L)):
        np.testing.assert_allclose(Vb[d], V[t[d]:t[d + 1]].mean(axis=0), rtol=1e-13)
    # linearity in V and Kr
    V2 = r.standard_normal((n, 2, 8))
    a = O.pool(K, V, Kr, L, 64, BASE)[1]; b = O.pool(K, V2, Kr, L, 64, BASE)[1]
    c = O.pool(K, 2 * V - 3 * V2, Kr, L, 64, BASE)[1]
    np.testing.assert_allclose(c, 2 * a - 3 * b, atol=1e-12)
    # full chunks of an unrotated tensor equal torch avg_pool1d over the document
    Kb, Vb, Rb, off = O.pool(K, V, Kr, L, 64, BASE)
    doc0 = torch.from_numpy(V[:128].reshape(128, 16).T.copy())[None]       # [1, C, L]
    ap = torch.nn.functional.avg_pool1d(doc0, 64, 64)[0].T.numpy().reshape(2, 2, 8)
    np.testing.assert_allclose(Vb[:2], ap, atol=1e-13)
    # partial trailing chunk of doc 0: tokens 128..129 only
    np.testing.assert_allclose(Vb[2], V[128:130].mean(axis=0), atol=1e-14)
    assert list(off) == [0, 3, 4, 5, 9]


def test_pool_rope_positions_restart_per_document():
    # same raw K in two documents -> same pooled Kbar (positions restart at 0)
    r = rng(6)
    Kdoc = r.standard_normal((70, 2, 8))
    K = np.concatenate([Kdoc, Kdoc]); V = np.zeros_like(K)
    Kb, _, _, _ = O.pool(K, V, V, [70, 70], 64, BASE)
    np.testing.assert_allclose(Kb[0:2], Kb[2:4], atol=1e-14)
    # and the first chunk differs from the unrotated mean (rotation really applied)
    assert np.abs(Kb[0] - Kdoc[:64].mean(axis=0)).max() > 1e-3


def test_pool_bruteforce():
    r = rng(7)
    L = [5, 3, 8]
    n = sum(L)
    K, V, Kr = (r.standard_normal((n, 2, 4)) for _ in range(3))
    Kb, Vb, Rb, _ = O.pool(K, V, Kr, L, 3, 100.0)
    bK, bV, bR = bf.pool(K.tolist(), V.tolist(), Kr.tolist(), L, 3, 100.0)
    np.testing.assert_allclose(Kb, bK, atol=1e-13)
    np.testing.assert_allclose(Vb, bV, atol=1e-13)
    np.testing.assert_allclose(Rb, bR, atol=1e-13)


# ----------------------------------------------------- router-key encoding
def test_pool_means_equals_pool_and_native():
    """The whole-corpus chunk means (numpy and C) against the pinned pooling: the V and K_r outputs
    of O.pool on random bf16 rows with partial chunks and one-token documents, bit for bit."""
    from oracle import native as ON
    r = rng(31)
    lens = [1, 64, 65, 130, 7, 200, 63, 128]
    n = int(sum(lens))
    bits = sm.normal_bf16(31, 5, 0, 0, n * 2 * 16).reshape(n, 2, 16)
    X = O.bf16_to_f64(bits)
    _, Vb, Rb, off = O.pool(r.standard_normal((n, 2, 16)), X, X, lens, 64, 1e6)
    M = O.pool_means(X, lens, 64)
    np.testing.assert_array_equal(M, Vb)
    np.testing.assert_array_equal(M, Rb)
    np.testing.assert_array_equal(ON.pool_means_bf16(bits, lens, 64), M)
    assert M.shape[0] == off[-1] == 1 + 1 + 2 + 3 + 1 + 4 + 1 + 2
    # constant rows pool to that constant; a one-token document is its token
    c = np.full((n, 2, 16), 0.375)
    np.testing.assert_array_equal(O.pool_means(c, lens, 64), np.full((int(off[-1]), 2, 16), 0.375))
    np.testing.assert_array_equal(M[0], X[0])


def test_encode_one_hot_closed_form():
    # one-hot hidden states select columns of W: K_r,t = W[:, i_t]; chunk means by hand
    W = np.array([[1.0, 2.0, 3.0], [4.0, 5.0, 6.0]])            # [H*D = 2, d_model = 3]
    hidden = np.eye(3)[[0, 2, 1, 0]]                              # tokens e0, e2, e1 | e0
    out, off = O.encode_router_keys(hidden, W, [3, 1], 2, 1, 2)
    np.testing.assert_array_equal(out.reshape(3, 2), [[2.0, 5.0], [2.0, 5.0], [1.0, 4.0]])
    assert list(off) == [0, 2, 3]


def test_encode_identity_projection_is_router_key_pooling():
    r = rng(40)
    L = [130, 64, 1, 77]
    H, D = 2, 8
    hid = r.standard_normal((sum(L), H * D))
    out, off = O.encode_router_keys(hid, np.eye(H * D), L, 64, H, D)
    K = r.standard_normal((sum(L), H, D))
    _, _, Rb, off2 = O.pool(K, K, hid.reshape(-1, H, D), L, 64, BASE)
    np.testing.assert_allclose(out, Rb, atol=1e-14)
    assert np.array_equal(off, off2)


def test_encode_bruteforce():
    r = rng(41)
    L = [5, 3, 7]
    hid = r.standard_normal((sum(L), 6)); W = r.standard_normal((4, 6))
    out, _ = O.encode_router_keys(hid, W, L, 3, 2, 2)
    ref = bf.encode_router_keys(hid.tolist(), W.tolist(), L, 3, 2, 2)
    np.testing.assert_allclose(out, ref, atol=1e-13)


def test_encode_torch_linear_avgpool_and_pool_first():
    r = rng(42)
    L = [192, 100]
    H, D, dm = 2, 4, 24
    hid = r.standard_normal((sum(L), dm)); W = r.standard_normal((H * D, dm))
    out, off = O.encode_router_keys(hid, W, L, 64, H, D)
    # full chunks: torch Linear (no bias) then avg_pool1d over the first document
    kr = torch.nn.functional.linear(torch.from_numpy(hid[:192]), torch.from_numpy(W))       # [192, H*D]
    ap = torch.nn.functional.avg_pool1d(kr.T[None], 64, 64)[0].T.numpy()                    # [3, H*D]
    np.testing.assert_allclose(out[:3].reshape(3, H * D), ap, atol=1e-12)
    # the projection is linear: projecting each chunk's mean hidden state gives the same keys
    t = 0
    for d, Ld in enumerate(L):
        for j in range(int(off[d + 1] - off[d])):
            a, b = t + 64 * j, t + min(64 * (j + 1), Ld)
            np.testing.assert_allclose(out[off[d] + j].ravel(), hid[a:b].mean(axis=0) @ W.T, atol=1e-12)
        t += Ld


# ------------------------------------------------------- routing backward
def _route_loss(Qr, Kb, off, G):
    return float((O.route(Qr, Kb, off)[1] * G).sum())


def test_route_backward_finite_differences():
    # L = sum_d G_d * doc_score_d; central differences in fp64 on well-separated maxima
    r = rng(60)
    Qr = r.standard_normal((2, 5, 2, 6)); Kb = r.standard_normal((9, 2, 6))
    off = np.array([0, 3, 4, 9]); G = r.standard_normal((2, 3))
    dQ, dK, sel = O.route_backward(Qr, Kb, off, G)
    eps = 1e-6
    num = np.zeros_like(Qr)
    for idx in np.ndindex(Qr.shape):
        a = Qr.copy(); a[idx] += eps
        c = Qr.copy(); c[idx] -= eps
        num[idx] = (_route_loss(a, Kb, off, G) - _route_loss(c, Kb, off, G)) / (2 * eps)
    np.testing.assert_allclose(dQ, num, atol=1e-7)
    numK = np.zeros_like(Kb)
    for idx in np.ndindex(Kb.shape):
        a = Kb.copy(); a[idx] += eps
        c = Kb.copy(); c[idx] -= eps
        numK[idx] = (_route_loss(Qr, a, off, G) - _route_loss(Qr, c, off, G)) / (2 * eps)
    # dK holds one row per (query, document): scatter it onto the selected chunks
    dense = np.zeros_like(Kb)
    for b in range(2):
        for d in range(3):
            dense[sel[b, d, 0]] += dK[b, d]
    np.testing.assert_allclose(dense, numK, atol=1e-7)


def test_route_backward_torch_autograd():
    r = rng(61)
    Qr = r.standard_normal((1, 7, 3, 8)); Kb = r.standard_normal((12, 3, 8))
    off = np.array([0, 5, 6, 12]); G = r.standard_normal((1, 3))
    q = torch.tensor(Qr, requires_grad=True); k = torch.tensor(Kb, requires_grad=True)
    cos = torch.nn.functional.cosine_similarity(q[0][:, None], k[None], dim=-1).mean(-1)   # [T, n_chunks]
    chunk = cos.max(dim=0).values
    doc = torch.stack([chunk[off[d]:off[d + 1]].max() for d in range(3)])
    (doc * torch.tensor(G[0])).sum().backward()
    dQ, dK, sel = O.route_backward(Qr, Kb, off, G)
    np.testing.assert_allclose(dQ, q.grad.numpy(), atol=1e-12)
    dense = np.zeros_like(Kb)
    for d in range(3):
        dense[sel[0, d, 0]] += dK[0, d]
    np.testing.assert_allclose(dense, k.grad.numpy(), atol=1e-12)


def test_route_backward_ties_exclusion_zero_vectors():
    H, D = 1, 2
    Kb = np.array([[[1.0, 0.0]], [[1.0, 0.0]], [[0.0, 0.0]]])          # chunks 0 and 1 tie, chunk 2 is zero
    Qr = np.array([[[[1.0, 0.0]], [[2.0, 0.0]]]])                       # tokens 0 and 1 tie (same direction)
    off = np.array([0, 2, 3])
    dQ, dK, sel = O.route_backward(Qr, Kb, off, np.array([[1.0, 5.0]]))
    assert sel[0, 0].tolist() == [0, 0]                                 # first chunk, first token
    assert np.all(dK[0, 1] == 0) and sel[0, 1].tolist() == [2, 0]       # zero key: no gradient
    # q^ = k^: the cosine is at its maximum, so the gradient vanishes
    assert np.allclose(dQ, 0.0) and np.allclose(dK, 0.0)
    _, _, sel = O.route_backward(Qr, Kb, off, np.array([[1.0, 5.0]]), exclude=np.array([[True, False]]))
    assert sel[0, 0].tolist() == [-1, -1]


# ------------------------------------------------------------ store updates
def _store_of(docs):
    """An independent construction: a store built from scratch from a list of per-document row blocks."""
    rows = np.concatenate(docs) if docs else np.zeros((0, 2, 3))
    return rows, O.chunk_offsets([len(d) for d in docs], 1)


def test_store_delete_equals_rebuild_and_ids():
    r = rng(50)
    docs = [r.standard_normal((n, 2, 3)) for n in (3, 1, 4, 2, 5)]
    rows, off = _store_of(docs)
    keep = np.array([1, 0, 1, 1, 0], bool)
    out, off_out, new_id = O.store_delete(rows, off, keep)
    ref_rows, ref_off = _store_of([docs[0], docs[2], docs[3]])
    assert np.array_equal(out, ref_rows) and np.array_equal(off_out, ref_off)
    assert new_id.tolist() == [0, -1, 1, 2, -1]
    # keep everything: identity; keep nothing: empty store
    out, off_out, new_id = O.store_delete(rows, off, np.ones(5, bool))
    assert np.array_equal(out, rows) and np.array_equal(off_out, off) and new_id.tolist() == [0, 1, 2, 3, 4]
    out, off_out, new_id = O.store_delete(rows, off, np.zeros(5, bool))
    assert out.shape == (0, 2, 3) and off_out.tolist() == [0] and (new_id == -1).all()


def test_store_append_then_delete_round_trip():
    r = rng(51)
    docs = [r.standard_normal((n, 2, 3)) for n in (2, 6, 1)]
    more = [r.standard_normal((n, 2, 3)) for n in (4, 3)]
    rows, off = _store_of(docs)
    mrows, moff = _store_of(more)
    a_rows, a_off = O.store_append(rows, off, mrows, moff)
    ref_rows, ref_off = _store_of(docs + more)
    assert np.array_equal(a_rows, ref_rows) and np.array_equal(a_off, ref_off)
    back, back_off, _ = O.store_delete(a_rows, a_off, np.array([1, 1, 1, 0, 0], bool))
    assert np.array_equal(back, rows) and np.array_equal(back_off, off)
    # deleting from the middle and appending again keeps routing positions consistent
    mid, mid_off, ids = O.store_delete(a_rows, a_off, np.array([1, 0, 1, 1, 1], bool))
    assert np.array_equal(mid[mid_off[ids[3]]:mid_off[ids[3] + 1]], more[0])


# -------------------------------------------------------------------- routing
def test_route_golden():
    g = GOLD["route_two_docs"]
    off = np.concatenate([[0], np.cumsum(g["doc_chunks"])])
    ch, doc = O.route(np.array(g["Qr"], float), np.array(g["Krbar"], float), off)
    np.testing.assert_allclose(ch, g["expect_chunk"], atol=1e-15)
    np.testing.assert_allclose(doc, g["expect_doc"], atol=1e-15)


def _rand_route_case(seed, B=2, T=5, H=3, D=16, ndocs=7):
    r = rng(seed)
    n_ch = r.integers(1, 4, ndocs)
    off = np.concatenate([[0], np.cumsum(n_ch)])
    Qr = r.standard_normal((B, T, H, D))
    Kb = r.standard_normal((int(off[-1]), H, D))
    return Qr, Kb, off, n_ch


def test_route_bruteforce_and_exclusion():
    Qr, Kb, off, n_ch = _rand_route_case(8)
    excl = np.zeros((2, 7), bool); excl[1, 3] = True
    ch, doc = O.route(Qr, Kb, off, excl)
    bch, bdoc = bf.route(Qr.tolist(), Kb.tolist(), list(n_ch), excl.tolist())
    np.testing.assert_allclose(ch, bch, atol=1e-13)
    np.testing.assert_allclose(doc, bdoc, atol=1e-13)
    assert doc[1, 3] == -np.inf and np.isfinite(doc[0, 3])


def test_route_empty_documents_score_minus_inf():
    """Documents without chunks (equal consecutive offsets): leading, in the middle, several in a
    row and trailing.  Each scores -inf and the others keep their own chunks' maximum, as the
    brute-force scan gives; removing the empty documents leaves the others' scores unchanged."""
    r = rng(21)
    n_ch = np.array([0, 2, 0, 0, 3, 1, 0, 2, 0, 0])
    off = np.concatenate([[0], np.cumsum(n_ch)])
    Qr = r.standard_normal((2, 4, 3, 8))
    Kb = r.standard_normal((int(off[-1]), 3, 8))
    excl = np.zeros((2, len(n_ch)), bool); excl[0, 4] = True; excl[1, 2] = True
    ch, doc = O.route(Qr, Kb, off, excl)
    bch, bdoc = bf.route(Qr.tolist(), Kb.tolist(), list(n_ch), excl.tolist())
    np.testing.assert_allclose(ch, bch, atol=1e-13)
    np.testing.assert_array_equal(np.isfinite(doc), np.isfinite(bdoc))
    np.testing.assert_allclose(doc[np.isfinite(doc)], np.asarray(bdoc)[np.isfinite(doc)], atol=1e-13)
    assert np.all(doc[:, n_ch == 0] == -np.inf)
    ne = np.flatnonzero(n_ch > 0)
    _, doc_ne = O.route(Qr, Kb, np.concatenate([[0], np.cumsum(n_ch[ne])]), excl[:, ne])
    np.testing.assert_array_equal(doc[:, ne], doc_ne)
    # each non-empty document's score is the max of its own chunk scores, by explicit slicing
    for d in ne:
        if not excl[1, d]:
            assert doc[1, d] == ch[1, off[d]:off[d + 1]].max()


def test_route_invariants():
    Qr, Kb, off, _ = _rand_route_case(9, B=1, T=4, H=8, D=32, ndocs=9)
    ch, doc = O.route(Qr, Kb, off)
    assert np.all(np.abs(ch) <= 1 + 1e-12)
    # scaling rows by powers of two (exact) leaves every score unchanged
    sc = 2.0 ** rng(10).integers(-6, 7, size=(Kb.shape[0], 8, 1))
    ch2, doc2 = O.route(Qr * 4.0, Kb * sc, off)
    np.testing.assert_allclose(ch2, ch, atol=1e-14)
    # a router row identical to a chunk in every head scores exactly 1 there
    Q1 = Qr.copy(); Q1[0, 2] = Kb[5]
    ch3, _ = O.route(Q1, Kb, off)
    assert abs(ch3[0, 5] - 1.0) < 1e-14
    # permuting documents permutes document scores
    n_docs = len(off) - 1
    perm = rng(11).permutation(n_docs)
    blocks = [Kb[off[d]:off[d + 1]] for d in perm]
    Kp = np.concatenate(blocks)
    offp = np.concatenate([[0], np.cumsum([len(b) for b in blocks])])
    _, docp = O.route(Qr, Kp, offp)
    np.testing.assert_allclose(docp[0], doc[0, perm], atol=1e-14)
    # head mean, not head sum: H identical heads give the single-head cosine
    qs = rng(12).standard_normal((1, 1, 1, 32)); ks = rng(13).standard_normal((3, 1, 32))
    c1, _ = O.route(qs, ks, [0, 3])
    c8, _ = O.route(np.repeat(qs, 8, axis=2), np.repeat(ks, 8, axis=1), [0, 3])
    np.testing.assert_allclose(c8, c1, atol=1e-14)


def test_route_reduces_to_torch_cosine_similarity():
    r = rng(14)
    q = r.standard_normal((1, 1, 1, 64)); k = r.standard_normal((10, 1, 64))
    ch, _ = O.route(q, k, np.arange(11))
    ref = torch.nn.functional.cosine_similarity(torch.from_numpy(q[0, 0]), torch.from_numpy(k[:, 0]), dim=-1)
    np.testing.assert_allclose(ch[0], ref.numpy(), atol=1e-14)


def test_route_zero_vectors_score_zero():
    q = np.zeros((1, 1, 2, 4)); q[0, 0, 1] = [1, 0, 0, 0]
    k = np.zeros((1, 2, 4)); k[0, 0] = [1, 1, 1, 1]; k[0, 1] = [2, 0, 0, 0]
    ch, _ = O.route(q, k, [0, 1])
    assert ch[0, 0] == 0.5          # head 0 has a zero query -> 0; head 1 -> 1; mean 0.5


def test_route_token_max_not_mean():
    # two tokens, one matching: the chunk score is the max over tokens
    k = rng(15).standard_normal((1, 2, 8))
    q = np.stack([k[0], -k[0]])[None]
    ch, _ = O.route(q, k, [0, 1])
    assert abs(ch[0, 0] - 1.0) < 1e-14


# ---------------------------------------------------------------------- top-k
def test_topk_golden_ties():
    g = GOLD["topk_ties"]
    idx, sc = O.topk(np.array([g["scores"]]), g["k"])
    assert list(idx[0]) == g["expect"]


def test_topk_vs_sorted_torch_and_bruteforce():
    r = rng(16)
    s = np.round(r.standard_normal((3, 50)), 1)      # many ties
    for b in range(3):
        ref = sorted(range(50), key=lambda i: (-s[b, i], i))[:9]
        idx, _ = O.topk(s[b:b + 1], 9)
        assert list(idx[0]) == ref
        assert list(idx[0]) == bf.topk(list(s[b]), 9)
    d = r.standard_normal((2, 40))
    idx, sc = O.topk(d, 7)
    tv, ti = torch.topk(torch.from_numpy(d), 7, dim=1)
    assert np.array_equal(idx, ti.numpy())
    np.testing.assert_array_equal(sc, tv.numpy())
    # -inf (excluded) documents come last, lowest id first
    e = np.array([[-np.inf, 0.3, -np.inf, 0.1]])
    assert list(O.topk(e, 4)[0][0]) == [1, 3, 0, 2]


def test_assemble_rank_order():
    off = np.array([0, 2, 5, 6])
    assert list(O.assemble([2, 0, 1], off)) == [5, 0, 1, 2, 3, 4]


# ------------------------------------------------------------------ attention
def test_attend_golden():
    g = GOLD["attend_tiny"]
    for c in g["cases"]:
        o = O.attend(np.array(g["Q"], float), np.array(g["Kloc"], float), np.array(g["Vloc"], float),
                     np.array(g["Kmem"], float), np.array(g["Vmem"], float), c["offset"], g["base"], g["scale"])
        np.testing.assert_allclose(o, c["expect"], atol=1e-14)


def _att_case(seed, Tq=3, Tl=5, M=4, Hq=4, Hkv=2, D=16):
    r = rng(seed)
    return (r.standard_normal((Tq, Hq, D)), r.standard_normal((Tl, Hkv, D)), r.standard_normal((Tl, Hkv, D)),
            r.standard_normal((M, Hkv, D)), r.standard_normal((M, Hkv, D)))


def test_attend_bruteforce():
    Q, Kl, Vl, Km, Vm = _att_case(17)
    for off in (0, 3):
        o = O.attend(Q, Kl, Vl, Km, Vm, off, 100.0, 0.25)
        b = bf.attend(Q.tolist(), Kl.tolist(), Vl.tolist(), Km.tolist(), Vm.tolist(), off, 100.0, 0.25)
        np.testing.assert_allclose(o, b, atol=1e-12)


def test_attend_invariants():
    Q, Kl, Vl, Km, Vm = _att_case(18, Tq=4, Tl=6, M=5, Hq=8, Hkv=2, D=32)
    o, P = O.attend(Q, Kl, Vl, Km, Vm, 5, BASE, 32 ** -0.5, return_probs=True)
    np.testing.assert_allclose(P.sum(axis=-1), 1.0, atol=1e-13)
    # causal: row i sees local keys j <= (Tl - Tq) + i only
    assert np.all(P[:, 0, 5 + 3:] == 0) and np.all(P[:, 0, 5:5 + 3] > 0)
    # constant V -> that V
    vc = rng(19).standard_normal((1, 2, 32))
    oc = O.attend(Q, Kl, np.broadcast_to(vc, Vl.shape), Km, np.broadcast_to(vc, Vm.shape), 5, BASE, 0.2)
    np.testing.assert_allclose(oc, np.broadcast_to(np.repeat(vc, 4, axis=1), oc.shape), atol=1e-13)
    # permuting memory entries leaves the output unchanged
    p = rng(20).permutation(5)
    np.testing.assert_allclose(O.attend(Q, Kl, Vl, Km[p], Vm[p], 5, BASE, 0.2),
                               O.attend(Q, Kl, Vl, Km, Vm, 5, BASE, 0.2), atol=1e-13)
    # a single dominant logit returns that memory row's V (kv-head 1 serves q-heads 4..7)
    # (dimension 15 of D=32 has frequency 1e6**(-30/32): RoPE barely turns it)
    Km2 = Km.copy(); Km2[3, 1] = 0.0
    Qd = np.zeros_like(Q); Qd[:, 4:, 15] = 1.0
    Km2[3, 1, 15] = 1e4
    od = O.attend(Qd, np.zeros_like(Kl), Vl, Km2, Vm, 0, BASE, 1.0)
    np.testing.assert_allclose(od[0, 4], Vm[3, 1], atol=1e-12)


def test_attend_m0_is_causal_gqa_sdpa_and_offset_free():
    Q, Kl, Vl, Km, Vm = _att_case(21, Tq=4, Tl=7, M=0, Hq=8, Hkv=2, D=32)
    o = O.attend(Q, Kl, Vl, Km[:0], Vm[:0], 0, BASE, 32 ** -0.5)
    # textbook: rotate at positions (Tl-Tq)+i and j, repeat kv heads, bottom-right causal mask
    Qr = O.rope(Q, (3 + np.arange(4))[:, None], BASE)
    Kr = O.rope(Kl, np.arange(7)[:, None], BASE)
    q = torch.from_numpy(Qr).permute(1, 0, 2)[None]
    k = torch.from_numpy(np.repeat(Kr, 4, axis=1)).permute(1, 0, 2)[None]
    v = torch.from_numpy(np.repeat(Vl, 4, axis=1)).permute(1, 0, 2)[None]
    mask = torch.from_numpy(np.arange(7)[None, :] <= (3 + np.arange(4))[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=32 ** -0.5)
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), atol=1e-12)
    # with no memory, shifting the offset changes nothing (RoPE depends on differences)
    o7 = O.attend(Q, Kl, Vl, Km[:0], Vm[:0], 7, BASE, 32 ** -0.5)
    np.testing.assert_allclose(o7, o, atol=1e-11)


def test_attend_offset_matters_with_memory():
    Q, Kl, Vl, Km, Vm = _att_case(22, M=4)
    a = O.attend(Q, Kl, Vl, Km, Vm, 4, BASE, 0.25)
    b = O.attend(Q, Kl, Vl, Km, Vm, 5, BASE, 0.25)
    assert np.abs(a - b).max() > 1e-6


def test_attend_gqa_mapping():
    # q-head h must read kv-head h // (Hq/Hkv): zero one kv head's V and see which q-heads go to 0
    Q, Kl, Vl, Km, Vm = _att_case(23, Hq=8, Hkv=2)
    Vl2, Vm2 = Vl.copy(), Vm.copy()
    Vl2[:, 1] = 0; Vm2[:, 1] = 0
    o = O.attend(Q, Kl, Vl2, Km, Vm2, 2, BASE, 0.25)
    assert np.all(o[:, 4:] == 0) and np.all(np.abs(o[:, :4]).max(axis=-1) > 0)


# ------------------------------------------------------ attention backward
def _attend_loss(G, *args):
    Q, Kl, Vl, Km, Vm, off, base, scale = args
    return float((O.attend(Q, Kl, Vl, Km, Vm, off, base, scale) * G).sum())


def test_attend_backward_finite_differences():
    # L = sum(G * O); central differences of the oracle's own forward, every element of every input
    Q, Kl, Vl, Km, Vm = _att_case(70, Tq=3, Tl=5, M=4, Hq=4, Hkv=2, D=8)
    G = rng(71).standard_normal(Q.shape)
    args = [Q, Kl, Vl, Km, Vm]
    grads = O.attend_backward(Q, Kl, Vl, Km, Vm, 3, 50.0, 0.4, G)
    order = [0, 1, 2, 3, 4]                       # attend_backward returns dQ, dKloc, dVloc, dKmem, dVmem
    eps = 1e-6
    for which, gidx in zip(range(5), order):
        x = args[which]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            a = [y.copy() for y in args]; a[which][idx] += eps
            c = [y.copy() for y in args]; c[which][idx] -= eps
            num[idx] = (_attend_loss(G, *a, 3, 50.0, 0.4) - _attend_loss(G, *c, 3, 50.0, 0.4)) / (2 * eps)
        np.testing.assert_allclose(grads[gidx], num, atol=2e-8, err_msg=f"input {which}")


def test_attend_backward_torch_autograd():
    # an independent forward in torch (textbook masked softmax attention with explicit rotation
    # matrices and repeated kv heads), differentiated by autograd
    Tq, Tl, M, Hq, Hkv, D, off, base, scale = 4, 6, 5, 8, 2, 16, 9, 1e4, 0.3
    Q, Kl, Vl, Km, Vm = _att_case(72, Tq=Tq, Tl=Tl, M=M, Hq=Hq, Hkv=Hkv, D=D)
    G = rng(73).standard_normal(Q.shape)
    t = [torch.tensor(a, requires_grad=True) for a in (Q, Kl, Vl, Km, Vm)]

    def rot_matrix(p):
        R = torch.zeros(D, D, dtype=torch.float64)
        for i in range(D // 2):
            a = p * base ** (-2.0 * i / D)
            R[i, i], R[i, i + D // 2] = np.cos(a), -np.sin(a)
            R[i + D // 2, i], R[i + D // 2, i + D // 2] = np.sin(a), np.cos(a)
        return R

    qr = torch.stack([t[0][i] @ rot_matrix(off + Tl - Tq + i).T for i in range(Tq)])
    kr = torch.stack([t[1][j] @ rot_matrix(off + j).T for j in range(Tl)])
    keys = torch.cat([t[3], kr]).repeat_interleave(Hq // Hkv, dim=1)            # [M+Tl, Hq, D]
    vals = torch.cat([t[4], t[2]]).repeat_interleave(Hq // Hkv, dim=1)
    logits = torch.einsum("ihd,jhd->hij", qr, keys) * scale
    mask = torch.ones(Tq, M + Tl, dtype=torch.bool)
    mask[:, M:] = torch.arange(Tl)[None, :] <= (Tl - Tq + torch.arange(Tq))[:, None]
    P = torch.softmax(logits.masked_fill(~mask, float("-inf")), dim=-1)
    out = torch.einsum("hij,jhd->ihd", P, vals)
    (out * torch.tensor(G)).sum().backward()
    grads = O.attend_backward(Q, Kl, Vl, Km, Vm, off, base, scale, G)
    for g, ref in zip(grads, (t[0], t[1], t[2], t[3], t[4])):
        np.testing.assert_allclose(g, ref.grad.numpy(), atol=1e-11)


def test_attend_backward_closed_forms():
    # one visible key: P = 1, so dV = dO, and dS = P (dP - dP) = 0 gives zero dQ and dK
    Q, Kl, Vl, Km, Vm = _att_case(74, Tq=1, Tl=1, M=0, Hq=2, Hkv=1, D=8)
    G = rng(75).standard_normal(Q.shape)
    dQ, dKl, dVl, dKm, dVm = O.attend_backward(Q, Kl, Vl, Km, Vm, 2, BASE, 0.5, G)
    np.testing.assert_allclose(dVl[0, 0], G[0].sum(axis=0), atol=1e-14)
    assert np.abs(dQ).max() < 1e-14 and np.abs(dKl).max() < 1e-14 and dKm.shape == (0, 1, 8)
    # Q = 0: uniform weights over the n visible keys, so dV_j = sum of dO over the rows that see j, / n;
    # dK = scale dS^T Q = 0; dQrot_i = scale * sum_j (1/n)(dP_ij - mean_j dP_ij) k_j
    Q, Kl, Vl, Km, Vm = _att_case(76, Tq=2, Tl=3, M=2, Hq=1, Hkv=1, D=8)
    Q = np.zeros_like(Q)
    G = rng(77).standard_normal(Q.shape)
    dQ, dKl, dVl, dKm, dVm = O.attend_backward(Q, Kl, Vl, Km, Vm, 0, BASE, 0.5, G)
    assert np.abs(dKl).max() < 1e-14 and np.abs(dKm).max() < 1e-14
    # row 0 sees memory 0, 1 and local 0, 1 (n = 4); row 1 sees all five (n = 5)
    np.testing.assert_allclose(dVm[0, 0], G[0, 0] / 4 + G[1, 0] / 5, atol=1e-14)
    np.testing.assert_allclose(dVl[2, 0], G[1, 0] / 5, atol=1e-14)
    # with Q = 0 the rotation of Q is irrelevant; the gradient of row 1 before un-rotation:
    keys = np.concatenate([Km[:, 0], O.rope(Kl[:, 0], np.arange(3), BASE)])
    vals = np.concatenate([Vm[:, 0], Vl[:, 0]])
    dP = vals @ G[1, 0]
    want = 0.5 * ((dP - dP.mean()) / 5) @ keys
    np.testing.assert_allclose(O.rope(dQ[1:2, 0], np.array([2]), BASE)[0], want, atol=1e-13)


def test_attend_backward_gqa_and_memory_permutation():
    Q, Kl, Vl, Km, Vm = _att_case(78, Tq=3, Tl=4, M=6, Hq=8, Hkv=2, D=16)
    G = rng(79).standard_normal(Q.shape)
    # a kv head collects only its own q-heads: zero the gradient of q-heads 4..7 -> kv head 1 gets nothing
    G2 = G.copy(); G2[:, 4:] = 0
    _, dKl, dVl, dKm, dVm = O.attend_backward(Q, Kl, Vl, Km, Vm, 1, BASE, 0.25, G2)
    for x in (dKl, dVl, dKm, dVm):
        assert np.all(x[:, 1] == 0) and np.abs(x[:, 0]).max() > 0
    # permuting the memory entries permutes their gradients and changes nothing else
    p = rng(80).permutation(6)
    a = O.attend_backward(Q, Kl, Vl, Km, Vm, 1, BASE, 0.25, G)
    b = O.attend_backward(Q, Kl, Vl, Km[p], Vm[p], 1, BASE, 0.25, G)
    for x, y in zip(a[:3], b[:3]):
        np.testing.assert_allclose(x, y, atol=1e-12)
    np.testing.assert_allclose(a[3][p], b[3], atol=1e-12)
    np.testing.assert_allclose(a[4][p], b[4], atol=1e-12)


# ------------------------------------------------------------- attention log-sum-exp
def test_attend_lse_single_key_is_the_scaled_score():
    """One query row, one local key at the same position, no memory: the rotation
    preserves the dot product, so lse = scale * <q, k> exactly (closed form)."""
    r = np.random.default_rng(3)
    q = r.standard_normal((1, 4, 128)); k = r.standard_normal((1, 2, 128))
    lse = O.attend_lse(q, k, np.zeros((0, 2, 128)), 5, 1e6, 0.25)
    for h in range(4):
        assert abs(lse[0, h] - 0.25 * float(q[0, h] @ k[0, h // 2])) < 1e-12


def test_attend_lse_equal_scores_is_log_count():
    """Zero keys give equal scores, so lse of row i is ln(number of visible keys):
    M memory entries + (Tl - Tq) + i + 1 local keys."""
    Tq, Tl, M = 5, 9, 7
    q = np.random.default_rng(4).standard_normal((Tq, 8, 128))
    lse = O.attend_lse(q, np.zeros((Tl, 2, 128)), np.zeros((M, 2, 128)), 3, 1e6, 0.1)
    for i in range(Tq):
        assert np.allclose(lse[i], np.log(M + (Tl - Tq) + i + 1), rtol=0, atol=1e-13)


def test_attend_lse_memory_and_causal_mask_closed_form():
    """rope_offset 0, so row 0 and local key 0 sit at position 0 (no rotation):
    with one memory entry m, row 0's lse = ln(exp(s*<q0,m>) + exp(s*<q0,k0>)) -- the
    memory entry is visible and local key 1 is not (causal)."""
    r = np.random.default_rng(6)
    q = r.standard_normal((2, 2, 128)); kl = r.standard_normal((2, 1, 128)); km = r.standard_normal((1, 1, 128))
    s_ = 0.05
    lse = O.attend_lse(q, kl, km, 0, 1e6, s_)
    for h in range(2):
        a, b = s_ * float(q[0, h] @ km[0, 0]), s_ * float(q[0, h] @ kl[0, 0])
        assert abs(lse[0, h] - np.logaddexp(a, b)) < 1e-12
