"""The oracle on the synthetic workloads: planted needles and chains must be
recovered (checks the generator's plants and the oracle together), and the
interleave loop must keep its stated invariants."""

import numpy as np
import pytest

from oracle import msa_oracle as O
from synth import workloads as C


def _bf(x):
    return O.bf16_to_f64(x)


def pooled_from_raw(w):
    K = _bf(C.raw_block(w, "K", 0, w.n_tok))
    V = _bf(C.raw_block(w, "V", 0, w.n_tok))
    Kr = _bf(C.raw_block(w, "Kr", 0, w.n_tok))
    Kb, Vb, Rb, off = O.pool(K, V, Kr, w.doc_len, w.chunk, w.rope_base)
    assert np.array_equal(off, w.doc_chunk_off)
    # the pooled cache is stored in bf16
    return O.round_bf16(Kb), O.round_bf16(Vb), O.round_bf16(Rb)


def test_tiny_corpus_needle_retrieved():
    w = C.workload("tiny-32K")
    Kb, Vb, Rb = pooled_from_raw(w)
    q = C.queries(w)
    ch, doc = O.route(_bf(q["Qr"]), Rb, w.doc_chunk_off)
    idx, sc = O.topk(doc, w.k)
    (b, d), = C.planted_docs(w)
    assert idx[0, 0] == d
    assert doc[0, d] > 0.2 and np.sort(doc[0])[-2] < doc[0, d] - 0.05


def test_1M_corpus_needles_retrieved():
    w = C.workload("1M")
    Rb = _bf(C.krbar_block(w, 0, 0, w.n_chunks))
    q = C.queries(w)
    ch, doc = O.route(_bf(q["Qr"]), Rb, w.doc_chunk_off)
    idx, sc = O.topk(doc, w.k)
    for b, d in C.planted_docs(w):
        assert d in idx[b]
        assert doc[b, d] > 0.9


def test_10M_batch16_shape_needles_retrieved_reduced():
    w = C.workload("10M-batch16", n_docs=2000)
    Rb = _bf(C.krbar_block(w, 0, 0, w.n_chunks))
    q = C.queries(w)
    ch, doc = O.route(_bf(q["Qr"]), Rb, w.doc_chunk_off)
    idx, _ = O.topk(doc, w.k)
    for b, d in C.planted_docs(w):
        assert idx[b, 0] == d


def test_interleave_chain_recovered_reduced():
    w = C.workload("10M-interleave", n_docs=300)
    Kb, Vb, Rb = pooled_from_raw(w)
    q = C.queries(w)
    Qr, Q, Kl, Vl = (_bf(q[x]) for x in ("Qr", "Q", "Kloc", "Vloc"))
    for b, ch in enumerate(C.chains(w)):
        res = O.interleave(Qr[b], Rb, Kb, Vb, w.doc_chunk_off, w.k, w.rounds, Q[b], Kl[b], Vl[b],
                           w.rope_base, w.D ** -0.5)
        assert ch["A"] in res[0]["top_idx"]
        assert ch["B"] in res[1]["top_idx"]
        assert ch["C"] in res[2]["top_idx"]
        allr = res[-1]["retrieved"]
        assert len(allr) == len(set(allr)) == w.k * w.rounds
        # the first interleave round is the single-step route + top-k
        _, doc1 = O.route(Qr[b][None], Rb, w.doc_chunk_off)
        i1, _ = O.topk(doc1, w.k)
        assert list(i1[0]) == list(res[0]["top_idx"])
        # later rounds route with the original rows plus the retrieved chunks' router keys
        nrows = w.T + sum(int(w.doc_n_chunks[d]) for d in res[0]["top_idx"])
        assert res[1]["rows"].shape[0] == nrows
        # excluded documents score -inf
        assert np.all(res[1]["doc_scores"][res[0]["top_idx"]] == -np.inf)
