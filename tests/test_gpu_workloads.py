"""The path at the workloads' full sizes on the GPU, in the launch
configurations the benchmark uses, against the oracle: every document score,
every query's top-k and every query's attention output (Tq = T and Tq = 1) of
the 1M, 10M batch-16 and 100M-token workloads, and all three interleave rounds
of the 10M-token interleave workload (pooled on the GPU from raw tokens; the
oracle pools every document's router keys itself).  Rules P1-P4 are in
tests/parity.py."""

import sys

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O
from sparse_retrieval_memory_amd import ops
from synth import workloads as C
from synth import native
from synth import splitmix as sm

from tests.parity import (ATT_TOL, GRAD_REL, SCORE_TOL, check_topk, dev_bits, encoded_keys_ok, host_bits,
                          pooled_k_ok, pooled_k_scales, rel_rows)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def announce(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def f32(bits):
    """bf16 bits -> float32 (exact); the oracle widens to float64 block by block."""
    return (np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


class LazyKrbar:
    """The oracle's view of a drawn pooled router-key store: chunk blocks regenerated on the host
    generator when the oracle slices them (float32, exact bf16 values), so a 3.4 GB layer is never
    held whole."""

    def __init__(self, w, layer):
        self.w, self.layer = w, layer
        self.shape = (w.n_chunks, w.H, w.D)

    def __getitem__(self, sl):
        assert isinstance(sl, slice) and sl.step is None
        return f32(C.krbar_block(self.w, self.layer, sl.start, min(sl.stop, self.w.n_chunks)))


def device_krbar(w, layer):
    """The pooled router-key store drawn on the device (same bits as the host generator), plants applied."""
    t = torch.empty((w.n_chunks, w.H, w.D), dtype=torch.int16, device=DEV)
    native.fill_normal_bf16_device(t, w.seed, sm.TID_KRBAR, layer, 0)
    for g, row in C.pooled_plants(w, layer).items():
        t[g].copy_(dev_bits(row))
    return t


def content_store(w):
    """Pinned host content tier [G, 2, H, D]: pooled K and V drawn on the device, copied once."""
    G = w.n_chunks
    st = torch.empty((G, 2, w.H, w.D), dtype=torch.int16, pin_memory=True)
    for j, tid in enumerate((sm.TID_KBAR, sm.TID_VBAR)):
        t = torch.empty((G, w.H, w.D), dtype=torch.int16, device=DEV)
        native.fill_normal_bf16_device(t, w.seed, tid, 0, 0)
        st[:, j].copy_(t)
        del t
    return st


def content_rows(w, chunks):
    """The oracle's copy of the content rows (host generator): K, V [len(chunks), H, D] float32."""
    K = np.stack([C.content_block(w, "K", int(g), int(g) + 1)[0] for g in chunks]) if len(chunks) else \
        np.zeros((0, w.H, w.D), np.uint16)
    V = np.stack([C.content_block(w, "V", int(g), int(g) + 1)[0] for g in chunks]) if len(chunks) else \
        np.zeros((0, w.H, w.D), np.uint16)
    return f32(K), f32(V)


def sample_docs(w, extra, n=2000, seed=1):
    rng = np.random.default_rng(seed)
    lens = w.doc_n_chunks
    s = set(int(x) for x in rng.choice(w.n_docs, size=min(n, w.n_docs), replace=False))
    s |= {int(np.argmin(lens)), int(np.argmax(lens)), 0, w.n_docs - 1}
    s |= set(int(x) for x in extra)
    return np.array(sorted(s))


def fetch_and_attend(w, idx_dev, store_t, q, b_rows=None):
    """Fetch the selected documents' pooled K/V from the pinned tier and attend (Tq = T and Tq = 1)."""
    B = idx_dev.shape[0]
    Mmax = int(w.doc_n_chunks.max()) * w.k
    staging = torch.zeros((B, Mmax, 2, w.H, w.D), dtype=torch.int16, device=DEV)
    ml = ops.fetch_docs(idx_dev.cpu(), store_t, torch.from_numpy(w.doc_chunk_off), staging, Mmax)
    ml_dev = ml.to(DEV)
    outs = {}
    for Tq in (w.Tq, 1):
        outs[Tq] = ops.sparse_attn_decode(dev_bits(q["Q"][:, -Tq:]), dev_bits(q["Kloc"]), dev_bits(q["Vloc"]),
                                          staging, staging[:, :, 1], 2 * w.H * w.D, Mmax, ml_dev, w.k,
                                          w.rope_base)
    torch.cuda.synchronize()
    return {Tq: o.cpu().numpy() for Tq, o in outs.items()}, ml.numpy()


def check_attention(w, q, outs, gpu_idx, batches):
    for b in batches:
        mem = O.assemble(gpu_idx[b], w.doc_chunk_off)
        Km, Vm = content_rows(w, mem)
        for Tq, o in outs.items():
            ref = O.attend(f32(q["Q"][b, -Tq:]), f32(q["Kloc"][b]), f32(q["Vloc"][b]), Km, Vm, w.k, w.rope_base,
                           w.D ** -0.5)
            assert rel_rows(o[b], ref) <= ATT_TOL, (b, Tq)


# ------------------------------------------------------------------ 1M tokens
def test_1M_corpus_full_step():
    """1,000 documents, 16.6K chunks, T = 128, k = 16: every score against the oracle."""
    w = C.workload("1M")
    announce("1M full", w.describe())
    kr = device_krbar(w, 0)
    host_kr = C.krbar_block(w, 0, 0, w.n_chunks)
    q = C.queries(w)
    off = torch.from_numpy(w.doc_chunk_off).to(DEV)
    _, ref_doc = O.route(f32(q["Qr"]), f32(host_kr), w.doc_chunk_off)
    for norms in (None, ops.krbar_inv_norms(kr)):
        doc = ops.route_scores(dev_bits(q["Qr"]), kr, off, krbar_inv_norm=norms)
        assert np.abs(doc.cpu().numpy() - ref_doc).max() <= SCORE_TOL
    idx, sc = ops.topk_docs(doc, w.k)
    gi = idx.cpu().numpy()
    check_topk(gi[0], ref_doc[0], w.k)
    assert np.abs(sc.cpu().numpy()[0] - ref_doc[0, gi[0]]).max() <= SCORE_TOL
    for b, d in C.planted_docs(w):
        assert d in gi[b]
    outs, ml = fetch_and_attend(w, idx, content_store(w), q)
    assert ml[0] == len(O.assemble(gi[0], w.doc_chunk_off))
    check_attention(w, q, outs, gi, [0])


# ----------------------------------------------------------------- 10M tokens
@pytest.mark.timeout(900)
def test_10M_batch16_full_against_oracle():
    """20,000 documents, 165K chunks, 16 queries x 64 tokens (the MFMA-bound shape), in the benchmark's
    launch: msa_route_topk with stored norms over all 16 queries.  Every document score of every query
    (P2), every query's top-16 (P3), every planted needle, and every query's attention output over its
    selected documents (Tq = 64 and Tq = 1, P4)."""
    w = C.workload("10M-batch16")
    announce("10M-batch16 full", w.describe())
    kr = device_krbar(w, 0)
    q = C.queries(w)
    off = torch.from_numpy(w.doc_chunk_off).to(DEV)
    doc, idx, sc = ops.route_topk(dev_bits(q["Qr"]), kr, off, w.k, krbar_inv_norm=ops.krbar_inv_norms(kr))
    gd, gi, gs = doc.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy()
    del kr
    _, ref_doc = O.route(f32(q["Qr"]), LazyKrbar(w, 0), w.doc_chunk_off)
    assert np.abs(gd - ref_doc).max() <= SCORE_TOL
    for b in range(w.B):
        check_topk(gi[b], ref_doc[b], w.k)
        assert np.abs(gs[b] - ref_doc[b, gi[b]]).max() <= SCORE_TOL
    for b, d in C.planted_docs(w):
        assert gi[b, 0] == d
    outs, ml = fetch_and_attend(w, idx, content_store(w), q)
    for b in range(w.B):
        assert ml[b] == len(O.assemble(gi[b], w.doc_chunk_off))
    check_attention(w, q, outs, gi, range(w.B))


# ---------------------------------------------------------------- 100M tokens
def test_100M_layer_route_topk_equals_separate_calls():
    """msa_route_topk, the call the 18-layer step times, on a full 100M-token layer (200,000
    documents, 1.66M chunks, 128 router rows, stored norms, a tenth of the documents excluded):
    document scores, selection and selected scores bit-identical to msa_route_scores followed by
    msa_topk_docs; every planted needle of the layer that is not excluded is selected."""
    w = C.workload("100M-18layer")
    layer = 5
    announce("100M route_topk", layer, w.describe())
    kr = device_krbar(w, layer)
    q = C.queries(w, layer)
    off = torch.from_numpy(w.doc_chunk_off).to(DEV)
    nrm = ops.krbar_inv_norms(kr)
    qr = dev_bits(q["Qr"])
    needles = set(d for _, d in C.planted_docs(w, layer))
    excl = (np.arange(w.n_docs) % 10 == 7).astype(np.uint8)
    excl[list(needles)] = 0
    ex = torch.from_numpy(excl[None]).to(DEV)
    d1, i1, s1 = ops.route_topk(qr, kr, off, w.k, doc_exclude=ex, krbar_inv_norm=nrm)
    d2 = ops.route_scores(qr, kr, off, doc_exclude=ex, krbar_inv_norm=nrm)
    i2, s2 = ops.topk_docs(d2, w.k)
    torch.cuda.synchronize()
    assert np.array_equal(d1.cpu().numpy().view(np.uint32), d2.cpu().numpy().view(np.uint32))
    assert np.array_equal(i1.cpu().numpy(), i2.cpu().numpy())
    assert np.array_equal(s1.cpu().numpy().view(np.uint32), s2.cpu().numpy().view(np.uint32))
    sel = set(int(x) for x in i1.cpu().numpy()[0])
    assert needles <= sel, f"needles {sorted(needles - sel)} not selected"
    assert not any(excl[d] for d in sel)


@pytest.mark.timeout(900)
def test_100M_layer_full_against_oracle():
    """One routed layer of the 100M-token store (200,000 documents, 1.66M chunks, 128 router rows,
    stored norms) in the benchmark's launch (msa_route_topk): all 200,000 document scores against the
    oracle's scan of the whole layer (P2), the top-16 (P3: exact ids where the oracle's rank-16 gap
    is >= 1e-3), every planted needle, and the attention over the GPU's selection at Tq = 128 and
    Tq = 1 (P4)."""
    w = C.workload("100M-18layer")
    layer = 3
    announce("100M layer full", layer, w.describe())
    kr = device_krbar(w, layer)
    q = C.queries(w, layer)
    off = torch.from_numpy(w.doc_chunk_off).to(DEV)
    doc, idx, sc = ops.route_topk(dev_bits(q["Qr"]), kr, off, w.k, krbar_inv_norm=ops.krbar_inv_norms(kr))
    gd, gi, gs = doc.cpu().numpy()[0], idx.cpu().numpy()[0], sc.cpu().numpy()[0]
    del kr
    _, ref_doc = O.route(f32(q["Qr"]), LazyKrbar(w, layer), w.doc_chunk_off)
    ref = ref_doc[0]
    err = np.abs(gd - ref)
    announce("100M layer full: max |score error|", float(err.max()))
    assert err.max() <= SCORE_TOL
    check_topk(gi, ref, w.k)
    assert np.abs(gs - ref[gi]).max() <= SCORE_TOL
    for _, d in C.planted_docs(w, layer):
        assert d in gi
    outs, _ = fetch_and_attend(w, idx, content_store(w), q)
    check_attention(w, q, outs, gi[None], [0])


# ------------------------------------------------------- interleave (10M tokens)
def gpu_pool_corpus(w, slab_tokens=1_000_000):
    """Offline encoding on the device: raw K, V, K_r drawn on the device in document-aligned slabs (chain
    plants applied), pooled into the full (Kbar, Vbar, Krbar) store."""
    G, H, D, E = w.n_chunks, w.H, w.D, w.row_elems
    out = tuple(torch.empty((G, H, D), dtype=torch.int16, device=DEV) for _ in range(3))
    plants = C.raw_plants(w)
    d0 = 0
    while d0 < w.n_docs:
        d1 = int(np.searchsorted(w.doc_tok_off, w.doc_tok_off[d0] + slab_tokens, side="right")) - 1
        d1 = min(max(d1, d0 + 1), w.n_docs)
        t0, t1 = int(w.doc_tok_off[d0]), int(w.doc_tok_off[d1])
        c0, c1 = int(w.doc_chunk_off[d0]), int(w.doc_chunk_off[d1])
        raw = []
        for tid in (sm.TID_K, sm.TID_V, sm.TID_KR):
            t = torch.empty((t1 - t0, H, D), dtype=torch.int16, device=DEV)
            native.fill_normal_bf16_device(t, w.seed, tid, 0, t0 * E)
            raw.append(t)
        for tok, row in plants.items():
            if t0 <= tok < t1:
                raw[2][tok - t0].copy_(dev_bits(row))
        ops.pool_chunks(*raw, torch.from_numpy(w.doc_tok_off[d0:d1 + 1].copy()).to(DEV),
                        torch.from_numpy(w.doc_chunk_off[d0:d1 + 1].copy()).to(DEV), c1 - c0, w.chunk, w.rope_base,
                        out=tuple(o[c0:c1] for o in out))
        torch.cuda.synchronize()
        del raw
        d0 = d1
    return out


def interleave_on_gpu(w, pooled, q, fetch="gather"):
    from sparse_retrieval_memory_amd.interleave import Interleave
    Kb, Vb, Rb = pooled
    store = torch.stack([Kb, Vb], dim=1).cpu().pin_memory()
    il = Interleave(krbar=Rb, doc_chunk_off=torch.from_numpy(w.doc_chunk_off).to(DEV),
                    doc_chunk_off_host=torch.from_numpy(w.doc_chunk_off.copy()), content=store,
                    krbar_inv_norm=ops.krbar_inv_norms(Rb), rope_base=w.rope_base)
    res = il.run(dev_bits(q["Qr"]), dev_bits(q["Q"]), dev_bits(q["Kloc"]), dev_bits(q["Vloc"]), w.k, w.rounds,
                 keep_scores=True, fetch=fetch)
    torch.cuda.synchronize()
    return res


def test_interleave_reduced_against_oracle():
    """300 documents of the interleave corpus: pooled on the GPU from raw tokens, then 3 rounds per query,
    every round against the oracle's own pooling and interleave loop."""
    from tests.parity import bf16_ulp_diff, host_bits, pooled_k_ok, pooled_k_scales
    w = C.workload("10M-interleave", n_docs=300)
    announce("interleave reduced", w.describe())
    pooled = gpu_pool_corpus(w)
    K = O.bf16_to_f64(C.raw_block(w, "K", 0, w.n_tok)); V = O.bf16_to_f64(C.raw_block(w, "V", 0, w.n_tok))
    Kr = O.bf16_to_f64(C.raw_block(w, "Kr", 0, w.n_tok))
    rK, rV, rR, off = O.pool(K, V, Kr, w.doc_len, w.chunk, w.rope_base)
    assert pooled_k_ok(host_bits(pooled[0]), rK, *pooled_k_scales(K, w.doc_len, w.chunk))
    rK, rV, rR = O.round_bf16(rK), O.round_bf16(rV), O.round_bf16(rR)
    assert bf16_ulp_diff(host_bits(pooled[1]), O.f64_to_bf16_bits(rV)).max() <= 1
    assert bf16_ulp_diff(host_bits(pooled[2]), O.f64_to_bf16_bits(rR)).max() <= 1
    q = C.queries(w)
    res = interleave_on_gpu(w, pooled, q)
    # the host-copy assembly gives bit-identical rounds
    res_copy = interleave_on_gpu(w, pooled, q, fetch="copy")
    for r in range(w.rounds):
        assert np.array_equal(res[r].retrieved, res_copy[r].retrieved)
        assert torch.equal(res[r].O, res_copy[r].O)
    for b, ch in enumerate(C.chains(w)):
        ref = O.interleave(f32(q["Qr"][b]), rR, rK, rV, off, w.k, w.rounds, f32(q["Q"][b]), f32(q["Kloc"][b]),
                           f32(q["Vloc"][b]), w.rope_base, w.D ** -0.5)
        for r in range(w.rounds):
            g = res[r].doc_scores.cpu().numpy()[b]
            s = ref[r]["doc_scores"]
            fin = np.isfinite(s)
            assert np.array_equal(fin, np.isfinite(g))                     # the same documents are excluded
            assert np.abs(g[fin] - s[fin]).max() <= 1e-4                   # pooled stores may differ by an ulp
            if check_topk(res[r].top_idx[b], s, w.k):
                break      # an admissible different set (gap < 1e-3): later rounds no longer share inputs
            assert rel_rows(res[r].O.cpu().numpy()[b], ref[r]["O"]) <= ATT_TOL
        assert ch["A"] in res[0].top_idx[b] and ch["B"] in res[1].top_idx[b] and ch["C"] in res[2].top_idx[b]


def oracle_krbar_corpus(w, slab_tokens=1_000_000):
    """The oracle's pooled router keys of every document: chunk means of the raw K_r (regenerated on the
    host in document-aligned slabs, chain plants applied) in float64, rounded to bf16; float64 [G, H, D]."""
    from oracle import native as ON
    out = np.empty((w.n_chunks, w.H, w.D))
    d0 = 0
    while d0 < w.n_docs:
        d1 = int(np.searchsorted(w.doc_tok_off, w.doc_tok_off[d0] + slab_tokens, side="right")) - 1
        d1 = min(max(d1, d0 + 1), w.n_docs)
        t0, t1 = int(w.doc_tok_off[d0]), int(w.doc_tok_off[d1])
        c0, c1 = int(w.doc_chunk_off[d0]), int(w.doc_chunk_off[d1])
        out[c0:c1] = O.round_bf16(ON.pool_means_bf16(C.raw_block(w, "Kr", t0, t1), w.doc_len[d0:d1], w.chunk))
        announce("oracle router-key pooling: documents", d0, "..", d1 - 1, "of", w.n_docs)
        d0 = d1
    return out


class OracleContent:
    """The oracle's pooled content rows (rotated K, V; rounded to bf16), pooled per document from the raw
    tokens when first asked for.  ``K[idx]`` / ``V[idx]`` take arrays of global chunk ids."""

    class _View:
        def __init__(self, owner, j):
            self.owner, self.j = owner, j

        def __getitem__(self, idx):
            return self.owner.rows(np.asarray(idx, dtype=np.int64), self.j)

    def __init__(self, w):
        self.w, self.cache = w, {}
        self.K, self.V = OracleContent._View(self, 0), OracleContent._View(self, 1)

    def doc(self, d):
        if d not in self.cache:
            w = self.w
            t0, t1 = int(w.doc_tok_off[d]), int(w.doc_tok_off[d + 1])
            K, V, Kr = (O.bf16_to_f64(C.raw_block(w, x, t0, t1)) for x in ("K", "V", "Kr"))
            pk, pv, _, _ = O.pool(K, V, Kr, [t1 - t0], w.chunk, w.rope_base)
            m, n = pooled_k_scales(K, [t1 - t0], w.chunk)
            self.cache[d] = (O.round_bf16(pk), O.round_bf16(pv), pk, m, n)
        return self.cache[d]

    def rows(self, idx, j):
        w = self.w
        if len(idx) == 0:
            return np.zeros((0, w.H, w.D))
        docs = w.doc_of_chunk(idx)
        return np.stack([self.doc(int(d))[j][int(g - w.doc_chunk_off[d])] for g, d in zip(idx, docs)])


@pytest.mark.timeout(1200)
def test_10M_interleave_full_against_oracle():
    """The whole 10M-token interleave workload (20,000 documents, 165K chunks): pooled on the GPU in
    1M-token slabs, then 4 queries x 3 rounds of route -> top-8 -> assemble -> attend.

    P1 on every pooled router key of the corpus (the oracle pools all 10M tokens' K_r itself) and on
    the pooled K and V of the retrieved and sampled documents; then each query's three rounds against
    the oracle's interleave loop over its own pooled store: all 20,000 document scores per round
    (excluded documents -inf on both sides), the top-8 (P3), and the attention output over the
    retrieved documents (P4, rounds until the first admissible different selection); every planted
    3-hop chain recovered hop by hop; no document retrieved twice."""
    from tests.parity import bf16_ulp_diff, host_bits
    w = C.workload("10M-interleave")
    announce("10M interleave full", w.describe())
    pooled = gpu_pool_corpus(w)
    q = C.queries(w)
    res = interleave_on_gpu(w, pooled, q)
    chains = C.chains(w)
    for b, ch in enumerate(chains):
        assert ch["A"] in res[0].top_idx[b], (b, "hop 1")
        assert ch["B"] in res[1].top_idx[b], (b, "hop 2")
        assert ch["C"] in res[2].top_idx[b], (b, "hop 3")
        allr = res[-1].retrieved[b]
        assert len(set(int(x) for x in allr)) == len(allr) == w.k * w.rounds
    Kb, Vb, Rb = (host_bits(t) for t in pooled)
    del pooled
    announce("10M interleave full: oracle pools the router keys of all documents")
    rR = oracle_krbar_corpus(w)
    assert bf16_ulp_diff(Rb, O.f64_to_bf16_bits(rR)).max() <= 1
    content = OracleContent(w)
    extra = [ch[x] for ch in chains for x in ("A", "B", "C")] + [int(d) for d in np.ravel(res[-1].retrieved)]
    for d in sample_docs(w, extra, n=60):
        pk, pv, pk_exact, m, n = content.doc(int(d))
        g0, g1 = int(w.doc_chunk_off[d]), int(w.doc_chunk_off[d + 1])
        assert bf16_ulp_diff(Vb[g0:g1], O.f64_to_bf16_bits(pv)).max() <= 1
        assert pooled_k_ok(Kb[g0:g1], pk_exact, m, n)
    for b in range(w.B):
        announce("10M interleave full: oracle rounds of query", b)
        ref = O.interleave(f32(q["Qr"][b]), rR, content.K, content.V, w.doc_chunk_off, w.k, w.rounds,
                           f32(q["Q"][b]), f32(q["Kloc"][b]), f32(q["Vloc"][b]), w.rope_base, w.D ** -0.5)
        for r in range(w.rounds):
            g = res[r].doc_scores.cpu().numpy()[b]
            s = ref[r]["doc_scores"]
            fin = np.isfinite(s)
            assert np.array_equal(fin, np.isfinite(g)), (b, r)           # the same documents are excluded
            assert np.abs(g[fin] - s[fin]).max() <= 1e-4, (b, r)         # pooled stores may differ by an ulp
            if check_topk(res[r].top_idx[b], s, w.k):
                announce("10M interleave full: admissible different selection", b, r)
                break      # an admissible different set (gap < 1e-3): later rounds no longer share inputs
            assert rel_rows(res[r].O.cpu().numpy()[b], ref[r]["O"]) <= ATT_TOL, (b, r)


# ------------------------------------------------------- router-key encoding
D_MODEL = 2560      # hidden size of the pages' backbone family (Qwen3-4B)


def test_encode_router_keys_10M_slab_sampled_chunks():
    """Router-key encoding of the first ~1M-token slab of the 10M-token corpus (document-aligned,
    hidden states and projection drawn by the generator on the device), checked on sampled chunks
    against the oracle run on the same rows regenerated on the host."""
    w = C.workload("10M-interleave")
    H, D = w.H, w.D
    d1 = int(np.searchsorted(w.doc_tok_off, 1_000_000, side="right")) - 1
    t1, c1 = int(w.doc_tok_off[d1]), int(w.doc_chunk_off[d1])
    announce("encode-10M-slab", d1, t1, c1)
    hid = torch.empty((t1, D_MODEL), dtype=torch.int16, device=DEV)
    native.fill_normal_bf16_device(hid, w.seed, sm.TID_HIDDEN, 0, 0)
    Wd = torch.empty((H * D, D_MODEL), dtype=torch.int16, device=DEV)
    native.fill_normal_bf16_device(Wd, w.seed, sm.TID_WKR, 0, 0)
    out = ops.encode_router_keys(hid, Wd, torch.from_numpy(w.doc_tok_off[:d1 + 1].copy()).to(DEV),
                                 torch.from_numpy(w.doc_chunk_off[:d1 + 1].copy()).to(DEV), c1, H, w.chunk)
    torch.cuda.synchronize()
    del hid
    W = O.bf16_to_f64(C.normal_bf16(w.seed, sm.TID_WKR, 0, 0, H * D * D_MODEL).reshape(H * D, D_MODEL))
    r = np.random.default_rng(3)
    chunks = set(r.choice(c1, 60, replace=False).tolist()) | {0, c1 - 1}
    # plus the partial trailing chunks of a few documents
    for d in r.choice(d1, 8, replace=False):
        chunks.add(int(w.doc_chunk_off[d + 1]) - 1)
    gpu = host_bits(out)
    for g in sorted(chunks):
        d = int(np.searchsorted(w.doc_chunk_off, g, side="right")) - 1
        j = g - int(w.doc_chunk_off[d])
        a = int(w.doc_tok_off[d]) + j * w.chunk
        b = min(a + w.chunk, int(w.doc_tok_off[d + 1]))
        rows = O.bf16_to_f64(C.normal_bf16(w.seed, sm.TID_HIDDEN, 0, a * D_MODEL, (b - a) * D_MODEL)
                             .reshape(b - a, D_MODEL))
        ref, _ = O.encode_router_keys(rows, W, [b - a], w.chunk, H, D)
        mag = (np.abs(rows.mean(axis=0)) @ np.abs(W).T).reshape(ref.shape)
        assert encoded_keys_ok(gpu[g:g + 1], ref, mag), f"chunk {g}"


# ------------------------------------------------------------ store updates
def test_store_delete_100M_layer_sampled():
    """Delete 10% of the documents of one 100M-token routing layer (1.66M chunks, with stored norms): offsets
    and new ids exact against the oracle, moved rows equal to their source rows on sampled documents."""
    w = C.workload("100M-18layer")
    announce("store-delete-100M", w.n_docs, w.n_chunks)
    kr = device_krbar(w, 0)
    nrm = ops.krbar_inv_norms(kr)
    r = np.random.default_rng(9)
    keep = r.random(w.n_docs) >= 0.1
    keep[0] = False
    keep[-1] = True
    off = torch.from_numpy(w.doc_chunk_off).to(DEV)
    kr_o, nrm_o, off_o, ids, counts = ops.store_delete(kr, off, torch.from_numpy(keep.astype(np.uint8)).to(DEV),
                                                       inv_norm=nrm)
    torch.cuda.synchronize()
    _, ref_off, ref_ids = O.store_delete(np.zeros(w.n_chunks, np.int8), w.doc_chunk_off, keep)
    nd, nc = (int(x) for x in counts.cpu())
    assert nd == int(keep.sum()) and nc == int(ref_off[-1])
    assert np.array_equal(off_o.cpu().numpy()[:nd + 1], ref_off)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    for d in list(r.choice(np.flatnonzero(keep), 300, replace=False)) + [w.n_docs - 1]:
        a, b = int(w.doc_chunk_off[d]), int(w.doc_chunk_off[d + 1])
        na = int(ref_off[ref_ids[d]])
        assert torch.equal(kr_o[na:na + b - a], kr[a:b]), f"doc {d}"
        assert torch.equal(nrm_o[na:na + b - a], nrm[a:b]), f"doc {d}"


# ------------------------------------------------ routing backward (100M tokens)
def _doc_decisions(Qr, Krows):
    """The oracle's token scores of one document: (S [T, n], chunk gap, token gap) for P6's tie rule."""
    S = O.head_mean_cosine(Qr, Krows)
    cm = S.max(axis=0)
    g = int(np.argmax(cm))
    gap = lambda v: np.inf if len(v) < 2 else float(np.diff(np.sort(v)[-2:])[0])
    return S, gap(cm), gap(S[:, g])


def test_route_backward_100M_layer_sampled():
    """The routing-score backward over one 100M-token layer (200,000 documents, every one with an
    upstream gradient), in the launch configuration the benchmark times.  On sampled documents:
    the (chunk, token) decision is the oracle's where it is clear by 1e-4 and within 1e-4 of the
    maximum otherwise, and the key gradient is the oracle's for that decision (P6).  On sampled
    tokens: every document that selected the token is checked the same way, and dQr is the
    oracle's sum over exactly those documents."""
    w = C.workload("100M-18layer")
    layer = 3
    announce("route-backward-100M", w.n_docs, w.n_chunks)
    kr = device_krbar(w, layer)
    nrm = ops.krbar_inv_norms(kr)
    q = C.queries(w, layer)
    off = torch.from_numpy(w.doc_chunk_off).to(DEV)
    qr = dev_bits(q["Qr"])
    _, ch = ops.route_scores(qr, kr, off, want_chunk_scores=True, krbar_inv_norm=nrm)
    dDoc = np.random.default_rng(10).standard_normal((1, w.n_docs)).astype(np.float32)
    dQ, dK, sel = ops.route_scores_backward(qr, kr, off, ch, torch.from_numpy(dDoc).to(DEV), krbar_inv_norm=nrm)
    torch.cuda.synchronize()
    dQ, sel = dQ.cpu().numpy()[0], sel.cpu().numpy()[0]
    assert np.all(sel[:, 0] >= 0)                            # every document has a gradient and chunks
    Qr = f32(q["Qr"])[0].astype(np.float64)

    def check_doc(d):
        g0, g1 = int(w.doc_chunk_off[d]), int(w.doc_chunk_off[d + 1])
        K = f32(C.krbar_block(w, layer, g0, g1)).astype(np.float64)
        S, cgap, tgap = _doc_decisions(Qr, K)
        g, t = int(sel[d, 0]) - g0, int(sel[d, 1])
        assert 0 <= g < g1 - g0 and 0 <= t < w.T, f"doc {d}: selection {sel[d]} outside the document"
        if cgap >= 1e-4 and tgap >= 1e-4:
            gr = int(np.argmax(S.max(axis=0)))
            assert (g, t) == (gr, int(np.argmax(S[:, gr]))), f"doc {d}"
        else:
            assert S.max() - S[t, g] <= 1e-4 and S[:, g].max() - S[t, g] <= 1e-4, f"doc {d}"
        return K[g]

    def pair_grads(docs, t):
        """The oracle's gradients of the pairs (token t, each document's selected chunk)."""
        K = np.stack([check_doc(int(d)) for d in docs])
        one = np.arange(len(docs) + 1, dtype=np.int64)
        return O.route_backward(Qr[None, t:t + 1], K, one, dDoc[:, docs].astype(np.float64))

    r = np.random.default_rng(4)
    docs = sample_docs(w, [d for _, d in C.planted_docs(w, layer)], n=300, seed=4)
    for d in docs:
        t = int(sel[d, 1])
        _, rK, _ = pair_grads(np.array([d]), t)
        gpu = dK[0, d].cpu().numpy()
        k64 = np.linalg.norm(f32(C.krbar_block(w, layer, int(sel[d, 0]), int(sel[d, 0]) + 1))[0], axis=-1)
        bound = np.where(k64 > 0, 2 * abs(float(dDoc[0, d])) / w.H / np.where(k64 > 0, k64, 1), 0.0)
        assert np.all(np.abs(gpu - rK[0, 0]) <= GRAD_REL * bound[:, None]), f"dK of doc {d}"
    counts = np.bincount(sel[:, 1], minlength=w.T)
    for t in [int(np.argmax(counts)), int(r.integers(w.T))]:
        Dt = np.flatnonzero(sel[:, 1] == t)
        announce("route-backward-100M token", t, len(Dt))
        rQ, _, _ = pair_grads(Dt, t)
        nq = np.linalg.norm(Qr[t], axis=-1)
        bound = 2 * np.abs(dDoc[0, Dt]).astype(np.float64).sum() / w.H / nq
        assert np.all(np.abs(dQ[t] - rQ[0, 0]) <= GRAD_REL * bound[:, None]), f"dQr of token {t}"
