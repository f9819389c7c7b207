"""The seeded generator: determinism, bit equality of its three implementations
(numpy here, C host here, HIP on the GPU in test_gpu_parity), the table, and
the workloads' stated shapes."""

import numpy as np
import pytest

from synth import workloads as C
from synth import native
from synth import splitmix as sm


def test_splitmix_reference_values():
    # mix64 is a bijection with mix64(0) == 0; stream values are reproducible
    assert sm.mix64_int(0) == 0
    a = sm.raw_u64(7, 3, 1, 10, 5)
    b = sm.raw_u64(7, 3, 1, 12, 3)
    assert np.array_equal(a[2:], b)
    assert int(a[0]) == sm.mix64_int(sm.stream_start(7, 3, 1) + 11 * sm.GOLDEN)


def test_normal_table():
    t = sm.bf16_bits_to_f32(sm.NORMAL_TABLE).astype(np.float64)
    assert t.shape == (65536,)
    assert np.all(np.diff(t) >= 0)
    np.testing.assert_array_equal(t, -t[::-1])
    assert abs(t.mean()) < 1e-12 and abs(t.std() - 1.0) < 2e-3
    assert 4.3 < t.max() < 4.34


def test_streams_independent_and_normal():
    x = sm.normal_f64(1, sm.TID_K, 0, 0, 200000)
    y = sm.normal_f64(1, sm.TID_V, 0, 0, 200000)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    assert abs(np.corrcoef(x, y)[0, 1]) < 0.01


@pytest.mark.skipif(not native.available(), reason="C host generator not built")
def test_host_c_matches_numpy():
    for (s, t, l, st, n) in [(1, 1, 0, 0, 1000), (5, 11, 17, 123456789, 4097), (2**32 - 1, 65535, 65535, 2**40, 333)]:
        assert np.array_equal(native.normal_bf16(s, t, l, st, n), sm.normal_bf16(s, t, l, st, n))


def test_uniform_int_range():
    v = sm.uniform_int(3, sm.TID_LEN, 0, 0, 100000, 64, 936)
    assert v.min() == 64 and v.max() == 936
    assert abs(v.mean() - 500) < 3


def test_workload_shapes():
    w1 = C.workload("tiny-32K")
    assert (w1.n_docs, w1.n_tok, w1.n_chunks) == (64, 32768, 512)
    w2 = C.workload("1M")
    assert w2.doc_len.min() >= 256 and w2.doc_len.max() <= 1792 and abs(w2.n_tok - 1.0e6) < 0.1e6
    w3 = C.workload("10M-batch16")
    assert w3.doc_len.min() >= 64 and w3.doc_len.max() <= 8192
    assert abs(np.median(w3.doc_len) - 400) < 15 and abs(w3.n_tok - 1.0e7) < 0.5e6
    w4 = C.workload("100M-18layer")
    assert w4.doc_len.min() == 64 and w4.doc_len.max() == 936
    assert abs(w4.n_tok - 1.0e8) < 1e6 and w4.n_layers == 18
    # every document owns ceil(L/64) >= 1 chunks
    for w in (w1, w2, w3, w4):
        assert np.array_equal(np.diff(w.doc_chunk_off), (w.doc_len + 63) // 64)


def test_plants():
    w2 = C.workload("1M")
    nd = C.needles(w2)
    assert len(nd) == 10 and len({d for _, d, _, _ in nd}) == 10 and len({t for *_, t in nd}) == 10
    rows = C.pooled_plants(w2)
    assert len(rows) == 10
    g = next(iter(rows))
    blk = C.krbar_block(w2, 0, g, g + 1)
    assert np.array_equal(blk[0], rows[g])
    w3 = C.workload("10M-batch16")
    assert sorted(b for b, *_ in C.needles(w3)) == list(range(16))
    w5 = C.workload("10M-interleave", n_docs=400)
    ch = C.chains(w5)
    docs = [c[x] for c in ch for x in "ABC"]
    assert len(ch) == 4 and len(set(docs)) == 12
    rp = C.raw_plants(w5)
    assert len(rp) > 0
    t = next(iter(rp))
    assert np.array_equal(C.raw_block(w5, "Kr", t, t + 1)[0], rp[t])
