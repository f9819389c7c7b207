"""Benchmark of the MSA routed step on one MI355X.

Headline workload: a 100M-token memory of 200,000 synthetic documents
(lengths uniform on [64, 936], mean 500), chunk 64 -> 1.66M pooled chunks,
18 routed layers, each with its own HBM-resident Krbar store (bf16, 8 x 128 per
chunk, 61 GB in total) and its own 128-token router query (batch 1).  One step
runs the 18 layers in sequence; a layer is

    scan of all Krbar (msa_route_scan) -> document max + top-16
    (msa_route_select) -> assemble the selected pooled K/V from the pinned host
    tier (one kernel reading the mapped host memory; the ids never leave the
    GPU) -> GQA attention (32 q-heads, 128 query rows, 128 local tokens) over
    [fetched memory ++ local KV].

The scan kernel's own duration is taken live inside the timed steps with HIP
events around the scan of three of the 18 layers of every step; the roofline
is its algorithmic bytes over that duration.  Beside the headline the run
reports every workload's routed step (32K, 1M with rotating store copies, 10M
batch-16, 100M, 10M interleave), the routed decode step (Tq = 1), the scan time
against the memory size (32K .. 100M tokens), the side kernels, and the oracle
on the host per stage and workload on bounded samples.  Inputs are generated
on the device before timing (seeded, synthetic).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_route_100M.json")
SCAN_EVENT_LAYERS = (0, 6, 12)   # layers whose scan is bracketed by events in every timed step


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def code_text(src: str) -> str:
    """Source text with comments, trailing blanks and empty lines removed."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in src.splitlines())
    return "\n".join(ln for ln in lines if ln)


def route_source_hash() -> str:
    """Fingerprint of the scan kernel's code (comment edits leave it unchanged)."""
    h = hashlib.sha256()
    for f in ("route.hip", "msa_internal.h"):
        with open(os.path.join(ROOT, "sparse_retrieval_memory_amd", "csrc", f)) as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def scan_bytes(n_chunks, n_docs, B, T, H=8, D=128) -> int:
    """Algorithmic HBM bytes of one routing scan: the pooled router keys, the document offsets,
    the router rows and the document scores (32 B per memory token per layer at chunk 64)."""
    return n_chunks * H * D * 2 + 8 * (n_docs + 1) + B * T * H * D * 2 + 4 * B * n_docs


def scan_flops(n_chunks, B, T, H=8, D=128) -> float:
    return 2.0 * B * T * H * D * n_chunks


def pct(a):
    a = np.asarray(a, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90)),
            "mean": float(np.mean(a)), "n": int(len(a))}


# ------------------------------------------------------------------------ oracle on the host
def blas_info():
    try:
        from threadpoolctl import threadpool_info
        return [{k: i.get(k) for k in ("internal_api", "version", "num_threads", "threading_layer")}
                for i in threadpool_info()]
    except Exception as e:  # pragma: no cover
        return [{"error": str(e)}]


def cpu_baseline(seconds: float):
    """The oracle (fp64 numpy, as it stands) on the host, per stage and per workload, on bounded samples.
    value: route + top-k memory tokens/s on the 100M-token workload's layer 0 (documents from the start)."""
    from oracle import msa_oracle as O
    from synth import workloads as C
    affinity = len(os.sched_getaffinity(0))
    # BLAS threads: every CPU this process may run on, capped by the thread count the environment sets for
    # the machine's share (OMP_NUM_THREADS)
    cores = min(affinity, int(os.environ.get("OMP_NUM_THREADS", affinity) or affinity))
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(cores)
    except Exception:  # pragma: no cover
        pass
    f64 = O.bf16_to_f64
    stages = {}

    def attend_s(w, q, M, b=0):
        """Oracle attention over M memory entries (drawn content rows), Tq = T and Tq = 1."""
        Km = f64(C.content_block(w, "K", 0, M)) if w.pooled == "direct" else f64(C.normal_bf16(
            w.seed, 20, 0, 0, M * w.H * w.D).reshape(M, w.H, w.D))
        Vm = f64(C.content_block(w, "V", 0, M)) if w.pooled == "direct" else Km
        out = {}
        for Tq in (w.Tq, 1):
            t0 = time.perf_counter()
            O.attend(f64(q["Q"][b, -Tq:]), f64(q["Kloc"][b]), f64(q["Vloc"][b]), Km, Vm, w.k, w.rope_base,
                     w.D ** -0.5)
            out[f"attend_tq{Tq}_s"] = time.perf_counter() - t0
        return out

    # 32K: pool from raw tokens, route, top-k, attend (everything, one query)
    w = C.workload("tiny-32K")
    q = C.queries(w)
    K, V, Kr = (f64(C.raw_block(w, x, 0, w.n_tok)) for x in ("K", "V", "Kr"))
    t0 = time.perf_counter(); _, _, rR, off = O.pool(K, V, Kr, w.doc_len, w.chunk, w.rope_base)
    st = {"pool_s": time.perf_counter() - t0}
    t0 = time.perf_counter(); _, doc = O.route(f64(q["Qr"]), O.round_bf16(rR), off); st["route_s"] = time.perf_counter() - t0
    t0 = time.perf_counter(); O.topk(doc, w.k); st["topk_s"] = time.perf_counter() - t0
    st.update(attend_s(w, q, 32))
    st["sample"] = "whole workload (32,768 tokens, 1 query)"
    stages["tiny-32K"] = st
    del K, V, Kr
    # 1M: route, top-k, attend over the whole store
    w = C.workload("1M")
    q = C.queries(w)
    kr = f64(C.krbar_block(w, 0, 0, w.n_chunks))
    t0 = time.perf_counter(); _, doc = O.route(f64(q["Qr"]), kr, w.doc_chunk_off); st = {"route_s": time.perf_counter() - t0}
    t0 = time.perf_counter(); O.topk(doc, w.k); st["topk_s"] = time.perf_counter() - t0
    st.update(attend_s(w, q, 262))
    st["sample"] = "whole workload (1,000 documents, 1 query)"
    stages["1M"] = st
    # 10M batch-16: 2 of the 16 queries routed over the whole store
    w = C.workload("10M-batch16")
    q = C.queries(w)
    kr = f64(C.krbar_block(w, 0, 0, w.n_chunks))
    t0 = time.perf_counter(); _, doc = O.route(f64(q["Qr"][:2]), kr, w.doc_chunk_off)
    st = {"route_s_per_query": (time.perf_counter() - t0) / 2}
    t0 = time.perf_counter(); O.topk(doc, w.k); st["topk_s_per_query"] = (time.perf_counter() - t0) / 2
    st.update(attend_s(w, q, 133))
    st["sample"] = "queries 0 and 1 of 16 over all 20,000 documents"
    stages["10M-batch16"] = st
    del kr
    # 10M interleave: pooling throughput on a document sample (K with RoPE, V, K_r)
    w = C.workload("10M-interleave")
    d1 = 40
    t1 = int(w.doc_tok_off[d1])
    K, V, Kr = (f64(C.raw_block(w, x, 0, t1)) for x in ("K", "V", "Kr"))
    t0 = time.perf_counter(); O.pool(K, V, Kr, w.doc_len[:d1], w.chunk, w.rope_base)
    pool_s = time.perf_counter() - t0
    stages["10M-interleave"] = {"pool_tokens_per_s": t1 / pool_s,
                                "pool_10M_extrapolated_s": w.n_tok / (t1 / pool_s),
                                "sample": f"pooling of documents 0..{d1 - 1} ({t1} tokens, K, V and K_r)"}
    del K, V, Kr
    # 100M: route + top-k over a bounded slice of layer 0, growing until `seconds` of work
    w = C.workload("100M-18layer")
    q = C.queries(w, 0)
    Qr = f64(q["Qr"])
    d = 1000
    t_route, t_topk, tok_total, docs_done = 0.0, 0.0, 0, 0
    while t_route + t_topk < seconds and docs_done < w.n_docs:
        d1 = min(w.n_docs, docs_done + d)
        g0, g1 = int(w.doc_chunk_off[docs_done]), int(w.doc_chunk_off[d1])
        kr = f64(C.krbar_block(w, 0, g0, g1))
        off = w.doc_chunk_off[docs_done:d1 + 1] - g0
        t0 = time.perf_counter()
        _, doc = O.route(Qr, kr, off)
        t_route += time.perf_counter() - t0
        t0 = time.perf_counter()
        O.topk(doc, min(w.k, d1 - docs_done))
        t_topk += time.perf_counter() - t0
        tok_total += int(w.doc_tok_off[d1] - w.doc_tok_off[docs_done])
        docs_done = d1
        d = min(d * 2, 16000)
    frac = tok_total / w.n_tok
    st = {"route_s_per_layer": t_route / frac, "topk_s_per_layer": t_topk / frac,
          "route_topk_s_18_layers": 18 * (t_route + t_topk) / frac}
    st.update(attend_s(w, q, 133))
    st["sample"] = f"layer 0, documents 0..{docs_done - 1} ({tok_total} memory tokens), scaled to the layer"
    stages["100M-18layer"] = st
    value = tok_total / (t_route + t_topk)
    return {"value": value, "unit": "memory tokens/s", "cores": cores, "affinity_cpus": affinity, "kind": "oracle",
            "sample": f"100M-token workload, layer 0, documents 0..{docs_done - 1} ({tok_total} memory tokens), "
                      f"route + top-k, fp64 numpy, {t_route + t_topk:.1f} s; per-stage timings of every "
                      f"workload in 'stages'",
            "blas": blas_info(), "stages": stages}


# --------------------------------------------------------------------- counter-collection modes
def route_only(w, n, dev):
    """One layer of the 100M-token store scanned n times (msa_route_scan + select), after a 1 GiB
    device-to-device copy (the reference for scaling the traffic counters)."""
    import torch
    from sparse_retrieval_memory_amd import ops
    from synth import workloads as C
    from synth import native
    from synth import splitmix as sm
    kr = torch.empty((w.n_chunks, w.H, w.D), dtype=torch.int16, device=dev)
    native.fill_normal_bf16_device(kr, w.seed, sm.TID_KRBAR, 0, 0)
    qr = torch.from_numpy(C.queries(w, 0)["Qr"].view(np.int16)).to(dev)
    off = torch.from_numpy(w.doc_chunk_off).to(dev)
    nrm = ops.krbar_inv_norms(kr)
    a = torch.empty(1 << 29, dtype=torch.int16, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    ws = ops.workspace(ops.route_topk_workspace_bytes(1, w.T, w.H, w.D, w.n_chunks, w.n_docs, w.k), dev, "ro")
    torch.cuda.synchronize()
    for _ in range(n):
        ops.route_scan(qr, kr, ws, krbar_inv_norm=nrm)
        ops.route_select(1, w.n_chunks, off, w.k, ws)
    torch.cuda.synchronize()
    print(json.dumps({"route_only": n, "copy_bytes": a.numel() * 2, "n_chunks": w.n_chunks,
                      "source_hash": route_source_hash()}), flush=True)


def kernel_only(name, n, dev):
    """One kernel family on its benchmark shape, n calls after a 1 GiB reference copy (for counter runs)."""
    import torch
    from sparse_retrieval_memory_amd import ops
    from synth import workloads as C
    from synth import native
    from synth import splitmix as sm
    bits = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev)
    a = torch.empty(1 << 29, dtype=torch.int16, device=dev)
    torch.empty_like(a).copy_(a)
    if name == "scan3":                      # the 10M batch-16 scan (matrix-core bound)
        w = C.workload("10M-batch16")
        kr = torch.empty((w.n_chunks, w.H, w.D), dtype=torch.int16, device=dev)
        native.fill_normal_bf16_device(kr, w.seed, sm.TID_KRBAR, 0, 0)
        nrm = ops.krbar_inv_norms(kr)
        qr = bits(C.queries(w, 0)["Qr"])
        off = torch.from_numpy(w.doc_chunk_off).to(dev)
        ws = ops.workspace(ops.route_topk_workspace_bytes(w.B, w.T, 8, 128, w.n_chunks, w.n_docs, w.k), dev, "k3")
        fn = lambda: (ops.route_scan(qr, kr, ws, krbar_inv_norm=nrm), ops.route_select(w.B, w.n_chunks, off, w.k, ws))
    elif name == "pool":                     # pooling of one 1M-token slab of the 10M-token corpus
        w = C.workload("10M-interleave")
        d1 = int(np.searchsorted(w.doc_tok_off, 1_000_000, side="right")) - 1
        t1, c1 = int(w.doc_tok_off[d1]), int(w.doc_chunk_off[d1])
        raw = []
        for tid in (sm.TID_K, sm.TID_V, sm.TID_KR):
            t = torch.empty((t1, 8, 128), dtype=torch.int16, device=dev)
            native.fill_normal_bf16_device(t, w.seed, tid, 0, 0)
            raw.append(t)
        to = torch.from_numpy(w.doc_tok_off[:d1 + 1].copy()).to(dev)
        co = torch.from_numpy(w.doc_chunk_off[:d1 + 1].copy()).to(dev)
        out = tuple(torch.empty((c1, 8, 128), dtype=torch.int16, device=dev) for _ in range(3))
        fn = lambda: ops.pool_chunks(*raw, to, co, c1, w.chunk, w.rope_base, out=out)
    elif name == "encode":                   # router-key encoding of one 1M-token slab, d_model 2560
        w = C.workload("10M-interleave")
        d1 = int(np.searchsorted(w.doc_tok_off, 1_000_000, side="right")) - 1
        t1, c1 = int(w.doc_tok_off[d1]), int(w.doc_chunk_off[d1])
        hid = torch.empty((t1, 2560), dtype=torch.int16, device=dev)
        native.fill_normal_bf16_device(hid, w.seed, sm.TID_HIDDEN, 0, 0)
        wk = torch.empty((1024, 2560), dtype=torch.int16, device=dev)
        native.fill_normal_bf16_device(wk, w.seed, sm.TID_WKR, 0, 0)
        to = torch.from_numpy(w.doc_tok_off[:d1 + 1].copy()).to(dev)
        co = torch.from_numpy(w.doc_chunk_off[:d1 + 1].copy()).to(dev)
        out = torch.empty((c1, 8, 128), dtype=torch.int16, device=dev)
        fn = lambda: ops.encode_router_keys(hid, wk, to, co, c1, 8, w.chunk, out=out)
    elif name in ("delete", "route_bwd", "attn"):
        w = C.workload("100M-18layer")
        kr = torch.empty((w.n_chunks, w.H, w.D), dtype=torch.int16, device=dev)
        native.fill_normal_bf16_device(kr, w.seed, sm.TID_KRBAR, 0, 0)
        nrm = ops.krbar_inv_norms(kr)
        off = torch.from_numpy(w.doc_chunk_off).to(dev)
        q = C.queries(w, 0)
        qr = bits(q["Qr"])
        if name == "delete":
            keep = torch.from_numpy((np.random.default_rng(9).random(w.n_docs) >= 0.1).astype(np.uint8)).to(dev)
            out = (torch.empty_like(kr), torch.empty_like(nrm), torch.empty_like(off),
                   torch.empty(w.n_docs, dtype=torch.int32, device=dev), torch.empty(2, dtype=torch.int64, device=dev))
            fn = lambda: ops.store_delete(kr, off, keep, inv_norm=nrm, out=out)
        elif name == "route_bwd":
            _, ch = ops.route_scores(qr, kr, off, want_chunk_scores=True, krbar_inv_norm=nrm)
            dd = torch.from_numpy(np.random.default_rng(10).standard_normal((1, w.n_docs)).astype(np.float32)).to(dev)
            fn = lambda: ops.route_scores_backward(qr, kr, off, ch, dd, krbar_inv_norm=nrm)
        else:
            store = torch.empty((w.n_chunks, 2, 8, 128), dtype=torch.int16, device=dev)
            native.fill_normal_bf16_device(store, w.seed, sm.TID_KBAR, 0, 0)
            Mmax = int(w.doc_n_chunks.max()) * w.k
            staging = torch.empty((1, Mmax, 2, 8, 128), dtype=torch.int16, device=dev)
            _, idx, _ = ops.route_topk(qr, kr, off, w.k, krbar_inv_norm=nrm)
            ml = ops.gather_docs(idx, store, off, staging, Mmax)
            Q, Kl, Vl = bits(q["Q"]), bits(q["Kloc"]), bits(q["Vloc"])
            fn = lambda: ops.sparse_attn_decode(Q, Kl, Vl, staging, staging[:, :, 1], 2 * 8 * 128, Mmax, ml, w.k,
                                                w.rope_base)
    else:
        raise SystemExit(f"unknown --kernel-only {name!r}")
    torch.cuda.synchronize()
    for _ in range(n):
        fn()
    torch.cuda.synchronize()
    print(json.dumps({"kernel_only": name, "calls": n, "copy_bytes": a.numel() * 2}), flush=True)


def traffic_from(fetch_csv: str, write_csv: str, w) -> dict:
    """Per-launch HBM bytes of the scan kernel from two rocprofv3 --pmc runs of --route-only
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by what the same counter reads
    for the 1 GiB device-to-device copy that --route-only performs first."""
    import csv

    def read(path, counter):
        kern, copy = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            if "route_ring8_kernel<true, " in r["Kernel_Name"]:
                kern.append(float(r["Counter_Value"]))
            elif "copyBuffer" in r["Kernel_Name"]:
                copy.append(float(r["Counter_Value"]))
        if not kern or not copy:
            raise SystemExit(f"{path}: no {counter} values for the scan kernel or the reference copy")
        return float(np.mean(kern)), max(copy)

    copy_bytes = 1 << 30
    fk, fc = read(fetch_csv, "FETCH_SIZE")
    wk, wc = read(write_csv, "WRITE_SIZE")
    fs, ws = copy_bytes / (fc * 1024), copy_bytes / (wc * 1024)
    return {"kernel": "route_ring8_kernel<true, POL_NT> (8 heads, stored norms, non-temporal copies)",
            "workload": f"100M-token memory, one routed layer ({w.n_chunks:,} chunks), batch 1, "
                        f"{w.B * w.T} router rows, stored norms",
            "source_hash": route_source_hash(),
            "source_hash_note": "sha256 (first 16 hex) of route.hip + msa_internal.h with comments and "
                                "empty lines removed",
            "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
            "copy_reference": {"bytes": copy_bytes, "fetch_kib": fc, "write_kib": wc},
            "fetch_scale": fs, "write_scale": ws,
            "bytes_per_launch": int(round(fk * 1024 * fs + wk * 1024 * ws)),
            "algorithmic_bytes_per_launch": scan_bytes(w.n_chunks, w.n_docs, w.B, w.T),
            "commands": ["cd /tmp && rocprofv3 --pmc FETCH_SIZE -d <out> -o run --output-format csv -- "
                         "python3 <repo>/bench.py --route-only 5",
                         "cd /tmp && rocprofv3 --pmc WRITE_SIZE -d <out> -o run --output-format csv -- "
                         "python3 <repo>/bench.py --route-only 5",
                         "python3 <repo>/bench.py --traffic-from <out>/run_counter_collection.csv (FETCH) "
                         "<out>/run_counter_collection.csv (WRITE)"]}


# --------------------------------------------------------------------------------- the run
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-baseline-seconds", type=float, default=12.0)
    ap.add_argument("--skip-side", action="store_true", help="headline only (for profiler runs)")
    ap.add_argument("--jsonl", metavar="PATH", default=None,
                    help="also append the result line to PATH (one JSON object per run)")
    ap.add_argument("--route-only", type=int, default=0, metavar="N",
                    help="counter-collection mode: one 100M-token layer, a 1 GiB device copy (the reference for "
                         "scaling FETCH_SIZE/WRITE_SIZE), then N routing scans; prints one line and exits")
    ap.add_argument("--kernel-only", nargs=2, metavar=("NAME", "N"),
                    help="counter-collection mode for one kernel family: scan3 | pool | encode | delete | "
                         "route_bwd | attn, N calls")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the scan kernel's measured HBM traffic per launch (from the counter CSVs of two "
                         "--route-only runs) to profiles/traffic_route_100M.json and exit; needs no GPU")
    args = ap.parse_args()
    if args.traffic_from:
        from synth import workloads as C
        tr = traffic_from(args.traffic_from[0], args.traffic_from[1], C.workload("100M-18layer"))
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(tr, f, indent=1)
        print(json.dumps({k: tr[k] for k in ("bytes_per_launch", "algorithmic_bytes_per_launch", "source_hash")}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the library runs the path on a "
              "single MI355X and does not shard it across GPUs.", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_retrieval_memory_amd import ops
    from synth import workloads as C
    from synth import native
    from synth import splitmix as sm

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.route_only:
        route_only(C.workload("100M-18layer"), args.route_only, dev)
        return
    if args.kernel_only:
        kernel_only(args.kernel_only[0], int(args.kernel_only[1]), dev)
        return
    w = C.workload("100M-18layer")
    G, H, D, L, k = w.n_chunks, w.H, w.D, w.n_layers, w.k
    log(f"workload {w.name}: {w.n_docs} docs, {w.n_tok} tokens, {G} chunks, {L} layers")
    bits = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    Ev = lambda: torch.cuda.Event(enable_timing=True)

    def time_ms(fn, reps, warm=1):
        """Median over reps of one call bracketed by its own pair of events on the current stream."""
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        evs = [(Ev(), Ev()) for _ in range(reps)]
        for a, b_ in evs:
            a.record()
            fn()
            b_.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b_) for a, b_ in evs]))

    # ---------------------------------------------------------------- inputs (100M, 18 layers)
    t0 = time.time()
    off_dev = torch.from_numpy(w.doc_chunk_off).to(dev)
    off_host = torch.from_numpy(w.doc_chunk_off.copy())
    krbar, knorm, qr, Q, Q1, Kl, Vl = [], [], [], [], [], [], []
    for layer in range(L):
        t = torch.empty((G, H, D), dtype=torch.int16, device=dev)
        native.fill_normal_bf16_device(t, w.seed, sm.TID_KRBAR, layer, 0)
        for g, row in C.pooled_plants(w, layer).items():
            t[g].copy_(bits(row))
        krbar.append(t)
        knorm.append(ops.krbar_inv_norms(t))      # built once with the store, like the store itself
        q = C.queries(w, layer)
        qr.append(bits(q["Qr"])); Q.append(bits(q["Q"])); Q1.append(bits(q["Q"][:, -1:]))
        Kl.append(bits(q["Kloc"])); Vl.append(bits(q["Vloc"]))
    kd = torch.empty((G, H, D), dtype=torch.int16, device=dev)
    vd = torch.empty((G, H, D), dtype=torch.int16, device=dev)
    native.fill_normal_bf16_device(kd, w.seed, sm.TID_KBAR, 0, 0)
    native.fill_normal_bf16_device(vd, w.seed, sm.TID_VBAR, 0, 0)
    store = torch.empty((G, 2, H, D), dtype=torch.int16, pin_memory=True)
    store.copy_(torch.stack([kd, vd], dim=1))
    del kd, vd
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log(f"inputs ready in {time.time() - t0:.1f} s (Krbar {L * G * H * D * 2 / 1e9:.1f} GB in HBM, "
        f"content {store.numel() * 2 / 1e9:.1f} GB pinned host)")

    Mmax = int(w.doc_n_chunks.max()) * k
    staging = torch.empty((1, Mmax, 2, H, D), dtype=torch.int16, device=dev)
    top_host = torch.empty((1, k), dtype=torch.int32, pin_memory=True)
    ml_host = torch.empty(1, dtype=torch.int32, pin_memory=True)
    ml_dev = torch.empty(1, dtype=torch.int32, device=dev)
    O_out = torch.empty((1, w.Tq, w.Hq, D), dtype=torch.float32, device=dev)
    O1_out = torch.empty((1, 1, w.Hq, D), dtype=torch.float32, device=dev)
    doc = torch.empty((1, w.n_docs), dtype=torch.float32, device=dev)
    idx_d = torch.empty((1, k), dtype=torch.int32, device=dev)
    sc_d = torch.empty((1, k), dtype=torch.float32, device=dev)
    ws = ops.workspace(ops.route_topk_workspace_bytes(1, w.T, H, D, G, w.n_docs, k), dev, "bench-route")
    ws_k = ops.workspace(ops.topk_workspace_bytes(1, w.n_docs, k), dev, "bench-topk")
    comp = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side_attn = torch.cuda.Stream()
    ev_scan, ev_local, ev_ids, ev_fetch = (torch.cuda.Event() for _ in range(4))
    part = (torch.empty((1, w.Tq, w.Hq, D), dtype=torch.float32, device=dev),
            torch.empty((1, w.Tq, w.Hq, 2), dtype=torch.float32, device=dev))

    def layer_step(layer, scan_ev=None, decode=False, split=False):
        """scan -> document max + top-k -> device-side assembly from the pinned host tier -> attend; one
        stream, no host sync.  scan_ev: a pair of events recorded around the scan kernel.  decode: the
        attention takes the last query row only (Tq = 1).  split (side measurement): the local-key half
        of the attention runs on a second stream once the scan is done, overlapping the selection and the
        gather; the memory half then merges with it."""
        if scan_ev is not None:
            scan_ev[0].record(comp)
        ops.route_scan(qr[layer], krbar[layer], ws, krbar_inv_norm=knorm[layer])
        if scan_ev is not None:
            scan_ev[1].record(comp)
        if split:
            ev_scan.record(comp)
            side_attn.wait_event(ev_scan)
            ops.sparse_attn_local_partial(Q[layer], Kl[layer], Vl[layer], k, w.rope_base, part=part,
                                          stream=side_attn)
            ev_local.record(side_attn)
        ops.route_select(1, G, off_dev, k, ws, doc_scores=doc, top_idx=idx_d, top_scores=sc_d)
        ops.gather_docs(idx_d, store, off_dev, staging, Mmax, mem_len=ml_dev)
        if split:
            comp.wait_event(ev_local)
            ops.sparse_attn_memory_merge(Q[layer], w.Tl, H, staging, staging[:, :, 1], 2 * H * D, Mmax, ml_dev, k,
                                         part, w.rope_base, out=O_out)
        elif decode:
            ops.sparse_attn_decode(Q1[layer], Kl[layer], Vl[layer], staging, staging[:, :, 1], 2 * H * D, Mmax,
                                   ml_dev, k, w.rope_base, out=O1_out)
        else:
            ops.sparse_attn_decode(Q[layer], Kl[layer], Vl[layer], staging, staging[:, :, 1], 2 * H * D, Mmax,
                                   ml_dev, k, w.rope_base, out=O_out)

    def layer_step_host_fetch(layer):
        """The same layer with the ids sent to the host and the content copied by hipMemcpyAsync on a side stream."""
        ops.route_topk(qr[layer], krbar[layer], off_dev, k, krbar_inv_norm=knorm[layer], doc_scores=doc,
                       top_idx=idx_d, top_scores=sc_d, ws=ws)
        top_host.copy_(idx_d, non_blocking=True)
        ev_ids.record(comp)
        ev_ids.synchronize()
        ml = ops.fetch_docs(top_host, store, off_host, staging, Mmax, side, ev_fetch)
        ml_host.copy_(ml)
        ml_dev.copy_(ml_host, non_blocking=True)
        comp.wait_event(ev_fetch)
        ops.sparse_attn_decode(Q[layer], Kl[layer], Vl[layer], staging, staging[:, :, 1], 2 * H * D, Mmax, ml_dev,
                               k, w.rope_base, out=O_out)

    # ---------------------------------------------------------------- warmup
    selected = []
    for s_ in range(max(args.warmup, 1)):
        for layer in range(L):
            layer_step(layer)
            if s_ == 0:
                selected.append(idx_d.cpu().numpy()[0].copy())
    torch.cuda.synchronize()
    needles_found = sum(int(d in selected[layer]) for layer in range(L) for (_, d) in C.planted_docs(w, layer))
    log(f"warmup done; planted needles retrieved: {needles_found}/{L * w.n_needles}")

    # ----------------------------------------------------------------- timed
    n_ev = args.steps * len(SCAN_EVENT_LAYERS)
    scan_evs = [(Ev(), Ev()) for _ in range(n_ev)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    e = 0
    for s_ in range(args.steps):
        for layer in range(L):
            if layer in SCAN_EVENT_LAYERS:
                layer_step(layer, scan_ev=scan_evs[e])
                e += 1
            else:
                layer_step(layer)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_step = elapsed * 1e3 / args.steps
    tokens_per_s = w.n_tok * L * args.steps / elapsed
    scan_ms = np.array([a.elapsed_time(b_) for a, b_ in scan_evs])
    log(f"timed {args.steps} steps: {ms_step:.2f} ms/step; scan kernel {np.mean(scan_ms):.4f} ms (mean of {n_ev})")

    # ------------------------------------------------------- side measurements (100M)
    side_out = {}

    def steps_ms(n, **kw):
        torch.cuda.synchronize()
        t0_ = time.perf_counter()
        for _ in range(n):
            for layer in range(L):
                layer_step(layer, **kw)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0_) * 1e3 / n

    side_out["step_ms_no_scan_events"] = steps_ms(args.steps)
    side_out["decode_step_ms_tq1"] = steps_ms(args.steps, decode=True)
    side_out["step_ms_split_attention"] = steps_ms(max(args.steps // 2, 1), split=True)
    log(f"no-event step {side_out['step_ms_no_scan_events']:.2f} ms, decode step {side_out['decode_step_ms_tq1']:.2f} ms")
    # per-layer latency (events around each layer) and the scan alone, in a separate instrumented pass
    lay = [(Ev(), Ev()) for _ in range(L * 5)]
    for i, (a, b_) in enumerate(lay):
        a.record()
        layer_step(i % L)
        b_.record()
    torch.cuda.synchronize()
    layer_ms = np.array([a.elapsed_time(b_) for a, b_ in lay])
    # host round trip + hipMemcpyAsync fetch
    for layer in range(L):
        layer_step_host_fetch(layer)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        for layer in range(L):
            layer_step_host_fetch(layer)
    torch.cuda.synchronize()
    side_out["host_fetch_step_ms"] = (time.perf_counter() - t0) * 1e3 / 3
    ops.route_topk(qr[0], krbar[0], off_dev, k, krbar_inv_norm=knorm[0], doc_scores=doc, top_idx=idx_d,
                   top_scores=sc_d, ws=ws)
    ops.gather_docs(idx_d, store, off_dev, staging, Mmax, mem_len=ml_dev)
    side_out["attn_us"] = {
        "tq128": 1e3 * time_ms(lambda: ops.sparse_attn_decode(Q[0], Kl[0], Vl[0], staging, staging[:, :, 1], 2 * H * D,
                                                              Mmax, ml_dev, k, w.rope_base, out=O_out), 50),
        "tq1_decode": 1e3 * time_ms(lambda: ops.sparse_attn_decode(Q1[0], Kl[0], Vl[0], staging, staging[:, :, 1],
                                                                   2 * H * D, Mmax, ml_dev, k, w.rope_base,
                                                                   out=O1_out), 50)}
    side_out["topk_us"] = 1e3 * time_ms(lambda: ops.topk_docs(doc, k, top_idx=idx_d, top_scores=sc_d, ws=ws_k), 50)
    side_out["gather_us"] = 1e3 * time_ms(lambda: ops.gather_docs(idx_d, store, off_dev, staging, Mmax, mem_len=ml_dev),
                                          50)
    # document max + top-k alone: each call's events bracket only msa_route_select, after a scan
    sel_ev = []
    for _ in range(10):
        ops.route_scan(qr[0], krbar[0], ws, krbar_inv_norm=knorm[0])
        a_, b2 = Ev(), Ev()
        a_.record()
        ops.route_select(1, G, off_dev, k, ws, doc_scores=doc, top_idx=idx_d, top_scores=sc_d)
        b2.record()
        sel_ev.append((a_, b2))
    torch.cuda.synchronize()
    side_out["select_us"] = 1e3 * float(np.median([a_.elapsed_time(b2) for a_, b2 in sel_ev[1:]]))
    ws_nn = ops.workspace(ops.route_workspace_bytes(1, w.T, H, D, G, w.n_docs), dev, "bench-nonorm")
    side_out["scan_ms_norms_in_kernel"] = time_ms(lambda: (ops.route_scan(qr[0], krbar[0], ws_nn),
                                                           ops.route_workspace_clear(ws_nn)), 10)

    # attention backward at the step's shape
    d_out = torch.from_numpy(np.random.default_rng(11).standard_normal((1, w.Tq, w.Hq, D)).astype(np.float32)).to(dev)
    ab_out = (torch.empty((1, w.Tq, w.Hq, D), dtype=torch.float32, device=dev),
              torch.empty((1, w.Tl, H, D), dtype=torch.float32, device=dev),
              torch.empty((1, w.Tl, H, D), dtype=torch.float32, device=dev),
              torch.empty((1, Mmax, H, D), dtype=torch.float32, device=dev),
              torch.empty((1, Mmax, H, D), dtype=torch.float32, device=dev))
    ws_ab = ops.workspace(ops.attn_backward_workspace_bytes(1, w.Tq, w.Hq, D, w.Tl, H, Mmax), dev, "bench-attn-bwd")
    attn_bwd_us = 1e3 * time_ms(lambda: ops.sparse_attn_backward(Q[0], Kl[0], Vl[0], staging, staging[:, :, 1],
                                                                 2 * H * D, Mmax, ml_dev, k, d_out, w.rope_base,
                                                                 out=ab_out, ws=ws_ab), 50)
    o_fw, lse_fw = ops.sparse_attn_forward(Q[0], Kl[0], Vl[0], staging, staging[:, :, 1], 2 * H * D, Mmax, ml_dev, k,
                                           w.rope_base)
    attn_bwd_saved_us = 1e3 * time_ms(lambda: ops.sparse_attn_backward(Q[0], Kl[0], Vl[0], staging,
                                                                       staging[:, :, 1], 2 * H * D, Mmax, ml_dev, k,
                                                                       d_out, w.rope_base, out=ab_out, ws=ws_ab,
                                                                       O=o_fw, lse=lse_fw), 50)
    attn_fwd_lse_us = 1e3 * time_ms(lambda: ops.sparse_attn_forward(Q[0], Kl[0], Vl[0], staging, staging[:, :, 1],
                                                                    2 * H * D, Mmax, ml_dev, k, w.rope_base,
                                                                    out=o_fw, lse=lse_fw), 50)
    del o_fw, lse_fw
    n_mem = int(ml_dev.item())
    n_vis = w.Tq * n_mem + sum(w.Tl - w.Tq + i + 1 for i in range(w.Tq))      # visible (row, key) pairs per head
    attn_bwd_flops = 5 * 2.0 * n_vis * D * w.Hq                                  # S, dP, dV, dK, dQ
    side_out["attn_backward_tq128"] = {"us": attn_bwd_us, "memory_entries": n_mem,
                                       "TFLOPs": attn_bwd_flops / (attn_bwd_us * 1e-6) / 1e12,
                                       "us_with_saved_stats": attn_bwd_saved_us,
                                       "forward_with_lse_us": attn_fwd_lse_us}
    del ab_out
    # routing-store update: delete 10% of one layer's documents
    keep_d = torch.from_numpy((np.random.default_rng(9).random(w.n_docs) >= 0.1).astype(np.uint8)).to(dev)
    del_out = (torch.empty_like(krbar[0]), torch.empty_like(knorm[0]), torch.empty_like(off_dev),
               torch.empty(w.n_docs, dtype=torch.int32, device=dev), torch.empty(2, dtype=torch.int64, device=dev))
    delete_ms = time_ms(lambda: ops.store_delete(krbar[0], off_dev, keep_d, inv_norm=knorm[0], out=del_out), 5)
    kept_chunks = int(del_out[4][1].item())
    delete_bytes = 2 * kept_chunks * H * (D * 2 + 4) + w.n_docs * (1 + 8 + 4 + 8)
    del del_out
    side_out["store_delete_10pct_100M_layer"] = {"ms": delete_ms, "GBps": delete_bytes / (delete_ms * 1e-3) / 1e9,
                                                 "frac_of_8TBps": delete_bytes / (delete_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    # routing-score backward over one 100M-token layer: every document gets an upstream gradient
    _, ch0 = ops.route_scores(qr[0], krbar[0], off_dev, want_chunk_scores=True, krbar_inv_norm=knorm[0])
    d_doc = torch.from_numpy(np.random.default_rng(10).standard_normal((1, w.n_docs)).astype(np.float32)).to(dev)
    bwd_out = (torch.empty((1, w.T, H, D), dtype=torch.float32, device=dev),
               torch.empty((1, w.n_docs, H, D), dtype=torch.float32, device=dev),
               torch.empty((1, w.n_docs, 2), dtype=torch.int32, device=dev))
    ws_b = ops.workspace(ops.route_backward_workspace_bytes(1, w.T, H, D, w.n_docs), dev, "bench-route-bwd")
    bwd_ms = time_ms(lambda: ops.route_scores_backward(qr[0], krbar[0], off_dev, ch0, d_doc, krbar_inv_norm=knorm[0],
                                                       dQr=bwd_out[0], dKsel=bwd_out[1], sel=bwd_out[2], ws=ws_b), 5)
    bwd_bytes = (G * 4 + (w.n_docs + 1) * 8 + w.n_docs * 4 + w.n_docs * H * D * (2 + 4) + w.n_docs * 8
                 + w.T * H * D * (2 + 4))
    side_out["route_backward_100M_layer"] = {"ms": bwd_ms, "GBps": bwd_bytes / (bwd_ms * 1e-3) / 1e9,
                                             "frac_of_8TBps": bwd_bytes / (bwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                             "recompute_TFLOPs": 2.0 * w.n_docs * w.T * H * D / (bwd_ms * 1e-3) / 1e12,
                                             "docs_with_gradient": w.n_docs}
    del bwd_out, ch0

    # --------------------------------------------- scan time against memory size (T = 128, batch 1)
    # slices of the 18 layer stores, cycled so that >= 600 MB of distinct keys pass between reuses
    # (the 256 MB Infinity Cache cannot serve a repeat); the 32K point fits in any cache (launch-bound)
    curve = []
    for n_ch in (512, 4096, 16_611, 65_536, 165_789, 500_000, G):
        per_layer = G // n_ch
        slices = [(l_, j) for j in range(per_layer) for l_ in range(L)]
        need = max(2, int(np.ceil(600e6 / (n_ch * H * D * 2))))
        slices = slices[:need] if need <= len(slices) else slices
        ws_c = ops.workspace(ops.route_workspace_bytes(1, w.T, H, D, n_ch, 1), dev, "bench-curve")
        turn = [0]

        def scan_slice():
            l_, j = slices[turn[0] % len(slices)]
            turn[0] += 1
            ops.route_scan(qr[0], krbar[l_][j * n_ch:(j + 1) * n_ch], ws_c,
                           krbar_inv_norm=knorm[l_][j * n_ch:(j + 1) * n_ch])

        for _ in range(min(len(slices), 40)):
            scan_slice()
            ops.route_workspace_clear(ws_c)
        torch.cuda.synchronize()
        evs = [(Ev(), Ev()) for _ in range(40)]
        for a, b_ in evs:
            a.record()
            scan_slice()
            b_.record()
            ops.route_workspace_clear(ws_c)
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b_) for a, b_ in evs]))
        nbytes = scan_bytes(n_ch, max(1, n_ch // 8), 1, w.T)
        curve.append({"n_chunks": n_ch, "memory_tokens_approx": n_ch * 64, "scan_ms": ms,
                      "memory_tokens_per_s": n_ch * 64 / (ms * 1e-3), "GBps": nbytes / (ms * 1e-3) / 1e9,
                      "frac_of_8TBps": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "distinct_slices_cycled": len(slices)})
    log("scan curve: " + ", ".join(f"{c['n_chunks']}: {c['scan_ms']:.4f} ms" for c in curve))

    # ------------------------------------------------------------ per-workload routed steps
    workloads = {}

    def routed_step_record(wl, kr_list, nrm_list, q_dev, content, tq_rows=None):
        """Median latency of one routed step (scan -> select -> gather -> attend) of workload wl, cycling
        through the given store copies; plus the scan alone."""
        B = wl.B
        Gw = wl.n_chunks
        offd = torch.from_numpy(wl.doc_chunk_off).to(dev)
        ws_w = ops.workspace(ops.route_topk_workspace_bytes(B, wl.T, H, D, Gw, wl.n_docs, wl.k), dev, f"wl-{wl.name}")
        Mw = int(wl.doc_n_chunks.max()) * wl.k
        stg = torch.empty((B, Mw, 2, H, D), dtype=torch.int16, device=dev)
        mlw = torch.empty(B, dtype=torch.int32, device=dev)
        dw = torch.empty((B, wl.n_docs), dtype=torch.float32, device=dev)
        iw = torch.empty((B, wl.k), dtype=torch.int32, device=dev)
        sw = torch.empty((B, wl.k), dtype=torch.float32, device=dev)
        Ow = torch.empty((B, wl.Tq, wl.Hq, D), dtype=torch.float32, device=dev)
        turn = [0]

        def scan():
            c = turn[0] % len(kr_list)
            ops.route_scan(q_dev["Qr"], kr_list[c], ws_w, krbar_inv_norm=nrm_list[c])

        def rest():
            ops.route_select(B, Gw, offd, wl.k, ws_w, doc_scores=dw, top_idx=iw, top_scores=sw)
            ops.gather_docs(iw, content, offd, stg, Mw, mem_len=mlw)
            ops.sparse_attn_decode(q_dev["Q"], q_dev["Kloc"], q_dev["Vloc"], stg, stg[:, :, 1], 2 * H * D, Mw, mlw,
                                   wl.k, wl.rope_base, out=Ow)

        def step():
            scan()
            turn[0] += 1
            rest()

        step_ms = time_ms(step, 30, warm=3)
        se = [(Ev(), Ev()) for _ in range(30)]
        for a, b_ in se:
            a.record()
            scan()
            b_.record()
            turn[0] += 1
            rest()
        torch.cuda.synchronize()
        sms = float(np.median([a.elapsed_time(b_) for a, b_ in se]))
        nbytes = scan_bytes(Gw, wl.n_docs, B, wl.T)
        fl = scan_flops(Gw, B, wl.T)
        rec = {"memory_tokens": wl.n_tok, "queries": B, "router_rows_per_query": wl.T, "top_k": wl.k,
               "step_ms": step_ms, "memory_tokens_per_s_per_query": wl.n_tok / (step_ms * 1e-3),
               "memory_tokens_per_s_all_queries": B * wl.n_tok / (step_ms * 1e-3),
               "scan_ms": sms, "scan_GBps": nbytes / (sms * 1e-3) / 1e9,
               "scan_frac_of_8TBps": nbytes / (sms * 1e-3) / 1e9 / HBM_PEAK_GBS,
               "scan_TFLOPs": fl / (sms * 1e-3) / 1e12, "scan_mfma_frac": fl / (sms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
               "store_copies_cycled": len(kr_list),
               "step": "scan -> document max + top-k -> gather from pinned host -> attend, one stream"}
        del stg
        return rec

    def drawn_store(wl, n_copies):
        base = torch.empty((wl.n_chunks, H, D), dtype=torch.int16, device=dev)
        native.fill_normal_bf16_device(base, wl.seed, sm.TID_KRBAR, 0, 0)
        for g, row in C.pooled_plants(wl, 0).items():
            base[g].copy_(bits(row))
        krs = [base] + [base.clone() for _ in range(n_copies - 1)]
        nrm = ops.krbar_inv_norms(base)
        content = torch.empty((wl.n_chunks, 2, H, D), dtype=torch.int16, pin_memory=True)
        for j, tid in enumerate((sm.TID_KBAR, sm.TID_VBAR)):
            t = torch.empty((wl.n_chunks, H, D), dtype=torch.int16, device=dev)
            native.fill_normal_bf16_device(t, wl.seed, tid, 0, 0)
            content[:, j].copy_(t)
            del t
        return krs, [nrm] * n_copies, content

    def qdev(wl):
        qq = C.queries(wl, 0)
        return {x: bits(qq[x]) for x in ("Qr", "Q", "Kloc", "Vloc")}

    # 32K: pooled on the device from raw tokens (pooling timed too), then the routed step
    w1 = C.workload("tiny-32K")
    raw1 = []
    for tid in (sm.TID_K, sm.TID_V, sm.TID_KR):
        t = torch.empty((w1.n_tok, H, D), dtype=torch.int16, device=dev)
        native.fill_normal_bf16_device(t, w1.seed, tid, 0, 0)
        raw1.append(t)
    for tok, row in C.raw_plants(w1).items():
        raw1[2][tok].copy_(bits(row))
    to1 = torch.from_numpy(w1.doc_tok_off).to(dev)
    co1 = torch.from_numpy(w1.doc_chunk_off).to(dev)
    pooled1 = ops.pool_chunks(*raw1, to1, co1, w1.n_chunks, w1.chunk, w1.rope_base)
    pool1_ms = time_ms(lambda: ops.pool_chunks(*raw1, to1, co1, w1.n_chunks, w1.chunk, w1.rope_base, out=pooled1), 20)
    content1 = torch.stack([pooled1[0], pooled1[1]], dim=1).cpu().pin_memory()
    rec = routed_step_record(w1, [pooled1[2]], [ops.krbar_inv_norms(pooled1[2])], qdev(w1), content1)
    rec["pool_ms"] = pool1_ms
    rec["note"] = "1 MB routing store, cache-resident: launch-latency bound"
    workloads["tiny-32K"] = rec
    del raw1, pooled1
    # 1M: 16 copies of the 34 MB store (545 MB) cycled so the Infinity Cache cannot serve a repeat
    w2 = C.workload("1M")
    krs, nrms, content2 = drawn_store(w2, 16)
    workloads["1M"] = routed_step_record(w2, krs, nrms, qdev(w2), content2)
    del krs, nrms, content2
    # 10M batch-16: two copies of the 338 MB store used in turn
    w3 = C.workload("10M-batch16")
    krs, nrms, content3 = drawn_store(w3, 2)
    workloads["10M-batch16"] = routed_step_record(w3, krs, nrms, qdev(w3), content3)
    del krs, nrms, content3
    # library bf16 GEMM as the achievable dense matrix rate on this GPU
    ga = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
    gb = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
    gemm_ms = time_ms(lambda: torch.matmul(ga, gb), 10)
    gemm_tflops = 2.0 * 8192 ** 3 / (gemm_ms * 1e-3) / 1e12
    del ga, gb
    workloads["10M-batch16"]["gemm_bf16_8192_TFLOPs"] = gemm_tflops
    workloads["10M-batch16"]["scan_frac_of_gemm"] = workloads["10M-batch16"]["scan_TFLOPs"] / gemm_tflops
    log(f"per-workload steps: " + ", ".join(f"{n}: {r['step_ms']:.3f} ms" for n, r in workloads.items()))

    # 10M interleave: pooling and encoding over the whole corpus (1M-token slabs), then 3 rounds
    from sparse_retrieval_memory_amd.interleave import Interleave
    w5 = C.workload("10M-interleave")
    E = w5.row_elems
    pooled5 = tuple(torch.empty((w5.n_chunks, H, D), dtype=torch.int16, device=dev) for _ in range(3))
    plants5 = C.raw_plants(w5)
    pool_us, pool_bytes = [], 0
    slabs = []
    d0 = 0
    while d0 < w5.n_docs:
        d1 = min(max(int(np.searchsorted(w5.doc_tok_off, w5.doc_tok_off[d0] + 1_000_000, side="right")) - 1, d0 + 1),
                 w5.n_docs)
        slabs.append((d0, d1))
        d0 = d1
    for d0, d1 in slabs:
        t0_, t1_ = int(w5.doc_tok_off[d0]), int(w5.doc_tok_off[d1])
        c0_, c1_ = int(w5.doc_chunk_off[d0]), int(w5.doc_chunk_off[d1])
        raw = []
        for tid in (sm.TID_K, sm.TID_V, sm.TID_KR):
            t = torch.empty((t1_ - t0_, H, D), dtype=torch.int16, device=dev)
            native.fill_normal_bf16_device(t, w5.seed, tid, 0, t0_ * E)
            raw.append(t)
        for tok, row in plants5.items():
            if t0_ <= tok < t1_:
                raw[2][tok - t0_].copy_(bits(row))
        tok_off5 = torch.from_numpy(w5.doc_tok_off[d0:d1 + 1].copy()).to(dev)
        ch_off5 = torch.from_numpy(w5.doc_chunk_off[d0:d1 + 1].copy()).to(dev)
        outs = tuple(o[c0_:c1_] for o in pooled5)
        pool_us.append(1e3 * time_ms(lambda: ops.pool_chunks(*raw, tok_off5, ch_off5, c1_ - c0_, w5.chunk,
                                                             w5.rope_base, out=outs), 3))
        pool_bytes += 3 * (t1_ - t0_) * H * D * 2 + 3 * (c1_ - c0_) * H * D * 2
        del raw
    DM = 2560
    w_kr = torch.empty((H * D, DM), dtype=torch.int16, device=dev)
    native.fill_normal_bf16_device(w_kr, w5.seed, sm.TID_WKR, 0, 0)
    enc_out = torch.empty((w5.n_chunks, H, D), dtype=torch.int16, device=dev)
    enc_ms, enc_bytes, enc_flops = [], 0, 0
    for d0, d1 in slabs:
        t0_, t1_ = int(w5.doc_tok_off[d0]), int(w5.doc_tok_off[d1])
        c0_, c1_ = int(w5.doc_chunk_off[d0]), int(w5.doc_chunk_off[d1])
        hid = torch.empty((t1_ - t0_, DM), dtype=torch.int16, device=dev)
        native.fill_normal_bf16_device(hid, w5.seed, sm.TID_HIDDEN, 0, t0_ * DM)
        tok_off5 = torch.from_numpy(w5.doc_tok_off[d0:d1 + 1].copy()).to(dev)
        ch_off5 = torch.from_numpy(w5.doc_chunk_off[d0:d1 + 1].copy()).to(dev)
        enc_ms.append(time_ms(lambda: ops.encode_router_keys(hid, w_kr, tok_off5, ch_off5, c1_ - c0_, H, w5.chunk,
                                                             out=enc_out[c0_:c1_]), 3))
        enc_bytes += (t1_ - t0_) * DM * 2 + (c1_ - c0_) * H * D * 2
        enc_flops += 2 * (c1_ - c0_) * DM * H * D
        del hid
    enc_bytes += H * D * DM * 2
    del w_kr, enc_out
    store5 = torch.stack([pooled5[0], pooled5[1]], dim=1).cpu().pin_memory()
    q5 = C.queries(w5, 0)
    il = Interleave(krbar=pooled5[2], doc_chunk_off=torch.from_numpy(w5.doc_chunk_off).to(dev),
                    doc_chunk_off_host=torch.from_numpy(w5.doc_chunk_off.copy()), content=store5,
                    krbar_inv_norm=ops.krbar_inv_norms(pooled5[2]), rope_base=w5.rope_base)
    args5 = (bits(q5["Qr"]), bits(q5["Q"]), bits(q5["Kloc"]), bits(q5["Vloc"]), w5.k, w5.rounds)
    il.run(*args5)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    res5 = il.run(*args5)
    torch.cuda.synchronize()
    interleave_ms = (time.perf_counter() - t0) * 1e3
    round_ms = [rd.ms for rd in il.run(*args5, timing=True)]
    chains_ok = sum(int(ch["A"] in res5[0].top_idx[b] and ch["B"] in res5[1].top_idx[b] and
                        ch["C"] in res5[2].top_idx[b]) for b, ch in enumerate(C.chains(w5)))
    del pooled5, store5
    pool_GBps = pool_bytes / (sum(pool_us) * 1e-6) / 1e9
    workloads["10M-interleave"] = {
        "memory_tokens": w5.n_tok, "queries": w5.B, "rounds": w5.rounds, "top_k": w5.k,
        "three_rounds_ms": interleave_ms, "round_ms": round_ms,
        "memory_tokens_per_s_per_query_per_round": w5.rounds * w5.n_tok / (interleave_ms * 1e-3),
        "chains_recovered": f"{chains_ok}/{w5.B}",
        "pool_ms_10M": sum(pool_us) * 1e-3, "pool_GBps": pool_GBps, "pool_frac_of_8TBps": pool_GBps / HBM_PEAK_GBS,
        "encode_router_keys_ms_10M": float(sum(enc_ms)),
        "encode_GBps": enc_bytes / (sum(enc_ms) * 1e-3) / 1e9,
        "encode_frac_of_8TBps": enc_bytes / (sum(enc_ms) * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "encode_projection_TFLOPs_equiv": enc_flops / (sum(enc_ms) * 1e-3) / 1e12,
        "round": "append router rows -> scan + top-k -> ids to host -> gather -> attend (one host round trip)"}
    log(f"interleave: 3 rounds in {interleave_ms:.2f} ms, chains {chains_ok}/{w5.B}; pool {pool_GBps:.0f} GB/s")

    # ---------------------------------------------------------------- report
    bytes_algo = scan_bytes(G, w.n_docs, w.B, w.T)
    scan_avg_s = float(scan_ms.mean()) * 1e-3
    achieved = bytes_algo / scan_avg_s / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        if tr.get("source_hash") == route_source_hash():
            traffic = tr.get("bytes_per_launch")
    workloads["100M-18layer"] = {
        "memory_tokens": w.n_tok, "queries": 1, "router_rows_per_query": w.T, "top_k": k, "layers": L,
        "step_ms_18_layers": ms_step, "layer_ms": pct(layer_ms), "scan_ms": pct(scan_ms),
        "memory_tokens_per_s_per_layer": w.n_tok / scan_avg_s,
        "decode_step_ms_18_layers_tq1": side_out["decode_step_ms_tq1"],
        "scan_TFLOPs": scan_flops(G, 1, w.T) / scan_avg_s / 1e12}
    cpu = None
    if args.cpu_baseline_seconds > 0:
        log("timing the oracle on the host ...")
        cpu = cpu_baseline(args.cpu_baseline_seconds)
    out = {
        "metric": "memory tokens/s routed per query (Krbar scan GB/s) + route+attn step latency",
        "value": tokens_per_s,
        "unit": "memory tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "100M-token memory, 18 routed layers, batch 1, 128-token query, top-16",
                   "n_docs": w.n_docs, "memory_tokens": w.n_tok, "n_chunks": G, "layers": L,
                   "router_heads": H, "head_dim": D, "q_heads": w.Hq, "chunk": w.chunk, "top_k": k,
                   "krbar_store": f"18 distinct layer stores in HBM ({L * G * H * D * 2 / 1e9:.1f} GB) with stored "
                                  "inverse norms",
                   "content_tier": f"one {store.numel() * 2 / 1e9:.1f} GB pooled K/V store in pinned host memory, "
                                   "shared (aliased) by all 18 layers (18 distinct stores would need 122 GB pinned)",
                   "step": "18 x (msa_route_scan -> msa_route_select (document max + top-16) -> assemble the selected "
                           "K/V from the pinned host tier by a device kernel -> attend), one stream, no host round "
                           "trip"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "route_ring8_kernel (msa_route_scan), mean of HIP-event durations around the scan of "
                               f"layers {list(SCAN_EVENT_LAYERS)} in every timed step ({len(scan_ms)} launches); bytes = "
                               "Krbar + doc offsets + Qr + doc scores (32 B per memory token)",
                     "bytes_per_launch": bytes_algo,
                     "achieved_incl_stored_norms": (bytes_algo + G * H * 4) / scan_avg_s / 1e9},
        "cpu_baseline": cpu,
        "workloads": workloads,
        "scan_vs_memory_size": curve,
        "needles_retrieved": f"{needles_found}/{L * w.n_needles}",
    }
    out.update(side_out)
    line = json.dumps(out)
    print(line, flush=True)
    if args.jsonl:
        with open(args.jsonl, "a") as fh:
            fh.write(line + "\n")


if __name__ == "__main__":
    main()
