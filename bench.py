"""Benchmark of the MSA routed step on one MI355X.

Workload (default): a 100M-token memory of 200,000 synthetic documents
(lengths uniform on [64, 936], mean 500), chunk 64 -> 1.66M pooled chunks,
18 routed layers, each with its own HBM-resident Krbar store (bf16, 8 x 128 per
chunk, 61 GB in total) and its own 128-token router query (batch 1).  One step
runs the 18 layers in sequence; a layer is

    route (scan of all Krbar + document max) -> top-16 documents ->
    assemble the selected pooled K/V from the pinned host tier (one kernel
    reading the mapped host memory; the ids never leave the GPU) ->
    GQA attention (32 q-heads, 128 query rows, 128 local tokens) over
    [fetched memory ++ local KV].

The same step with the ids copied to the host and the content fetched by
hipMemcpyAsync on a side stream is timed beside it, as are attention alone
(128 rows and 1-row decode), top-k alone, the scan of the 10M-token batch-16
workload (matrix-core bound), pooling throughput and the rounds of the
10M-token interleave workload.  Inputs are generated on the device before
timing (seeded, synthetic); the pooled content store (Kbar|Vbar, 6.8 GB) sits
in pinned host memory and is shared by all layers.  The printed JSON line
reports memory tokens routed per second (per query), the step latency, the
roofline of the routing call and the oracle's CPU throughput on a bounded
sample of the same workload.
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

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_route_100M.json")


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


def cpu_baseline(w, seconds: float):
    """Oracle route + top-k on a bounded slice of layer 0 (documents from the start)."""
    from oracle import msa_oracle as O
    from synth import workloads as C
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    q = C.queries(w, 0)
    Qr = O.bf16_to_f64(q["Qr"])
    d = 1000
    t_total, tok_total, docs_done = 0.0, 0, 0
    while t_total < seconds and docs_done < w.n_docs:
        d1 = min(w.n_docs, docs_done + d)
        g0, g1 = int(w.doc_chunk_off[docs_done]), int(w.doc_chunk_off[d1])
        kr = O.bf16_to_f64(C.krbar_block(w, 0, g0, g1))
        off = w.doc_chunk_off[docs_done:d1 + 1] - g0
        t0 = time.perf_counter()
        _, doc = O.route(Qr, kr, off)
        O.topk(doc, min(w.k, d1 - docs_done))
        t_total += time.perf_counter() - t0
        tok_total += int(w.doc_tok_off[d1] - w.doc_tok_off[docs_done])
        docs_done = d1
        d = min(d * 2, 16000)
    return {"value": tok_total / t_total, "unit": "memory tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"layer 0, documents 0..{docs_done - 1} ({tok_total} memory tokens), route + top-k, "
                      f"fp64 numpy, {t_total:.1f} s"}


def route_only(w, n, dev):
    """One layer of the 100M-token store routed n times, after a 1 GiB device-to-device copy."""
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
    torch.cuda.synchronize()
    for _ in range(n):
        ops.route_scores(qr, kr, off, krbar_inv_norm=nrm)
    torch.cuda.synchronize()
    print(json.dumps({"route_only": n, "copy_bytes": a.numel() * 2, "n_chunks": w.n_chunks,
                      "source_hash": route_source_hash()}), flush=True)


def route_bytes_100M(w) -> int:
    """Algorithmic HBM bytes of one route call: K̄_r + stored norms + offsets + Qr + document scores."""
    G, H, D = w.n_chunks, w.H, w.D
    return G * H * D * 2 + G * H * 4 + 8 * (w.n_docs + 1) + w.B * w.T * H * D * 2 + 4 * w.B * w.n_docs


def traffic_from(fetch_csv: str, write_csv: str, w) -> dict:
    """Per-launch HBM bytes of the scan kernel from two rocprofv3 --pmc runs of --route-only
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by what the same counter
    reads for the 1 GiB device-to-device copy that --route-only performs first."""
    import csv

    def read(path, counter):
        kern, copy = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            if "route_mfma_kernel<8, true, " in r["Kernel_Name"]:
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
    return {"kernel": "route_mfma_kernel<8, true, POL_NT> (stored norms, non-temporal copies)",
            "workload": f"100M-token memory, one routed layer ({w.n_chunks:,} chunks), batch 1, "
                        f"{w.B * w.T} router rows, stored norms",
            "source_hash": route_source_hash(),
            "source_hash_note": "sha256 (first 16 hex) of route.hip + msa_internal.h with comments and "
                                "empty lines removed",
            "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
            "copy_reference": {"bytes": copy_bytes, "fetch_kib": fc, "write_kib": wc},
            "fetch_scale": fs, "write_scale": ws,
            "bytes_per_launch": int(round(fk * 1024 * fs + wk * 1024 * ws)),
            "algorithmic_bytes_per_launch": route_bytes_100M(w),
            "commands": ["cd /tmp && rocprofv3 --pmc FETCH_SIZE -d <out> -o run --output-format csv -- "
                         "python3 <repo>/bench.py --route-only 5",
                         "cd /tmp && rocprofv3 --pmc WRITE_SIZE -d <out> -o run --output-format csv -- "
                         "python3 <repo>/bench.py --route-only 5",
                         "python3 <repo>/bench.py --traffic-from <out>/run_counter_collection.csv (FETCH) "
                         "<out>/run_counter_collection.csv (WRITE)"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0)
    ap.add_argument("--route-only", type=int, default=0, metavar="N",
                    help="counter-collection mode: one 100M-token layer, a 1 GiB device copy (the reference for "
                         "scaling FETCH_SIZE/WRITE_SIZE), then N routing calls; prints one line and exits")
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
        print(f"bench.py measures one GPU's share only (--gpus {args.gpus} requested); the path runs on a "
              "single GPU and is not sharded across GPUs.", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_retrieval_memory_amd import ops
    from synth import workloads as C
    from synth import native
    from synth import splitmix as sm

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = C.workload("100M-18layer")
    if args.route_only:
        route_only(w, args.route_only, dev)
        return
    G, H, D, L, k = w.n_chunks, w.H, w.D, w.n_layers, w.k
    log(f"workload {w.name}: {w.n_docs} docs, {w.n_tok} tokens, {G} chunks, {L} layers")

    # ---------------------------------------------------------------- inputs
    t0 = time.time()
    bits = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    off_dev = torch.from_numpy(w.doc_chunk_off).to(dev)
    off_host = torch.from_numpy(w.doc_chunk_off.copy())
    krbar, knorm, qr, Q, Kl, Vl = [], [], [], [], [], []
    for layer in range(L):
        t = torch.empty((G, H, D), dtype=torch.int16, device=dev)
        native.fill_normal_bf16_device(t, w.seed, sm.TID_KRBAR, layer, 0)
        for g, row in C.pooled_plants(w, layer).items():
            t[g].copy_(bits(row))
        krbar.append(t)
        knorm.append(ops.krbar_inv_norms(t))      # built once with the store, like the store itself
        q = C.queries(w, layer)
        qr.append(bits(q["Qr"])); Q.append(bits(q["Q"])); Kl.append(bits(q["Kloc"])); Vl.append(bits(q["Vloc"]))
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
    doc = torch.empty((1, w.n_docs), dtype=torch.float32, device=dev)
    idx_d = torch.empty((1, k), dtype=torch.int32, device=dev)
    sc_d = torch.empty((1, k), dtype=torch.float32, device=dev)
    ws_r = ops.workspace(ops.route_workspace_bytes(1, w.T, H, D, G, w.n_docs), dev, "bench-route")
    ws_k = ops.workspace(ops.topk_workspace_bytes(1, w.n_docs, k), dev, "bench-topk")
    ws_rt = ops.workspace(ops.route_topk_workspace_bytes(1, w.T, H, D, G, w.n_docs, k), dev, "bench-route-topk")
    comp = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side_attn = torch.cuda.Stream()          # local-key attention partial, overlapping top-k + gather
    ev_scan, ev_local = torch.cuda.Event(), torch.cuda.Event()
    part = (torch.empty((1, w.Tq, w.Hq, D), dtype=torch.float32, device=dev),
            torch.empty((1, w.Tq, w.Hq, 2), dtype=torch.float32, device=dev))
    ev_ids = torch.cuda.Event()
    ev_fetch = torch.cuda.Event()
    n_ev = L * args.steps
    ev_r0 = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ev_r1 = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ev_a1 = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]

    def layer_step(layer, rec=None, split=False):
        """route + top-k (one call) -> device-side assembly from the pinned host tier -> attend, one stream, no
        host sync (the instrumented pass times msa_route_scores and msa_topk_docs as separate calls).
        split (a side measurement): the local-key half of the attention runs on a second stream once the scan
        is done (it needs nothing retrieved), overlapping top-k and the gather; the memory half then merges
        with it."""
        fused = rec is None and not split
        if fused:
            # scan, document max with the top-k's group maxima, top-k: one call
            ops.route_topk(qr[layer], krbar[layer], off_dev, k, krbar_inv_norm=knorm[layer], doc_scores=doc,
                           top_idx=idx_d, top_scores=sc_d, ws=ws_rt)
        else:
            if rec is not None:
                ev_r0[rec].record(comp)
            ops.route_scores(qr[layer], krbar[layer], off_dev, doc_scores=doc, ws=ws_r, krbar_inv_norm=knorm[layer])
            if rec is not None:
                ev_r1[rec].record(comp)
        if split:
            ev_scan.record(comp)
            side_attn.wait_event(ev_scan)
            ops.sparse_attn_local_partial(Q[layer], Kl[layer], Vl[layer], k, w.rope_base, part=part,
                                          stream=side_attn)
            ev_local.record(side_attn)
        if not fused:
            ops.topk_docs(doc, k, top_idx=idx_d, top_scores=sc_d, ws=ws_k)
        ops.gather_docs(idx_d, store, off_dev, staging, Mmax, mem_len=ml_dev)
        if split:
            comp.wait_event(ev_local)
            ops.sparse_attn_memory_merge(Q[layer], w.Tl, H, staging, staging[:, :, 1], 2 * H * D, Mmax, ml_dev, k,
                                         part, w.rope_base, out=O_out)
        else:
            ops.sparse_attn_decode(Q[layer], Kl[layer], Vl[layer], staging, staging[:, :, 1], 2 * H * D, Mmax,
                                   ml_dev, k, w.rope_base, out=O_out)
        if rec is not None:
            ev_a1[rec].record(comp)

    def layer_step_host_fetch(layer):
        """The same layer with the ids sent to the host and the content copied by hipMemcpyAsync on a side stream."""
        ops.route_scores(qr[layer], krbar[layer], off_dev, doc_scores=doc, ws=ws_r, krbar_inv_norm=knorm[layer])
        ops.topk_docs(doc, k, top_idx=idx_d, top_scores=sc_d, ws=ws_k)
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
    for s_ in range(args.warmup):
        for layer in range(L):
            layer_step(layer)
            if s_ == 0:
                selected.append(idx_d.cpu().numpy()[0].copy())
    torch.cuda.synchronize()
    needles_found = sum(int(d in selected[layer]) for layer in range(L) for (_, d) in C.planted_docs(w, layer))
    log(f"warmup done; planted needles retrieved: {needles_found}/{L * w.n_needles}")

    # ----------------------------------------------------------------- timed
    # No events inside the timed steps: each recorded timing event idles the stream for ~5 us.
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s_ in range(args.steps):
        for layer in range(L):
            layer_step(layer)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_step = elapsed * 1e3 / args.steps
    tokens_per_s = w.n_tok * L * args.steps / elapsed
    log(f"timed {args.steps} steps: {ms_step:.2f} ms/step")
    # the same steps with the attention split over two streams (local half overlapping top-k + gather)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        for layer in range(L):
            layer_step(layer, split=True)
    torch.cuda.synchronize()
    ms_step_split = (time.perf_counter() - t0) * 1e3 / args.steps
    log(f"the same steps with the attention split over two streams: {ms_step_split:.2f} ms/step")
    # per-layer statistics from a second, instrumented pass of the same steps
    for s_ in range(args.steps):
        for layer in range(L):
            layer_step(layer, rec=s_ * L + layer)
    torch.cuda.synchronize()
    route_ms = np.array([a.elapsed_time(b) for a, b in zip(ev_r0, ev_r1)])
    layer_ms = np.array([a.elapsed_time(b) for a, b in zip(ev_r0, ev_a1)])

    # ------------------------------------------------------- side measurements
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def time_ms(fn, reps):
        """Median over reps of one call bracketed by its own pair of events on the current
        stream, so host launch overhead between calls is not counted as device time."""
        fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b_ in evs:
            a.record()
            fn()
            b_.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b_) for a, b_ in evs]))

    # the step with the host round trip and hipMemcpyAsync fetch
    for layer in range(L):
        layer_step_host_fetch(layer)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        for layer in range(L):
            layer_step_host_fetch(layer)
    torch.cuda.synchronize()
    host_fetch_step_ms = (time.perf_counter() - t0) * 1e3 / 3
    q1 = Q[0][:, -1:].contiguous()
    decode_attn_us = 1e3 * time_ms(lambda: ops.sparse_attn_decode(q1, Kl[0], Vl[0], staging, staging[:, :, 1], 2 * H * D,
                                                                  Mmax, ml_dev, k, w.rope_base), 50)
    attn_us = 1e3 * time_ms(lambda: ops.sparse_attn_decode(Q[0], Kl[0], Vl[0], staging, staging[:, :, 1], 2 * H * D,
                                                           Mmax, ml_dev, k, w.rope_base, out=O_out), 50)
    # attention backward at the step's shape (Tq = Tl = 128, 32 q-heads over 8 kv-heads, the assembled memory)
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
    # the same backward given the forward's output and log-sum-exp (no statistics pass)
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
    del ab_out
    topk_us = 1e3 * time_ms(lambda: ops.topk_docs(doc, k, top_idx=idx_d, top_scores=sc_d, ws=ws_k), 50)
    gather_us = 1e3 * time_ms(lambda: ops.gather_docs(idx_d, store, off_dev, staging, Mmax, mem_len=ml_dev), 50)
    route_nonorm_ms = time_ms(lambda: ops.route_scores(qr[0], krbar[0], off_dev, doc_scores=doc, ws=ws_r), 10)
    # routing-store update: delete 10% of one layer's documents (store + norms compacted into new buffers)
    keep_d = torch.from_numpy((np.random.default_rng(9).random(w.n_docs) >= 0.1).astype(np.uint8)).to(dev)
    del_out = (torch.empty_like(krbar[0]), torch.empty_like(knorm[0]), torch.empty_like(off_dev),
               torch.empty(w.n_docs, dtype=torch.int32, device=dev), torch.empty(2, dtype=torch.int64, device=dev))
    delete_ms = time_ms(lambda: ops.store_delete(krbar[0], off_dev, keep_d, inv_norm=knorm[0], out=del_out), 5)
    kept_chunks = int(del_out[4][1].item())
    delete_bytes = 2 * kept_chunks * H * (D * 2 + 4) + w.n_docs * (1 + 8 + 4 + 8)
    del del_out
    # routing-score backward over one 100M-token layer: every document gets an upstream gradient
    _, ch0 = ops.route_scores(qr[0], krbar[0], off_dev, want_chunk_scores=True, ws=ws_r, krbar_inv_norm=knorm[0])
    d_doc = torch.from_numpy(np.random.default_rng(10).standard_normal((1, w.n_docs)).astype(np.float32)).to(dev)
    bwd_out = (torch.empty((1, w.T, H, D), dtype=torch.float32, device=dev),
               torch.empty((1, w.n_docs, H, D), dtype=torch.float32, device=dev),
               torch.empty((1, w.n_docs, 2), dtype=torch.int32, device=dev))
    ws_b = ops.workspace(ops.route_backward_workspace_bytes(1, w.T, H, D, w.n_docs), dev, "bench-route-bwd")
    bwd_ms = time_ms(lambda: ops.route_scores_backward(qr[0], krbar[0], off_dev, ch0, d_doc, krbar_inv_norm=knorm[0],
                                                       dQr=bwd_out[0], dKsel=bwd_out[1], sel=bwd_out[2], ws=ws_b), 5)
    # algorithmic bytes: chunk scores, offsets and upstream gradients read; each document's selected
    # Krbar row read once; its fp32 key gradient and (chunk, token) written; Qr read, dQr written
    bwd_bytes = (G * 4 + (w.n_docs + 1) * 8 + w.n_docs * 4 + w.n_docs * H * D * (2 + 4) + w.n_docs * 8
                 + w.T * H * D * (2 + 4))
    bwd_flops = 2.0 * w.n_docs * w.T * H * D          # the recomputed token scores of the selected chunks
    del bwd_out, ch0

    log("side measurements: host-fetch step, attention, top-k, gather done")
    # the 10M-token batch-16 scan: 16 queries x 64 tokens over 165K chunks (matrix-core bound)
    w3 = C.workload("10M-batch16")
    kr3 = torch.empty((w3.n_chunks, H, D), dtype=torch.int16, device=dev)
    native.fill_normal_bf16_device(kr3, w3.seed, sm.TID_KRBAR, 0, 0)
    for g, row in C.pooled_plants(w3, 0).items():
        kr3[g].copy_(bits(row))
    # two copies of the 338 MB store, used in turn, so the 256 MB Infinity Cache cannot serve a scan
    kr3 = (kr3, kr3.clone())
    kn3 = ops.krbar_inv_norms(kr3[0])
    qr3 = bits(C.queries(w3, 0)["Qr"])
    off3 = torch.from_numpy(w3.doc_chunk_off).to(dev)
    doc3 = torch.empty((w3.B, w3.n_docs), dtype=torch.float32, device=dev)
    ws3 = ops.workspace(ops.route_workspace_bytes(w3.B, w3.T, H, D, w3.n_chunks, w3.n_docs), dev, "bench-route3")
    turn = [0]

    def scan3():
        turn[0] ^= 1
        ops.route_scores(qr3, kr3[turn[0]], off3, doc_scores=doc3, ws=ws3, krbar_inv_norm=kn3)
    scan3_ms = time_ms(scan3, 20)
    scan3_tflops = 2.0 * w3.B * w3.T * H * D * w3.n_chunks / (scan3_ms * 1e-3) / 1e12
    del kr3, kn3, doc3
    # achievable dense bf16 rate on this GPU: a plain library GEMM (hipBLASLt via torch), 8192^3
    ga = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
    gb = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
    gemm_ms = time_ms(lambda: torch.matmul(ga, gb), 10)
    gemm_tflops = 2.0 * 8192 ** 3 / (gemm_ms * 1e-3) / 1e12
    del ga, gb

    log(f"10M batch-16 scan: {scan3_ms:.3f} ms")
    # pooling throughput, then the interleave workload's rounds (10M tokens, 4 queries, 3 rounds, top-8)
    from sparse_retrieval_memory_amd.interleave import Interleave
    w5 = C.workload("10M-interleave")
    E = w5.row_elems
    pooled5 = tuple(torch.empty((w5.n_chunks, H, D), dtype=torch.int16, device=dev) for _ in range(3))
    plants5 = C.raw_plants(w5)
    pool_us, pool_bytes = [], 0
    d0 = 0
    while d0 < w5.n_docs:
        d1 = min(max(int(np.searchsorted(w5.doc_tok_off, w5.doc_tok_off[d0] + 1_000_000, side="right")) - 1, d0 + 1),
                 w5.n_docs)
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
        d0 = d1
    # router-key encoding of the same corpus from d_model = 2560 hidden states (1M-token slabs)
    DM = 2560
    w_kr = torch.empty((H * D, DM), dtype=torch.int16, device=dev)
    native.fill_normal_bf16_device(w_kr, w5.seed, sm.TID_WKR, 0, 0)
    enc_out = torch.empty((w5.n_chunks, H, D), dtype=torch.int16, device=dev)
    enc_ms, enc_bytes, enc_flops = [], 0, 0
    d0 = 0
    while d0 < w5.n_docs:
        d1 = min(max(int(np.searchsorted(w5.doc_tok_off, w5.doc_tok_off[d0] + 1_000_000, side="right")) - 1, d0 + 1),
                 w5.n_docs)
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
        d0 = d1
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
    log(f"interleave: 3 rounds in {interleave_ms:.2f} ms, chains {chains_ok}/{w5.B}")

    # ---------------------------------------------------------------- report
    route_bytes = route_bytes_100M(w)
    route_avg_s = float(route_ms.mean()) * 1e-3
    achieved = route_bytes / route_avg_s / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        if tr.get("source_hash") == route_source_hash():
            traffic = tr.get("bytes_per_launch")
    cpu = None
    if args.cpu_baseline_seconds > 0:
        log("timing the oracle on the host ...")
        cpu = cpu_baseline(w, args.cpu_baseline_seconds)
    pct = lambda a: {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
                     "p90": float(np.percentile(a, 90)), "mean": float(np.mean(a)), "n": int(len(a))}
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
                   "step": "18 x (route + top-k (msa_route_topk) -> assemble selected K/V from the pinned host "
                           "tier by a device kernel -> attend), one stream, no host round trip"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "msa_route_scores (scan + document max), bytes = Krbar + its stored norms + "
                               "doc offsets + Qr + doc scores"},
        "cpu_baseline": cpu,
        "step_ms_split_attention": ms_step_split,
        "route_ms_per_layer": pct(route_ms),
        "layer_latency_ms": pct(layer_ms),
        "krbar_scan_GBps": achieved,
        "memory_tokens_per_s_per_layer": w.n_tok / route_avg_s,
        "host_fetch_step_ms": host_fetch_step_ms,
        "route_ms_norms_in_kernel": route_nonorm_ms,
        "topk_us": topk_us,
        "gather_us": gather_us,
        "attn_us": {"tq128": attn_us, "tq1_decode": decode_attn_us},
        "attn_backward_tq128": {"us": attn_bwd_us, "memory_entries": n_mem,
                                "TFLOPs": attn_bwd_flops / (attn_bwd_us * 1e-6) / 1e12,
                                "us_with_saved_stats": attn_bwd_saved_us, "forward_with_lse_us": attn_fwd_lse_us},
        "scan_10M_batch16": {"ms": scan3_ms, "TFLOPs": scan3_tflops,
                             "mfma_frac": scan3_tflops / MFMA_BF16_PEAK_TFLOPS,
                             "gemm_bf16_8192_TFLOPs": gemm_tflops,
                             "frac_of_gemm": scan3_tflops / gemm_tflops},
        "pool_GBps": pool_bytes / (sum(pool_us) * 1e-6) / 1e9,
        "store_delete_10pct_100M_layer": {"ms": delete_ms, "GBps": delete_bytes / (delete_ms * 1e-3) / 1e9,
                                          "frac_of_8TBps": delete_bytes / (delete_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "route_backward_100M_layer": {"ms": bwd_ms, "GBps": bwd_bytes / (bwd_ms * 1e-3) / 1e9,
                                      "frac_of_8TBps": bwd_bytes / (bwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                      "recompute_TFLOPs": bwd_flops / (bwd_ms * 1e-3) / 1e12,
                                      "docs_with_gradient": w.n_docs},
        "encode_router_keys_10M": {"ms": float(sum(enc_ms)), "GBps": enc_bytes / (sum(enc_ms) * 1e-3) / 1e9,
                                   "frac_of_8TBps": enc_bytes / (sum(enc_ms) * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                   "d_model": 2560, "projection_TFLOPs_equiv": enc_flops / (sum(enc_ms) * 1e-3) / 1e12},
        "interleave_10M_b4_3rounds_ms": interleave_ms,
        "interleave_round_ms": round_ms,
        "interleave_chains_recovered": f"{chains_ok}/{w5.B}",
        "needles_retrieved": f"{needles_found}/{L * w.n_needles}",
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
