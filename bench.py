"""Benchmark of the MSA routed step on one MI355X.

Workload (default): a 100M-token memory of 200,000 synthetic documents
(lengths uniform on [64, 936], mean 500), chunk 64 -> 1.66M pooled chunks,
18 routed layers, each with its own HBM-resident Krbar store (bf16, 8 x 128 per
chunk, 61 GB in total) and its own 128-token router query (batch 1).  One step
runs the 18 layers in sequence; a layer is

    route (scan of all Krbar + document max) -> top-16 documents ->
    ids to the host -> hipMemcpyAsync of the selected pooled K/V from pinned
    host memory on a side stream -> GQA attention (32 q-heads, 128 query rows,
    128 local tokens) over [fetched memory ++ local KV].

Inputs are generated on the device before timing (seeded, synthetic); the
pooled content store (Kbar|Vbar, 6.8 GB) sits in pinned host memory and is
shared by all layers.  The printed JSON line reports memory tokens routed per
second (per query), the step latency, the roofline of the routing call and
the oracle's CPU throughput on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_route_100M.json")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def route_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("route.hip", "msa_internal.h"):
        h.update(open(os.path.join(ROOT, "sparse_retrieval_memory_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def cpu_baseline(w, seconds: float):
    """Oracle route + top-k on a bounded slice of layer 0 (documents from the start)."""
    from oracle import msa_oracle as O
    from synth import configs as C
    cores = len(os.sched_getaffinity(0))
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share only (--gpus {args.gpus} requested); the path is not "
              "sharded across GPUs in this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_retrieval_memory_amd import ops
    from synth import configs as C
    from synth import native
    from synth import splitmix as sm

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = C.config(4)
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
    ws_r = ops.workspace(ops.route_workspace_bytes(1, w.T, H, D, G, w.n_docs), dev, "bench-route")
    ws_k = ops.workspace(ops.topk_workspace_bytes(1, w.n_docs, k), dev, "bench-topk")
    comp = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ev_ids = torch.cuda.Event()
    ev_fetch = torch.cuda.Event()
    n_ev = L * args.steps
    ev_r0 = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ev_r1 = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ev_a1 = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    selected = []

    def layer_step(layer, rec=None):
        if rec is not None:
            ev_r0[rec].record(comp)
        ops.route_scores(qr[layer], krbar[layer], off_dev, doc_scores=doc, ws=ws_r, krbar_inv_norm=knorm[layer])
        if rec is not None:
            ev_r1[rec].record(comp)
        idx, _ = ops.topk_docs(doc, k, ws=ws_k)
        top_host.copy_(idx, non_blocking=True)
        ev_ids.record(comp)
        ev_ids.synchronize()
        ml = ops.fetch_docs(top_host, store, off_host, staging, Mmax, side, ev_fetch)
        ml_host.copy_(ml)
        ml_dev.copy_(ml_host, non_blocking=True)
        comp.wait_event(ev_fetch)
        ops.sparse_attn_decode(Q[layer], Kl[layer], Vl[layer], staging, staging[:, :, 1], 2 * H * D, Mmax, ml_dev,
                               k, w.rope_base, out=O_out)
        if rec is not None:
            ev_a1[rec].record(comp)
        return top_host

    # ---------------------------------------------------------------- warmup
    for s in range(args.warmup):
        for layer in range(L):
            ids = layer_step(layer)
            if s == 0:
                selected.append(ids.numpy()[0].copy())
    torch.cuda.synchronize()
    needles_found = sum(int(d in selected[layer]) for layer in range(L) for (_, d) in C.planted_docs(w, layer))
    log(f"warmup done; planted needles retrieved: {needles_found}/{L * w.n_needles}")

    # ----------------------------------------------------------------- timed
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        for layer in range(L):
            layer_step(layer, rec=s * L + layer)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_step = elapsed * 1e3 / args.steps
    route_ms = np.array([a.elapsed_time(b) for a, b in zip(ev_r0, ev_r1)])
    layer_ms = np.array([a.elapsed_time(b) for a, b in zip(ev_r0, ev_a1)])
    tokens_per_s = w.n_tok * L * args.steps / elapsed

    # ------------------------------------------------------- side measurements
    # decode (Tq = 1) attention, device-side gather path, pooling throughput
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    q1 = Q[0][:, -1:].contiguous()
    e0.record()
    for _ in range(50):
        ops.sparse_attn_decode(q1, Kl[0], Vl[0], staging, staging[:, :, 1], 2 * H * D, Mmax, ml_dev, k, w.rope_base)
    e1.record(); torch.cuda.synchronize()
    decode_attn_us = e0.elapsed_time(e1) * 1e3 / 50
    e0.record()
    for _ in range(50):
        ops.sparse_attn_decode(Q[0], Kl[0], Vl[0], staging, staging[:, :, 1], 2 * H * D, Mmax, ml_dev, k,
                               w.rope_base, out=O_out)
    e1.record(); torch.cuda.synchronize()
    attn_us = e0.elapsed_time(e1) * 1e3 / 50
    store_dev_view = store  # mapped pinned memory, read by the gather kernel over PCIe
    gstag = torch.empty_like(staging)
    e0.record()
    for layer in range(L):
        dscore = ops.route_scores(qr[layer], krbar[layer], off_dev, doc_scores=doc, ws=ws_r,
                                  krbar_inv_norm=knorm[layer])
        idx, _ = ops.topk_docs(dscore, k, ws=ws_k)
        mld = ops.gather_docs(idx, store_dev_view, off_dev, gstag, Mmax)
        ops.sparse_attn_decode(Q[layer], Kl[layer], Vl[layer], gstag, gstag[:, :, 1], 2 * H * D, Mmax, mld, k,
                               w.rope_base, out=O_out)
    e1.record(); torch.cuda.synchronize()
    gather_step_ms = e0.elapsed_time(e1)

    # the same scan without stored norms (the kernel derives them from the tiles it streams)
    e0.record()
    for layer in range(L):
        ops.route_scores(qr[layer], krbar[layer], off_dev, doc_scores=doc, ws=ws_r)
    e1.record(); torch.cuda.synchronize()
    route_nonorm_ms = e0.elapsed_time(e1) / L

    # pooling throughput on a 1M-token slab of the 10M-token interleave corpus
    w5 = C.config(5)
    d1 = int(np.searchsorted(w5.doc_tok_off, 1_000_000))
    ntok, nch = int(w5.doc_tok_off[d1]), int(w5.doc_chunk_off[d1])
    raw = []
    for tid in (sm.TID_K, sm.TID_V, sm.TID_KR):
        t = torch.empty((ntok, H, D), dtype=torch.int16, device=dev)
        native.fill_normal_bf16_device(t, w5.seed, tid, 0, 0)
        raw.append(t)
    tok_off5 = torch.from_numpy(w5.doc_tok_off[:d1 + 1].copy()).to(dev)
    ch_off5 = torch.from_numpy(w5.doc_chunk_off[:d1 + 1].copy()).to(dev)
    pooled = tuple(torch.empty((nch, H, D), dtype=torch.int16, device=dev) for _ in range(3))
    for _ in range(2):
        ops.pool_chunks(*raw, tok_off5, ch_off5, nch, w5.chunk, w5.rope_base, out=pooled)
    e0.record()
    for _ in range(10):
        ops.pool_chunks(*raw, tok_off5, ch_off5, nch, w5.chunk, w5.rope_base, out=pooled)
    e1.record(); torch.cuda.synchronize()
    pool_us = e0.elapsed_time(e1) * 1e3 / 10
    pool_bytes = 3 * ntok * H * D * 2 + 3 * nch * H * D * 2
    del raw, pooled

    # ---------------------------------------------------------------- report
    route_bytes = G * H * D * 2 + G * H * 4 + 8 * (w.n_docs + 1) + w.B * w.T * H * D * 2 + 4 * w.B * w.n_docs
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
                   "step": "18 x (route -> top-k -> ids to host -> hipMemcpyAsync fetch (side stream) -> attend)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "msa_route_scores (scan + document max), bytes = Krbar + its stored norms + "
                               "doc offsets + Qr + doc scores"},
        "cpu_baseline": cpu,
        "route_ms_per_layer": {"mean": float(route_ms.mean()), "p10": float(np.percentile(route_ms, 10)),
                               "p90": float(np.percentile(route_ms, 90))},
        "layer_latency_ms": {"mean": float(layer_ms.mean()), "p10": float(np.percentile(layer_ms, 10)),
                             "p90": float(np.percentile(layer_ms, 90))},
        "krbar_scan_GBps": achieved,
        "route_ms_per_layer_norms_in_kernel": route_nonorm_ms,
        "memory_tokens_per_s_per_layer": w.n_tok / route_avg_s,
        "attn_us": {"tq128": attn_us, "tq1_decode": decode_attn_us},
        "device_gather_18layer_step_ms": gather_step_ms,
        "pool_GBps": pool_bytes / (pool_us * 1e-6) / 1e9,
        "needles_retrieved": f"{needles_found}/{L * w.n_needles}",
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
