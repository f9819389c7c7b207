"""Memory Interleave: rounds of route -> top-k -> fetch -> attend (host control loop).

Pages: medium write-up sec. 4C and b-lab.team summary sec. 3 -- retrieval and
context expansion repeat, and the documents found in one round become part of
the next round's query.  Reading (the pages give no mechanics): each round
routes with the original router rows plus the pooled router keys of every
chunk retrieved so far (retrieval order), never selects a document twice, and
attends over all retrieved documents (retrieval order) with the global RoPE
offset equal to their count.

This module only sequences the library's calls; every step runs in libmsa's
kernels (``msa_append_router_rows``, ``msa_route_topk`` (``msa_route_scores`` +
``msa_topk_docs`` for k > 32),
``msa_gather_docs`` or ``msa_fetch_docs``, ``msa_sparse_attn_decode``).  The
one host round trip per round is the selected ids: the host sizes the next
round's router rows and the staging buffer from them.  The content is
assembled on the device from the mapped pinned tier by default
(``fetch="gather"``); ``fetch="copy"`` uses host-driven hipMemcpyAsync copies
on a side stream instead.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

from . import ops


@dataclass
class Round:
    top_idx: np.ndarray            # int32 [B, k], this round's new documents (rank order)
    top_scores: np.ndarray         # float32 [B, k]
    retrieved: np.ndarray          # int32 [B, k * (round + 1)], retrieval order
    n_rows: int                    # router rows routed this round (padded batch)
    O: torch.Tensor                # fp32 [B, Tq, Hq, D] on the device
    doc_scores: Optional[torch.Tensor] = None
    ms: Optional[float] = None     # device time from the round's first launch to O (timing=True)


@dataclass
class Interleave:
    """Device-resident inputs of one interleave run and reusable buffers."""
    krbar: torch.Tensor                       # bf16 [n_chunks, H, D] (device)
    doc_chunk_off: torch.Tensor               # int64 [n_docs + 1] (device)
    doc_chunk_off_host: torch.Tensor          # int64 [n_docs + 1] (host)
    content: torch.Tensor                     # bf16 [n_chunks, 2, H, D] pinned host tier
    krbar_inv_norm: Optional[torch.Tensor] = None
    rope_base: float = 1.0e6
    side: Optional[torch.cuda.Stream] = None
    _bufs: dict = field(default_factory=dict)

    def run(self, Qr, Q, Kloc, Vloc, k: int, rounds: int, keep_scores: bool = False,
            fetch: str = "gather", timing: bool = False) -> List[Round]:
        if fetch not in ("gather", "copy"):
            raise ValueError(f"fetch must be 'gather' or 'copy', not {fetch!r}")
        dev = Qr.device
        B, T0, H, D = Qr.shape
        off_h = self.doc_chunk_off_host.numpy()
        n_docs = len(off_h) - 1
        n_chunks_of = np.diff(off_h)
        exclude = torch.zeros((B, n_docs), dtype=torch.uint8, device=dev)
        retrieved = np.zeros((B, 0), dtype=np.int32)
        side = self.side if self.side is not None else torch.cuda.Stream(device=dev)
        fetched = torch.cuda.Event()
        out: List[Round] = []
        marks = []
        for r in range(rounds):
            if timing:
                marks.append([torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)])
                marks[-1][0].record()
            if r == 0:
                rows, n_rows = Qr, T0
            else:
                n_rows = T0 + int(n_chunks_of[retrieved].sum(axis=1).max())
                ids = torch.from_numpy(retrieved).to(dev, non_blocking=True)
                rows, _ = ops.append_router_rows(Qr, self.krbar, self.doc_chunk_off, ids, n_rows,
                                                 doc_exclude=exclude)
            if k <= 32:          # scan, document max and top-k in one call
                doc, idx, sc = ops.route_topk(rows, self.krbar, self.doc_chunk_off, k,
                                              doc_exclude=exclude if r else None, krbar_inv_norm=self.krbar_inv_norm)
            else:
                doc = ops.route_scores(rows, self.krbar, self.doc_chunk_off, doc_exclude=exclude if r else None,
                                       krbar_inv_norm=self.krbar_inv_norm)
                idx, sc = ops.topk_docs(doc, k)
            new = idx.cpu().numpy()
            retrieved = np.concatenate([retrieved, new], axis=1).astype(np.int32)
            Mmax = int(n_chunks_of[retrieved].sum(axis=1).max())
            staging = torch.empty((B, Mmax, 2, H, D), dtype=Qr.dtype, device=dev)
            if fetch == "gather":
                ml = ops.gather_docs(torch.from_numpy(retrieved).to(dev, non_blocking=True), self.content,
                                     self.doc_chunk_off, staging, Mmax)
            else:
                ml = ops.fetch_docs(torch.from_numpy(retrieved), self.content, self.doc_chunk_off_host, staging,
                                    Mmax, side, fetched)
                torch.cuda.current_stream().wait_event(fetched)
                ml = ml.to(dev)
            O = ops.sparse_attn_decode(Q, Kloc, Vloc, staging, staging[:, :, 1], 2 * H * D, Mmax, ml,
                                       retrieved.shape[1], self.rope_base)
            if timing:
                marks[-1][1].record()
            out.append(Round(top_idx=new, top_scores=sc.cpu().numpy(), retrieved=retrieved.copy(), n_rows=n_rows,
                             O=O, doc_scores=doc if keep_scores else None))
        if timing:
            torch.cuda.synchronize(dev)
            for rd, (a, b) in zip(out, marks):
                rd.ms = a.elapsed_time(b)
        return out
