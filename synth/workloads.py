"""The five synthetic workloads and their planted structure.

Shapes and sizes follow the workloads the pages measure on (a 32K-token tiny
memory, RULER-sized 1M memories, TriviaQA-sized 10M memories and the 100M
MS MARCO scale); the data itself is synthetic and seeded (see
``synth.splitmix``).  This module only decides *what the inputs are*; it holds
none of the method's arithmetic (no RoPE, pooling, cosine, top-k or softmax).

Plants are the only structured part:

* ``mean_raw``  every raw router-key token of one needle document is the
  query's mean router vector plus 0.1 * noise;
* ``token``     one pooled router-key chunk of each needle document is one
  query token's router vector plus 0.1 * noise;
* ``mean``      as ``token`` but planted on the query's mean router vector;
* ``chain``     per query a 3-document chain A -> B -> C on raw router keys:
  a chunk of A matches a query token, another chunk of A and a chunk of B
  share a random vector u, another chunk of B and a chunk of C share w.

Planted values are rounded to bf16 on the host (round-to-nearest-even of the
float64 value).
"""

from __future__ import annotations

import dataclasses
import functools
import math
from typing import Dict, List, Tuple

import numpy as np

from . import splitmix as sm
from . import native


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    n_docs: int
    length_law: str          # const512 | uniform256_1792 | lognormal400 | uniform64_936 | custom
    B: int                   # independent queries
    T: int                   # router rows per query (first round for interleave)
    Tq: int                  # attention query rows
    Tl: int                  # local KV length
    k: int                   # documents selected
    n_layers: int = 1
    H: int = 8               # KV heads = router heads
    D: int = 128
    Hq: int = 32
    chunk: int = 64
    rope_base: float = 1.0e6
    pooled: str = "direct"   # "raw": pool from raw tokens; "direct": pooled drawn directly
    plant: str = "token"     # mean_raw | token | mean | chain | none
    n_needles: int = 10      # token/mean plants per layer
    rounds: int = 1          # interleave rounds
    custom_lengths: Tuple[int, ...] = ()

    # ---------------------------------------------------------------- layout
    @functools.cached_property
    def doc_len(self) -> np.ndarray:
        n, s = self.n_docs, self.seed
        if self.length_law == "const512":
            L = np.full(n, 512, dtype=np.int64)
        elif self.length_law == "uniform256_1792":
            L = sm.uniform_int(s, sm.TID_LEN, 0, 0, n, 256, 1792)
        elif self.length_law == "uniform64_936":
            L = sm.uniform_int(s, sm.TID_LEN, 0, 0, n, 64, 936)
        elif self.length_law == "lognormal400":
            # median 400, sigma sqrt(2 ln 1.25) so the mean is 500; clipped to [64, 8192]
            z = sm.normal_f64(s, sm.TID_LEN, 0, 0, n)
            sigma = math.sqrt(2.0 * math.log(1.25))
            L = np.clip(np.rint(np.exp(math.log(400.0) + sigma * z)), 64, 8192).astype(np.int64)
        elif self.length_law == "custom":
            L = np.asarray(self.custom_lengths, dtype=np.int64)
            assert L.shape == (n,)
        else:
            raise ValueError(self.length_law)
        L.setflags(write=False)
        return L

    @functools.cached_property
    def doc_n_chunks(self) -> np.ndarray:
        return (self.doc_len + self.chunk - 1) // self.chunk

    @functools.cached_property
    def doc_tok_off(self) -> np.ndarray:
        off = np.zeros(self.n_docs + 1, dtype=np.int64)
        np.cumsum(self.doc_len, out=off[1:])
        return off

    @functools.cached_property
    def doc_chunk_off(self) -> np.ndarray:
        off = np.zeros(self.n_docs + 1, dtype=np.int64)
        np.cumsum(self.doc_n_chunks, out=off[1:])
        return off

    @property
    def n_tok(self) -> int:
        return int(self.doc_tok_off[-1])

    @property
    def n_chunks(self) -> int:
        return int(self.doc_chunk_off[-1])

    @property
    def row_elems(self) -> int:
        return self.H * self.D

    def doc_of_chunk(self, g) -> np.ndarray:
        return np.searchsorted(self.doc_chunk_off, np.asarray(g), side="right") - 1

    def describe(self) -> dict:
        return dict(name=self.name, seed=self.seed, n_docs=self.n_docs, n_tok=self.n_tok,
                    n_chunks=self.n_chunks, B=self.B, T=self.T, Tq=self.Tq, Tl=self.Tl,
                    k=self.k, n_layers=self.n_layers, H=self.H, D=self.D, Hq=self.Hq,
                    chunk=self.chunk, pooled=self.pooled, plant=self.plant)


# ------------------------------------------------------------------ workloads
# name -> (default seed, fields); the seeds are fixed so stored expected values stay valid
_WORKLOADS = {
    "tiny-32K": (1, dict(n_docs=64, length_law="const512", B=1, T=32, Tq=32, Tl=32, k=4,
                         pooled="raw", plant="mean_raw", n_needles=1)),
    "1M": (2, dict(n_docs=1000, length_law="uniform256_1792", B=1, T=128, Tq=128, Tl=128, k=16,
                   pooled="direct", plant="token", n_needles=10)),
    "10M-batch16": (3, dict(n_docs=20000, length_law="lognormal400", B=16, T=64, Tq=64, Tl=64, k=16,
                            pooled="direct", plant="token", n_needles=16)),
    "100M-18layer": (4, dict(n_docs=200000, length_law="uniform64_936", B=1, T=128, Tq=128, Tl=128,
                             k=16, n_layers=18, pooled="direct", plant="token", n_needles=10)),
    "10M-interleave": (5, dict(n_docs=20000, length_law="lognormal400", B=4, T=128, Tq=128, Tl=128,
                               k=8, pooled="raw", plant="chain", n_needles=0, rounds=3)),
}
WORKLOAD_NAMES = tuple(_WORKLOADS)


def workload(name: str, seed: int | None = None, **over) -> Workload:
    """The named workload with its default seed (or ``seed``), fields overridden by ``over``."""
    if name not in _WORKLOADS:
        raise ValueError(f"unknown workload {name!r}; known: {', '.join(WORKLOAD_NAMES)}")
    s0, fields = _WORKLOADS[name]
    w = Workload(name, s0 if seed is None else seed, **fields)
    return dataclasses.replace(w, **over) if over else w


# ---------------------------------------------------------------- generation
def normal_bf16(seed, tid, layer, start, count) -> np.ndarray:
    """bf16 bits; uses the C host generator when built, else numpy (same bits)."""
    if native.available():
        return native.normal_bf16(seed, tid, layer, start, count)
    return sm.normal_bf16(seed, tid, layer, start, count)


def _as_f64(bits: np.ndarray) -> np.ndarray:
    return sm.bf16_bits_to_f32(bits).astype(np.float64)


def queries(w: Workload, layer: int = 0) -> Dict[str, np.ndarray]:
    """Router queries Qr [B,T,H,D], attention Q [B,Tq,Hq,D], local K/V [B,Tl,H,D] (bf16 bits)."""
    H, D = w.H, w.D
    out = {
        "Qr": normal_bf16(w.seed, sm.TID_QR, layer, 0, w.B * w.T * H * D).reshape(w.B, w.T, H, D),
        "Q": normal_bf16(w.seed, sm.TID_Q, layer, 0, w.B * w.Tq * w.Hq * D).reshape(w.B, w.Tq, w.Hq, D),
        "Kloc": normal_bf16(w.seed, sm.TID_KLOC, layer, 0, w.B * w.Tl * H * D).reshape(w.B, w.Tl, H, D),
        "Vloc": normal_bf16(w.seed, sm.TID_VLOC, layer, 0, w.B * w.Tl * H * D).reshape(w.B, w.Tl, H, D),
    }
    return out


def _picks(w: Workload, layer: int, count: int) -> np.ndarray:
    return sm.raw_u64(w.seed, sm.TID_PICK, layer, 0, count)


@functools.lru_cache(maxsize=64)
def needles(w: Workload, layer: int = 0) -> Tuple[Tuple[int, int, int, int], ...]:
    """Token/mean plants: tuples (query b, doc, chunk index in doc, token t or -1)."""
    if w.plant not in ("token", "mean", "mean_raw"):
        return ()
    n = w.n_needles
    u = _picks(w, layer, 64 * n + 64)
    docs, toks_per_b = [], {}
    out = []
    j = 0
    for i in range(n):
        b = i % w.B
        while True:
            d = int((u[j] >> np.uint64(32)) * np.uint64(w.n_docs) >> np.uint64(32)); j += 1
            if d not in docs:
                break
        docs.append(d)
        if w.plant == "token":
            used = toks_per_b.setdefault(b, set())
            while True:
                t = int((u[j] >> np.uint64(32)) * np.uint64(w.T) >> np.uint64(32)); j += 1
                if t not in used:
                    break
            used.add(t)
        else:
            t = -1
        nc = int(w.doc_n_chunks[d])
        c = int((u[j] >> np.uint64(32)) * np.uint64(nc) >> np.uint64(32)); j += 1
        out.append((b, d, c, t))
    return tuple(out)


def _plant_target(w: Workload, Qr_f64: np.ndarray, b: int, t: int) -> np.ndarray:
    if t >= 0:
        return Qr_f64[b, t]
    return Qr_f64[b].mean(axis=0)


@functools.lru_cache(maxsize=64)
def pooled_plants(w: Workload, layer: int = 0) -> Dict[int, np.ndarray]:
    """Planted pooled router-key rows: global chunk index -> bf16 bits [H, D]."""
    if w.pooled != "direct" or w.plant not in ("token", "mean"):
        return {}
    Qr = _as_f64(queries(w, layer)["Qr"])
    rows = {}
    E = w.row_elems
    for i, (b, d, c, t) in enumerate(needles(w, layer)):
        noise = _as_f64(normal_bf16(w.seed, sm.TID_NOISE, layer, i * E, E)).reshape(w.H, w.D)
        g = int(w.doc_chunk_off[d]) + c
        rows[g] = sm.f64_to_bf16_bits(_plant_target(w, Qr, b, t) + 0.1 * noise)
    return rows


def krbar_block(w: Workload, layer: int, g0: int, g1: int) -> np.ndarray:
    """Pooled router keys drawn directly, chunks [g0, g1), plants applied: [g1-g0, H, D] bf16 bits."""
    E = w.row_elems
    x = normal_bf16(w.seed, sm.TID_KRBAR, layer, g0 * E, (g1 - g0) * E).reshape(g1 - g0, w.H, w.D)
    for g, row in pooled_plants(w, layer).items():
        if g0 <= g < g1:
            x[g - g0] = row
    return x


def content_block(w: Workload, which: str, g0: int, g1: int) -> np.ndarray:
    """Pooled content keys ('K') or values ('V') drawn directly, chunks [g0, g1).

    One content store serves every layer (the 18-layer workload aliases it)."""
    tid = sm.TID_KBAR if which == "K" else sm.TID_VBAR
    E = w.row_elems
    return normal_bf16(w.seed, tid, 0, g0 * E, (g1 - g0) * E).reshape(g1 - g0, w.H, w.D)


# ------------------------------------------------------------- chain plants
@functools.lru_cache(maxsize=16)
def chains(w: Workload) -> Tuple[Dict[str, int], ...]:
    """Per query b: docs A, B, C and chunk indices (global) a1, a2, b1, b2, c1 and token tA."""
    if w.plant != "chain":
        return ()
    u = _picks(w, 0, 4096)
    j = 0
    used = set()

    def draw(n):
        nonlocal j
        v = int((u[j] >> np.uint64(32)) * np.uint64(n) >> np.uint64(32)); j += 1
        return v

    out = []
    for b in range(w.B):
        docs = []
        for need in (2, 2, 1):
            while True:
                d = draw(w.n_docs)
                if d not in used and int(w.doc_n_chunks[d]) >= need:
                    break
            used.add(d)
            docs.append(d)
        A, Bd, C = docs
        offA, offB, offC = (int(w.doc_chunk_off[x]) for x in docs)
        nA, nB, nC = (int(w.doc_n_chunks[x]) for x in docs)
        a1 = draw(nA)
        a2 = (a1 + 1 + draw(nA - 1)) % nA
        b1 = draw(nB)
        b2 = (b1 + 1 + draw(nB - 1)) % nB
        c1 = draw(nC)
        tA = draw(w.T)
        out.append(dict(A=A, B=Bd, C=C, a1=offA + a1, a2=offA + a2, b1=offB + b1,
                        b2=offB + b2, c1=offC + c1, tA=tA))
    return tuple(out)


@functools.lru_cache(maxsize=16)
def raw_plants(w: Workload) -> Dict[int, np.ndarray]:
    """Planted raw router-key tokens: global token index -> bf16 bits [H, D]."""
    E = w.row_elems
    if w.pooled != "raw":
        return {}
    rows: Dict[int, np.ndarray] = {}
    if w.plant == "mean_raw":
        Qr = _as_f64(queries(w, 0)["Qr"])
        for (b, d, _c, _t) in needles(w, 0):
            target = Qr[b].mean(axis=0)
            t0, t1 = int(w.doc_tok_off[d]), int(w.doc_tok_off[d + 1])
            noise = _as_f64(normal_bf16(w.seed, sm.TID_NOISE, 0, 0, (t1 - t0) * E)).reshape(-1, w.H, w.D)
            for i in range(t1 - t0):
                rows[t0 + i] = sm.f64_to_bf16_bits(target + 0.1 * noise[i])
    elif w.plant == "chain":
        Qr = _as_f64(queries(w, 0)["Qr"])
        p = 0
        for b, ch in enumerate(chains(w)):
            uvec = _as_f64(normal_bf16(w.seed, sm.TID_CHAIN, 0, (2 * b) * E, E)).reshape(w.H, w.D)
            wvec = _as_f64(normal_bf16(w.seed, sm.TID_CHAIN, 0, (2 * b + 1) * E, E)).reshape(w.H, w.D)
            for g, target in ((ch["a1"], Qr[b, ch["tA"]]), (ch["a2"], uvec), (ch["b1"], uvec),
                              (ch["b2"], wvec), (ch["c1"], wvec)):
                d = int(w.doc_of_chunk(g))
                j = g - int(w.doc_chunk_off[d])
                t0 = int(w.doc_tok_off[d]) + j * w.chunk
                t1 = min(t0 + w.chunk, int(w.doc_tok_off[d + 1]))
                noise = _as_f64(normal_bf16(w.seed, sm.TID_NOISE, 0, p * w.chunk * E,
                                            (t1 - t0) * E)).reshape(-1, w.H, w.D)
                for i in range(t1 - t0):
                    rows[t0 + i] = sm.f64_to_bf16_bits(target + 0.1 * noise[i])
                p += 1
    return rows


def raw_block(w: Workload, which: str, t0: int, t1: int) -> np.ndarray:
    """Raw 'K', 'V' or 'Kr' for tokens [t0, t1): [t1-t0, H, D] bf16 bits (plants applied to Kr)."""
    tid = {"K": sm.TID_K, "V": sm.TID_V, "Kr": sm.TID_KR}[which]
    E = w.row_elems
    x = normal_bf16(w.seed, tid, 0, t0 * E, (t1 - t0) * E).reshape(t1 - t0, w.H, w.D)
    if which == "Kr":
        for t, row in raw_plants(w).items():
            if t0 <= t < t1:
                x[t - t0] = row
    return x


def planted_docs(w: Workload, layer: int = 0) -> List[Tuple[int, int]]:
    """(query b, doc) pairs that must be retrieved (needles; chain heads)."""
    if w.plant == "chain":
        return [(b, ch["A"]) for b, ch in enumerate(chains(w))]
    return [(b, d) for (b, d, _c, _t) in needles(w, layer)]
