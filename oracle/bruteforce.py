"""Brute-force checker for tiny inputs: explicit Python loops over scalars.

TEST INFRASTRUCTURE ONLY (see ``oracle/msa_oracle.py``).  Every quantity is
recomputed element by element with the ``math`` module, with no numpy
vectorisation and no shared helper, so that a mistake in the vectorised
oracle (a transposed operand, a wrong axis, a dropped term) shows up as a
mismatch.  Same readings as the oracle; same page citations.
"""

from __future__ import annotations

import math
from typing import List, Sequence


def rope_vec(x: Sequence[float], pos: int, base: float) -> List[float]:
    D = len(x)
    half = D // 2
    out = [0.0] * D
    for i in range(half):
        th = pos * base ** (-2.0 * i / D)
        c, s = math.cos(th), math.sin(th)
        out[i] = x[i] * c - x[i + half] * s
        out[i + half] = x[i + half] * c + x[i] * s
    return out


def pool(K, V, Kr, doc_len, chunk, base):
    """Returns lists Kb, Vb, Rb of [H][D] nested lists, one per chunk."""
    H, D = len(K[0]), len(K[0][0])
    Kb, Vb, Rb = [], [], []
    t0 = 0
    for Ld in doc_len:
        n = (Ld + chunk - 1) // chunk
        for j in range(n):
            a, b = j * chunk, min((j + 1) * chunk, Ld)
            cnt = b - a
            kk = [[0.0] * D for _ in range(H)]
            vv = [[0.0] * D for _ in range(H)]
            rr = [[0.0] * D for _ in range(H)]
            for t in range(a, b):
                for h in range(H):
                    kr = rope_vec(K[t0 + t][h], t, base)
                    for d in range(D):
                        kk[h][d] += kr[d] / cnt
                        vv[h][d] += V[t0 + t][h][d] / cnt
                        rr[h][d] += Kr[t0 + t][h][d] / cnt
            Kb.append(kk); Vb.append(vv); Rb.append(rr)
        t0 += Ld
    return Kb, Vb, Rb


def encode_router_keys(hidden, W, doc_len, chunk, H, D):
    """hidden: [n_tok][d_model]; W: [H*D][d_model].  Returns [n_chunks][H][D]:
    per token, out feature f = sum_i hidden[t][i] * W[f][i]; then chunk means."""
    dm = len(hidden[0])
    out = []
    t0 = 0
    for Ld in doc_len:
        n = (Ld + chunk - 1) // chunk
        for j in range(n):
            a, b = j * chunk, min((j + 1) * chunk, Ld)
            acc = [[0.0] * D for _ in range(H)]
            for t in range(a, b):
                for h in range(H):
                    for d in range(D):
                        f = h * D + d
                        s = 0.0
                        for i in range(dm):
                            s += hidden[t0 + t][i] * W[f][i]
                        acc[h][d] += s / (b - a)
            out.append(acc)
        t0 += Ld
    return out


def cosine(a, b) -> float:
    na = math.sqrt(sum(x * x for x in a))
    nb = math.sqrt(sum(x * x for x in b))
    if na == 0.0 or nb == 0.0:
        return 0.0
    return sum(x * y for x, y in zip(a, b)) / (na * nb)


def route(Qr, Krbar, doc_len_chunks, exclude=None):
    """Qr: [B][T][H][D]; Krbar: [G][H][D]; doc_len_chunks: chunks per document."""
    B, T, H = len(Qr), len(Qr[0]), len(Qr[0][0])
    G = len(Krbar)
    chunk = [[-math.inf] * G for _ in range(B)]
    for b in range(B):
        for g in range(G):
            for t in range(T):
                s = 0.0
                for h in range(H):
                    s += cosine(Qr[b][t][h], Krbar[g][h])
                s /= H
                if s > chunk[b][g]:
                    chunk[b][g] = s
    doc = []
    for b in range(B):
        row, g0 = [], 0
        for d, n in enumerate(doc_len_chunks):
            best = -math.inf
            for g in range(g0, g0 + n):
                best = max(best, chunk[b][g])
            if exclude is not None and exclude[b][d]:
                best = -math.inf
            row.append(best)
            g0 += n
        doc.append(row)
    return chunk, doc


def topk(doc_scores_row, k):
    """Selection by repeated scan: take the best remaining (highest score, then lowest id)."""
    taken = []
    for _ in range(k):
        best = None
        for d, s in enumerate(doc_scores_row):
            if d in taken:
                continue
            if best is None or s > doc_scores_row[best]:
                best = d
        taken.append(best)
    return taken


def attend(Q, Kloc, Vloc, Kmem, Vmem, offset, base, scale):
    """Q: [Tq][Hq][D]; Kloc/Vloc: [Tl][Hkv][D]; Kmem/Vmem: [M][Hkv][D]."""
    Tq, Hq, D = len(Q), len(Q[0]), len(Q[0][0])
    Tl, Hkv = len(Kloc), len(Kloc[0])
    M = len(Kmem)
    group = Hq // Hkv
    O = [[[0.0] * D for _ in range(Hq)] for _ in range(Tq)]
    for i in range(Tq):
        qpos = offset + (Tl - Tq) + i
        for h in range(Hq):
            g = h // group
            q = rope_vec(Q[i][h], qpos, base)
            logits, vals = [], []
            for m in range(M):
                logits.append(scale * sum(q[d] * Kmem[m][g][d] for d in range(D)))
                vals.append(Vmem[m][g])
            for j in range(Tl):
                if j > (Tl - Tq) + i:
                    continue
                kr = rope_vec(Kloc[j][g], offset + j, base)
                logits.append(scale * sum(q[d] * kr[d] for d in range(D)))
                vals.append(Vloc[j][g])
            mx = max(logits)
            w = [math.exp(z - mx) for z in logits]
            tot = sum(w)
            for d in range(D):
                O[i][h][d] = sum(wj * v[d] for wj, v in zip(w, vals)) / tot
    return O
