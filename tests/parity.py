"""Comparison rules shared by the GPU parity tests (not a test module).

P2  document / chunk scores: |gpu - oracle| <= 1e-5.
P3  top-k: the GPU set S is accepted iff every d in S has oracle score
    >= s_k - 1e-3 and every d outside S has oracle score <= s_k + 1e-3, where
    s_k is the oracle's k-th score; where the oracle's gap at rank k is >= 1e-3
    this is exact equality of the id sets.  Order inside S is compared where
    adjacent oracle gaps are >= 1e-3.
P4  attention: per output row ||o - o*|| / ||o*|| <= 2e-2 (bf16 inputs, fp32
    accumulation); the oracle attends over the GPU's selected set.
P1  pooled V/Kr within 1 bf16 ulp of the oracle's rounded mean, K within 2.
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import msa_oracle as O

SCORE_TOL = 1e-5
GAP = 1e-3
ATT_TOL = 2e-2


def dev_bits(a, device="cuda:0") -> torch.Tensor:
    """bf16 bit array (uint16) -> device int16 tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def check_topk(gpu_idx: np.ndarray, oracle_scores: np.ndarray, k: int, gap: float = GAP):
    """P3 for one query.  Returns the number of ids that differ from the oracle's top-k."""
    s = np.asarray(oracle_scores, dtype=np.float64)
    ref_idx, ref_sc = O.topk(s[None], k)
    sk = ref_sc[0, -1]
    S = set(int(x) for x in gpu_idx)
    assert len(S) == k, f"duplicate ids in {gpu_idx}"
    inside = np.array(sorted(S))
    outside = np.setdiff1d(np.arange(len(s)), inside)
    assert np.all(s[inside] >= sk - gap), "selected a document clearly below rank k"
    if len(outside):
        assert np.all(s[outside] <= sk + gap), "missed a document clearly above rank k"
    # order: compare ranks where the oracle's adjacent gaps are clear
    ordered = [int(x) for x in gpu_idx]
    for r in range(k - 1):
        a, b = ordered[r], ordered[r + 1]
        if abs(s[a] - s[b]) >= gap:
            assert s[a] > s[b], f"rank {r} out of order"
    return len(S ^ set(int(x) for x in ref_idx[0]))


def rel_rows(o: np.ndarray, ref: np.ndarray) -> float:
    o = o.astype(np.float64).reshape(-1, o.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    return float((np.linalg.norm(o - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)).max())


def bf16_ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 ulps between two bf16 bit arrays (sign-magnitude ordered)."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + (x & 0x7FFF))
    return np.abs(ordered(a_bits) - ordered(b_bits))
