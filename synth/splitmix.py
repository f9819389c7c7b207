"""Seeded synthetic-input generator (no part of the method's arithmetic).

Every input tensor element is a pure function of (seed, tensor id, layer,
linear index), so any slice of any tensor can be regenerated alone, on the
host here or on the device by ``synth/csrc/fill.hip``, with identical bits:

    s0    = mix64((seed << 32) ^ (tensor_id << 16) ^ layer)
    u(n)  = mix64(s0 + (n + 1) * GOLDEN)            (mod 2**64)
    value = NORMAL_TABLE[u(n) >> 48]                 (a bf16 bit pattern)

``mix64`` is the SplitMix64 output function published by Steele, Lea and
Flood ("Fast splittable pseudorandom number generators", OOPSLA 2014), and
``u(n)`` is the n-th output of a SplitMix64 stream started at ``s0``.
Only 64-bit integer arithmetic and a table lookup are involved, which is what
makes host and device agree bit for bit.

``NORMAL_TABLE[i]`` is the bf16 rounding (round-to-nearest-even) of the
standard normal quantile at (i + 0.5) / 65536, computed once in float64 with
``statistics.NormalDist``; it approximates N(0, 1) with tails at +-4.32.
"""

from __future__ import annotations

import statistics

import numpy as np

GOLDEN = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

# Tensor ids used by the workloads.  Values are part of the input recipe.
TID_K = 1          # raw keys                    [n_tok, H, D]
TID_V = 2          # raw values                  [n_tok, H, D]
TID_KR = 3         # raw router keys             [n_tok, H, D]
TID_Q = 4          # attention queries           [B, Tq, Hq, D]
TID_QR = 5         # router queries              [B, T, H, D]
TID_KLOC = 6       # local keys                  [B, Tl, Hkv, D]
TID_VLOC = 7       # local values                [B, Tl, Hkv, D]
TID_NOISE = 8      # plant noise
TID_KBAR = 9       # pooled keys drawn directly  [n_chunks, H, D]
TID_VBAR = 10      # pooled values drawn directly
TID_KRBAR = 11     # pooled router keys drawn directly (per layer)
TID_LEN = 12       # document lengths
TID_PICK = 13      # needle / chain placement choices
TID_CHAIN = 14     # chain link vectors (u, w)
TID_HIDDEN = 15    # hidden states of the corpus  [n_tok, d_model]
TID_WKR = 16       # router-key projection        [H * D, d_model]


def mix64_int(z: int) -> int:
    """SplitMix64 output function on a Python int (reference for tests)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * M1) & MASK64
    z = ((z ^ (z >> 27)) * M2) & MASK64
    return z ^ (z >> 31)


def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    z ^= z >> np.uint64(30)
    z *= np.uint64(M1)
    z ^= z >> np.uint64(27)
    z *= np.uint64(M2)
    z ^= z >> np.uint64(31)
    return z


def stream_start(seed: int, tensor_id: int, layer: int = 0) -> int:
    if not (0 <= seed < (1 << 32) and 0 <= tensor_id < (1 << 16) and 0 <= layer < (1 << 16)):
        raise ValueError("seed < 2**32, tensor_id < 2**16, layer < 2**16 required")
    return mix64_int((seed << 32) ^ (tensor_id << 16) ^ layer)


def raw_u64(seed: int, tensor_id: int, layer: int, start: int, count: int) -> np.ndarray:
    """u(n) for n in [start, start + count) as uint64."""
    s0 = np.uint64(stream_start(seed, tensor_id, layer))
    n = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = s0 + n * np.uint64(GOLDEN)
        return _mix64_np(z)


def _f64_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits, round to nearest even, via round-to-odd float32.

    Rounding float64 to float32 with round-to-odd and then float32 to bf16
    with round-to-nearest-even gives the correctly rounded bf16 (float32 keeps
    more than two extra bits), which plain double rounding would not.
    """
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    back = f.astype(np.float64)
    inexact = back != x
    # move f toward zero when rounding went away from zero, then set sticky bit
    away = inexact & (np.abs(back) > np.abs(x))
    f = np.where(away, np.nextafter(f, np.float32(0)), f)
    bits = f.view(np.uint32).copy()
    bits = np.where(inexact, bits | np.uint32(1), bits)
    # float32 -> bf16 round-to-nearest-even (finite inputs)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits.astype(np.uint64) + np.uint64(0x7FFF) + lsb.astype(np.uint64)) >> np.uint64(16)
    return rounded.astype(np.uint16)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bf16 (nearest even); returns uint16 bit patterns."""
    return _f64_to_bf16_rne(x)


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _build_table() -> np.ndarray:
    nd = statistics.NormalDist()
    q = np.array([nd.inv_cdf((i + 0.5) / 65536.0) for i in range(65536)], dtype=np.float64)
    return f64_to_bf16_bits(q)


NORMAL_TABLE: np.ndarray = _build_table()          # uint16[65536] bf16 bits
NORMAL_TABLE.setflags(write=False)


def normal_bf16(seed: int, tensor_id: int, layer: int, start: int, count: int) -> np.ndarray:
    """bf16 bit patterns of N(0,1) draws for linear indices [start, start+count)."""
    u = raw_u64(seed, tensor_id, layer, start, count)
    return NORMAL_TABLE[(u >> np.uint64(48)).astype(np.int64)]


def normal_f64(seed: int, tensor_id: int, layer: int, start: int, count: int) -> np.ndarray:
    return bf16_bits_to_f32(normal_bf16(seed, tensor_id, layer, start, count)).astype(np.float64)


def uniform_int(seed: int, tensor_id: int, layer: int, start: int, count: int,
                lo: int, hi: int) -> np.ndarray:
    """Integers in [lo, hi] (inclusive) from the top 32 bits: lo + (u>>32)*(hi-lo+1) >> 32."""
    u = raw_u64(seed, tensor_id, layer, start, count) >> np.uint64(32)
    span = np.uint64(hi - lo + 1)
    return (lo + ((u * span) >> np.uint64(32)).astype(np.int64)).astype(np.int64)
