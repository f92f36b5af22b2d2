"""Philox4x32-10 counter-based generator, NumPy, and the verify uniforms built on it.

The generator is the one published by Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): a 128-bit counter and a
64-bit key go through ten rounds of two 32x32->64 multiplications, with the key
bumped by two Weyl constants between rounds. It holds no state, so the uniforms
of any (row, position, round) can be produced independently on host or device.

The verify step draws a fresh uniform for each accept test and a separate one
for each resample / bonus draw (Speculative Decoding -- LLM推理优化技术（一）,
§4 code: a fresh rand per test and a separate multinomial draw; kwkr.cn notes
§3.1: r is a fresh uniform per position). Layout of the uniforms tensor
[B, K+1, 2]:
    [b, i, 0]  accept uniform r_i  (used for i < K)
    [b, i, 1]  sample uniform u_i  (resample at i < K, bonus draw at i = K)
Counter for (b, i) of round `rnd`: (i, b, rnd & 0xffffffff, rnd >> 32); key =
(seed & 0xffffffff, seed >> 32). Output word 0 -> r, word 1 -> u, each mapped as
(w >> 8) * 2^-24, so every value is a multiple of 2^-24 in [0, 1 - 2^-24] and is
exact in float32 and float64 alike.
"""
from __future__ import annotations

import numpy as np

PHILOX_M0 = np.uint64(0xD2511F53)
PHILOX_M1 = np.uint64(0xCD9E8D57)
PHILOX_W0 = np.uint32(0x9E3779B9)
PHILOX_W1 = np.uint32(0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)


def _mulhilo(m: np.uint64, a: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    prod = a.astype(np.uint64) * m
    return (prod >> np.uint64(32)).astype(np.uint32), (prod & _MASK32).astype(np.uint32)


def philox4x32_10(ctr: np.ndarray, key: np.ndarray) -> np.ndarray:
    """Apply Philox4x32-10 to counters `ctr` [..., 4] (uint32) with keys `key` [..., 2].

    Returns the four output words [..., 4] as uint32.
    """
    ctr = np.asarray(ctr, dtype=np.uint32)
    key = np.asarray(key, dtype=np.uint32)
    c0, c1, c2, c3 = (ctr[..., j].copy() for j in range(4))
    k0 = np.broadcast_to(key[..., 0], c0.shape).copy()
    k1 = np.broadcast_to(key[..., 1], c0.shape).copy()
    with np.errstate(over="ignore"):
        for rnd in range(10):
            if rnd:
                k0 = (k0 + PHILOX_W0).astype(np.uint32)
                k1 = (k1 + PHILOX_W1).astype(np.uint32)
            hi0, lo0 = _mulhilo(PHILOX_M0, c0)
            hi1, lo1 = _mulhilo(PHILOX_M1, c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1)


def words_to_unit(w: np.ndarray) -> np.ndarray:
    """Map 32-bit words to [0, 1 - 2^-24] on a 2^-24 grid (exact in float32)."""
    return (np.asarray(w, dtype=np.uint32) >> np.uint32(8)).astype(np.float64) * (2.0 ** -24)


def verify_uniforms(seed: int, rnd: int, B: int, K: int) -> np.ndarray:
    """Uniforms [B, K+1, 2] float32 for one verify round (layout in the module doc)."""
    if B < 0 or K < 0:
        raise ValueError("B and K must be non-negative")
    i = np.arange(K + 1, dtype=np.uint32)[None, :]
    b = np.arange(B, dtype=np.uint32)[:, None]
    ctr = np.zeros((B, K + 1, 4), dtype=np.uint32)
    ctr[..., 0] = i
    ctr[..., 1] = b
    ctr[..., 2] = np.uint32(rnd & 0xFFFFFFFF)
    ctr[..., 3] = np.uint32((rnd >> 32) & 0xFFFFFFFF)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint32)
    out = philox4x32_10(ctr, key)
    u = np.empty((B, K + 1, 2), dtype=np.float32)
    u[..., 0] = words_to_unit(out[..., 0])
    u[..., 1] = words_to_unit(out[..., 1])
    return u


def ngram_uniforms(seed: int, rnd: int, B: int, N: int, G: int) -> np.ndarray:
    """Uniforms [B, N, G+1] float32 for the sampling verify of n-gram candidates.

    Philox4x32-10 (same key as verify_uniforms) with counter (i | j << 16, b,
    round lo32, round hi32 | 1 << 31), j = h // 4, word h % 4 -> [b, i, h]: a
    stream of its own, disjoint from verify_uniforms' counters.
    """
    if B < 0 or N < 1 or G < 1:
        raise ValueError("bad sizes")
    H = G + 1
    nj = (H + 3) // 4
    i = np.arange(N, dtype=np.uint32)[None, :, None]
    j = np.arange(nj, dtype=np.uint32)[None, None, :]
    b = np.arange(B, dtype=np.uint32)[:, None, None]
    ctr = np.zeros((B, N, nj, 4), dtype=np.uint32)
    ctr[..., 0] = i | (j << np.uint32(16))
    ctr[..., 1] = b
    ctr[..., 2] = np.uint32(rnd & 0xFFFFFFFF)
    ctr[..., 3] = np.uint32(((rnd >> 32) & 0x7FFFFFFF) | 0x80000000)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint32)
    out = philox4x32_10(ctr, key).reshape(B, N, nj * 4)[:, :, :H]
    return words_to_unit(out).astype(np.float32)
