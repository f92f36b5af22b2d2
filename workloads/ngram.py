"""Seeded synthetic n-gram streams for the n-gram pool (random tokens only; no step of the pool's logic).

The Lookahead page's window produces W n-grams of length N per step (its
example: W=5, N=4; its experiments W up to 15, N up to 5) and the verify takes
G candidates (GUESS_SET_SIZE 7 in its configuration example). The generator
draws first tokens from a small "hot" set with probability `hot`, so keys
repeat and buckets fill, evict and refresh; the other tokens are uniform on
[0, V). A fraction `bad` of the n-grams get one token outside [0, V).
"""
from __future__ import annotations

import numpy as np


def ngram_steps(seed: int, steps: int, B: int, W: int, N: int, V: int, *, hot: float = 0.5, n_hot: int = 8,
                repeat: float = 0.3, bad: float = 0.0) -> list[np.ndarray]:
    """`steps` arrays of int32 n-grams [B, W, N]. `repeat`: chance an n-gram copies an earlier one of the stream."""
    rng = np.random.default_rng([seed, 4242])
    hot_keys = rng.integers(0, V, size=(B, n_hot))
    out, history = [], [[] for _ in range(B)]
    for _ in range(steps):
        g = rng.integers(0, V, size=(B, W, N)).astype(np.int64)
        for b in range(B):
            for w in range(W):
                if history[b] and rng.random() < repeat:
                    g[b, w] = history[b][rng.integers(0, len(history[b]))]
                elif rng.random() < hot:
                    g[b, w, 0] = hot_keys[b, rng.integers(0, n_hot)]
                    if rng.random() < 0.5:  # a few continuations per hot key
                        g[b, w, 1:] = (g[b, w, 0] + np.arange(1, N) * (1 + rng.integers(0, 3))) % V
                if rng.random() < bad:
                    g[b, w, rng.integers(0, N)] = rng.choice([-1, V, -7, V + 3])
                history[b].append(g[b, w].copy())
        out.append(g.astype(np.int32))
    return out


def lookup_tokens(seed: int, B: int, V: int, steps: list[np.ndarray]) -> np.ndarray:
    """Last tokens to look up [B]: mostly keys that were inserted, some fresh ones and some outside [0, V)."""
    rng = np.random.default_rng([seed, 4343])
    last = rng.integers(0, V, size=B)
    for b in range(B):
        u = rng.random()
        if u < 0.7 and steps and steps[0].shape[1] > 0:
            s = steps[rng.integers(0, len(steps))]
            last[b] = s[b, rng.integers(0, s.shape[1]), 0]
        elif u < 0.8:
            last[b] = rng.choice([-1, V])
    return last.astype(np.int32)
