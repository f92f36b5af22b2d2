"""CPU oracle of the n-gram pool that feeds the greedy (Lookahead) verify: plain Python.

TEST INFRASTRUCTURE. Only the tests, the package's smoke check and the bench's
CPU-baseline leg may import or run this module. The HIP library never does.

Source (page title, section):
  [LA]  Lookahead Decoding 完全拆解:Jacobi 迭代与 N-gram 池 ...:
        "Lookahead 分支": every step the 2D window produces W new n-grams of
        length N, collected into a pool; "N-gram 池与身份判定": the pool caches
        the n-grams gathered along the trajectory, and only those whose first
        token equals the last generated token go to verification;
        "验证分支": n-grams that are not adopted stay in the pool.

Readings where the page is silent (each is listed with its reason in the design
notes of the repository):
  * one pool per sequence (batch row), keyed by the n-gram's first token; a key
    holds at most G continuations (the N-1 tokens after the first), G being the
    number of candidates the verify takes;
  * a key keeps its G most recently inserted distinct continuations, newest
    first; inserting a continuation the key already holds makes it the newest
    (it is not stored twice); when a key is full the oldest one is dropped;
  * the W n-grams of one insert call enter in window order (index 0 first);
  * an n-gram with any token outside [0, V) is skipped (not inserted) and counted;
  * a lookup returns the key's continuations newest first; a token outside
    [0, V) has none.

The hashed pool (NgramCache) is the same pool held in a bounded table, the GPU hash
map the verify's candidate source asks for; the page is silent on its capacity, so
these are readings too:
  * a sequence's table has `sets` sets of `ways` entries (sets a power of two); a
    key lives in set h(key) = floor((key * 2654435769 mod 2^32) / 2^(32 - log2 sets))
    (Knuth's multiplicative hashing, the constant floor(2^32 / golden ratio));
  * every inserted (not skipped) n-gram gets the next value of the sequence's
    insertion clock; a key's stamp is the clock value of its newest n-gram;
  * a new key in a set that holds `ways` keys evicts the key with the oldest stamp,
    continuations and all; a key that comes back starts empty;
  * within a key, everything is as in the direct pool above. While no set
    overflows, the hashed pool holds exactly what the direct pool holds.
"""
from __future__ import annotations

import numpy as np


class NgramPool:
    """The pool of one sequence: key -> continuations, newest first."""

    def __init__(self, V: int, G: int, N: int):
        self.V, self.G, self.N = int(V), int(G), int(N)
        self.buckets: dict[int, list[tuple[int, ...]]] = {}

    def insert(self, ngram) -> bool:
        """Insert one n-gram of N tokens; False when it is skipped (a token out of range)."""
        toks = [int(t) for t in ngram]
        assert len(toks) == self.N
        if any(t < 0 or t >= self.V for t in toks):
            return False
        key, cont = toks[0], tuple(toks[1:])
        held = self.buckets.setdefault(key, [])
        if cont in held:
            held.remove(cont)
        held.insert(0, cont)
        del held[self.G:]
        return True

    def lookup(self, token: int) -> list[tuple[int, ...]]:
        """The continuations of `token`, newest first (at most G)."""
        token = int(token)
        if token < 0 or token >= self.V:
            return []
        return list(self.buckets.get(token, []))


def new_pools(B: int, V: int, G: int, N: int) -> list[NgramPool]:
    return [NgramPool(V, G, N) for _ in range(B)]


def pool_insert(pools: list[NgramPool], ngrams: np.ndarray) -> np.ndarray:
    """Insert ngrams [B, W, N] (sequence b into pools[b], index 0 first). Returns skipped counts [B]."""
    ngrams = np.asarray(ngrams)
    B, W, _ = ngrams.shape
    skipped = np.zeros(B, dtype=np.int32)
    for b in range(B):
        for w in range(W):
            if not pools[b].insert(ngrams[b, w]):
                skipped[b] += 1
    return skipped


def pool_lookup(pools: list[NgramPool], last_tokens: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Candidates [B, G, N-1] (newest first, -1 past the count) and counts [B] for each sequence's last token."""
    B = len(pools)
    G, N = pools[0].G, pools[0].N
    cand = np.full((B, G, N - 1), -1, dtype=np.int32)
    count = np.zeros(B, dtype=np.int32)
    for b in range(B):
        found = pools[b].lookup(int(last_tokens[b]))
        count[b] = len(found)
        for g, cont in enumerate(found):
            cand[b, g] = cont
    return cand, count


def pool_contents(pools: list[NgramPool]) -> dict[tuple[int, int], list[tuple[int, ...]]]:
    """Every non-empty (sequence, key) bucket, for comparisons."""
    return {(b, k): list(v) for b, p in enumerate(pools) for k, v in p.buckets.items() if v}


# ---------------------------------------------------------------- the hashed pool

GOLDEN32 = 2654435769  # floor(2^32 / golden ratio), Knuth's multiplicative hashing constant


def cache_set(key: int, sets: int) -> int:
    """The home set of `key` among `sets` (a power of two) sets."""
    bits = sets.bit_length() - 1
    if bits == 0:
        return 0
    return ((int(key) * GOLDEN32) % (1 << 32)) >> (32 - bits)


class NgramCache:
    """The hashed pool of one sequence: `sets` sets of at most `ways` keys, each key with
    its stamp and its continuations (newest first, at most G)."""

    def __init__(self, V: int, G: int, N: int, sets: int, ways: int):
        assert sets >= 1 and sets & (sets - 1) == 0 and ways >= 1
        self.V, self.G, self.N, self.sets, self.ways = int(V), int(G), int(N), int(sets), int(ways)
        self.clock = 0
        self.table: list[dict[int, list]] = [dict() for _ in range(sets)]  # set -> key -> [stamp, conts]

    def insert(self, ngram) -> bool:
        """Insert one n-gram of N tokens; False when it is skipped (a token out of range)."""
        toks = [int(t) for t in ngram]
        assert len(toks) == self.N
        if any(t < 0 or t >= self.V for t in toks):
            return False
        key, cont = toks[0], tuple(toks[1:])
        stamp = self.clock
        self.clock += 1
        entries = self.table[cache_set(key, self.sets)]
        if key not in entries:
            if len(entries) == self.ways:
                oldest = min(entries, key=lambda k: entries[k][0])
                del entries[oldest]
            entries[key] = [stamp, []]
        ent = entries[key]
        ent[0] = stamp
        held = ent[1]
        if cont in held:
            held.remove(cont)
        held.insert(0, cont)
        del held[self.G:]
        return True

    def lookup(self, token: int) -> list[tuple[int, ...]]:
        """The continuations of `token`, newest first (at most G)."""
        token = int(token)
        if token < 0 or token >= self.V:
            return []
        ent = self.table[cache_set(token, self.sets)].get(token)
        return list(ent[1]) if ent else []

    def contents(self) -> dict[int, tuple[int, list[tuple[int, ...]]]]:
        """key -> (stamp, continuations) over every set."""
        return {k: (e[0], list(e[1])) for tab in self.table for k, e in tab.items()}


def new_caches(B: int, V: int, G: int, N: int, sets: int, ways: int) -> list[NgramCache]:
    return [NgramCache(V, G, N, sets, ways) for _ in range(B)]
