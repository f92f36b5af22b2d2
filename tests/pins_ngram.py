"""Checks that pin the n-gram pool oracle (each takes the oracle module, like tests/pins.py).

Pinned facts:
  * hand-worked sequences in tests/golden/ngram_worked.json (derivations beside them);
  * a second, non-incremental statement of the same reading: from the whole
    insert history, a key's bucket is its distinct continuations ordered by
    their last insertion, newest first, cut to G;
  * invariants: at most G per key, no duplicates, every stored continuation was
    inserted under its key, insertion order within a call is the window order.
"""
from __future__ import annotations

import numpy as np

from golden_io import load
from workloads.ngram import lookup_tokens, ngram_steps


def check_golden_ngram(orc) -> None:
    for case in load("ngram_worked.json")["cases"]:
        V, G, N = case["V"], case["G"], case["N"]
        B = len(case["steps"][0]["ngrams"])
        pools = orc.new_pools(B, V, G, N)
        for st in case["steps"]:
            skipped = orc.pool_insert(pools, np.array(st["ngrams"]))
            assert skipped.tolist() == st["expect_skipped"], (case["name"], skipped, st["expect_skipped"])
        for lk in case["lookups"]:
            cand, count = orc.pool_lookup(pools, np.array(lk["last"]))
            assert count.tolist() == lk["expect_count"], (case["name"], lk["last"], count)
            assert cand.tolist() == lk["expect_cand"], (case["name"], lk["last"], cand.tolist())


def _replay(history, V, G):
    """Buckets from the whole history at once: key -> continuations by last insertion, newest first."""
    last_seen = {}
    for t, ng in enumerate(history):
        toks = [int(x) for x in ng]
        if any(x < 0 or x >= V for x in toks):
            continue
        last_seen[(toks[0], tuple(toks[1:]))] = t
    buckets = {}
    for (key, cont), t in last_seen.items():
        buckets.setdefault(key, []).append((t, cont))
    return {k: [c for _, c in sorted(v, reverse=True)][:G] for k, v in buckets.items()}


def check_ngram_history_replay(orc) -> None:
    for seed, (B, W, N, V, G) in enumerate([(3, 5, 4, 12, 3), (2, 15, 5, 40, 7), (4, 7, 2, 6, 1), (2, 9, 3, 20, 64)]):
        steps = ngram_steps(seed, 6, B, W, N, V, hot=0.6, n_hot=4, repeat=0.4, bad=0.1)
        pools = orc.new_pools(B, V, G, N)
        for st in steps:
            orc.pool_insert(pools, st)
        for b in range(B):
            history = [st[b, w] for st in steps for w in range(W)]
            want = _replay(history, V, G)
            got = {k: v for k, v in pools[b].buckets.items() if v}
            assert got == want, (seed, b)


def check_ngram_invariants(orc) -> None:
    B, W, N, V, G = 3, 11, 4, 15, 3
    steps = ngram_steps(7, 8, B, W, N, V, hot=0.7, n_hot=3, repeat=0.5, bad=0.15)
    pools = orc.new_pools(B, V, G, N)
    inserted = [set() for _ in range(B)]
    for st in steps:
        skipped = orc.pool_insert(pools, st)
        bad = ((st < 0) | (st >= V)).any(axis=2).sum(axis=1)
        assert skipped.tolist() == bad.tolist()
        for b in range(B):
            for w in range(W):
                if not ((st[b, w] < 0) | (st[b, w] >= V)).any():
                    inserted[b].add((int(st[b, w, 0]), tuple(int(x) for x in st[b, w, 1:])))
        # the newest n-gram of each key in this call heads its bucket
        for b in range(B):
            newest = {}
            for w in range(W):
                if not ((st[b, w] < 0) | (st[b, w] >= V)).any():
                    newest[int(st[b, w, 0])] = tuple(int(x) for x in st[b, w, 1:])
            for k, cont in newest.items():
                assert pools[b].lookup(k)[0] == cont
    for b in range(B):
        for k, v in pools[b].buckets.items():
            assert len(v) <= G and len(set(v)) == len(v)
            assert all((k, c) in inserted[b] for c in v)
    cand, count = orc.pool_lookup(pools, lookup_tokens(3, B, V, steps))
    assert cand.shape == (B, G, N - 1) and np.all((count >= 0) & (count <= G))
    for b in range(B):
        assert np.all(cand[b, count[b]:] == -1) and np.all(cand[b, :count[b]] >= 0)


# ---------------------------------------------------------------- the hashed pool

def _cache_contents_list(cache) -> list:
    """[[key, stamp, [continuation, ...]], ...] sorted by key, as the fixtures write it."""
    return sorted([k, st, [list(c) for c in conts]] for k, (st, conts) in cache.contents().items())


def check_golden_cache(orc) -> None:
    for case in load("ngram_cache_worked.json")["cases"]:
        V, G, N, sets, ways = case["V"], case["G"], case["N"], case["sets"], case["ways"]
        B = len(case["steps"][0]["ngrams"])
        caches = orc.new_caches(B, V, G, N, sets, ways)
        for st in case["steps"]:
            skipped = orc.pool_insert(caches, np.array(st["ngrams"]))
            assert skipped.tolist() == st["expect_skipped"], (case["name"], skipped, st["expect_skipped"])
            for b in range(B):
                assert _cache_contents_list(caches[b]) == st["expect_contents"][b], (case["name"], b)
        for lk in case["lookups"]:
            cand, count = orc.pool_lookup(caches, np.array(lk["last"]))
            assert count.tolist() == lk["expect_count"], (case["name"], lk["last"], count)
            assert cand.tolist() == lk["expect_cand"], (case["name"], lk["last"], cand.tolist())


def _golden_ratio_constant() -> int:
    """floor(2^32 / phi) from the decimal expansion of sqrt(5), with no float in the way."""
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    phi = (1 + Decimal(5).sqrt()) / 2
    return int((Decimal(2) ** 32 / phi).to_integral_value(rounding="ROUND_FLOOR"))


def _home_set(key: int, sets: int) -> int:
    """floor(sets * frac(key * C / 2^32)) with C = floor(2^32 / phi): the top log2(sets) bits of key * C mod 2^32."""
    return (int(key) * _golden_ratio_constant() % 2 ** 32) * sets // 2 ** 32


def check_cache_hash(orc) -> None:
    assert orc.GOLDEN32 == _golden_ratio_constant() == 2654435769
    rng = np.random.default_rng(5)
    keys = np.concatenate([np.arange(0, 300), rng.integers(0, 2 ** 31 - 1, 300)])
    for sets in (1, 2, 8, 64, 1024, 1 << 16, 1 << 20):
        for k in keys:
            assert orc.cache_set(int(k), sets) == _home_set(int(k), sets), (int(k), sets)
    # small keys against the golden ratio itself: set = floor(sets * frac(key * 0.6180339887...))
    inv_phi = (5 ** 0.5 - 1) / 2
    for sets in (2, 8, 64, 256):
        for k in range(1000):
            x = (k * inv_phi) % 1.0 * sets
            if abs(x - round(x)) > 1e-4:
                assert orc.cache_set(k, sets) == int(x), (k, sets)


def _replay_cache(history, V, G, sets, ways):
    """The hashed pool from the whole history at once (LRU reading): a set holds the `ways`
    distinct keys of that set inserted most recently; a held key's life began at its latest
    insertion that followed `ways` or more distinct other keys of its set since its previous
    insertion (or at its first); its continuations are those inserted in its life, by last
    insertion, newest first, cut to G; its stamp is its last insertion (clocks count valid n-grams)."""
    valid = []
    for ng in history:
        toks = [int(x) for x in ng]
        if all(0 <= x < V for x in toks):
            valid.append((toks[0], tuple(toks[1:])))
    out = {}
    for s in range(sets):
        ev = [(t, k, c) for t, (k, c) in enumerate(valid) if _home_set(k, sets) == s]
        last = {}
        for t, k, _ in ev:
            last[k] = t
        held = sorted(last, key=lambda k: last[k], reverse=True)[:ways]
        for k in held:
            times = [t for t, kk, _ in ev if kk == k]
            start = times[0]
            for prev, cur in zip(times, times[1:]):
                others = {kk for t, kk, _ in ev if prev < t < cur and kk != k}
                if len(others) >= ways:
                    start = cur
            seen = {}
            for t, kk, c in ev:
                if kk == k and t >= start:
                    seen[c] = t
            conts = [c for c, _ in sorted(seen.items(), key=lambda it: it[1], reverse=True)][:G]
            out[k] = (last[k], conts)
    return out


def check_cache_history_replay(orc) -> None:
    shapes = [(3, 5, 4, 12, 3, 1, 2), (2, 15, 5, 40, 7, 4, 2), (4, 7, 2, 30, 1, 8, 1), (2, 9, 3, 50, 4, 2, 3),
              (2, 12, 3, 25, 2, 1, 5)]
    for seed, (B, W, N, V, G, sets, ways) in enumerate(shapes):
        steps = ngram_steps(seed + 20, 6, B, W, N, V, hot=0.5, n_hot=6, repeat=0.4, bad=0.1)
        caches = orc.new_caches(B, V, G, N, sets, ways)
        for st in steps:
            orc.pool_insert(caches, st)
        for b in range(B):
            history = [st[b, w] for st in steps for w in range(W)]
            assert caches[b].contents() == _replay_cache(history, V, G, sets, ways), (seed, b)


def check_cache_equals_pool_without_overflow(orc) -> None:
    """With room for every key (no set ever overflows) the hashed pool holds what the direct pool holds."""
    for seed, (B, W, N, V, G, sets) in enumerate([(3, 9, 4, 16, 3, 4), (2, 15, 5, 40, 7, 8), (2, 6, 2, 10, 1, 1)]):
        steps = ngram_steps(seed + 40, 5, B, W, N, V, hot=0.6, n_hot=4, repeat=0.4, bad=0.1)
        caches = orc.new_caches(B, V, G, N, sets, V)
        pools = orc.new_pools(B, V, G, N)
        for st in steps:
            assert orc.pool_insert(caches, st).tolist() == orc.pool_insert(pools, st).tolist()
            for b in range(B):
                got = {k: conts for k, (_, conts) in caches[b].contents().items()}
                assert got == {k: v for k, v in pools[b].buckets.items() if v}, (seed, b)
        last = lookup_tokens(seed, B, V, steps)
        c1, n1 = orc.pool_lookup(caches, last)
        c2, n2 = orc.pool_lookup(pools, last)
        assert np.array_equal(c1, c2) and np.array_equal(n1, n2)


def check_cache_invariants(orc) -> None:
    B, W, N, V, G, sets, ways = 3, 13, 3, 60, 3, 4, 2
    steps = ngram_steps(9, 7, B, W, N, V, hot=0.4, n_hot=8, repeat=0.4, bad=0.15)
    caches = orc.new_caches(B, V, G, N, sets, ways)
    n_valid = np.zeros(B, dtype=np.int64)
    for st in steps:
        orc.pool_insert(caches, st)
        n_valid += (~((st < 0) | (st >= V)).any(axis=2)).sum(axis=1)
        for b in range(B):
            cont = caches[b].contents()
            per_set = {}
            for k in cont:
                per_set.setdefault(_home_set(k, sets), []).append(k)
            assert all(len(v) <= ways for v in per_set.values())
            stamps = [stp for stp, _ in cont.values()]
            assert len(set(stamps)) == len(stamps) and all(0 <= s < n_valid[b] for s in stamps)
            assert caches[b].clock == n_valid[b]
            # the newest valid n-gram of the call is held, with its continuation first
            for w in reversed(range(W)):
                if not ((st[b, w] < 0) | (st[b, w] >= V)).any():
                    assert caches[b].lookup(int(st[b, w, 0]))[0] == tuple(int(x) for x in st[b, w, 1:])
                    assert cont[int(st[b, w, 0])][0] == n_valid[b] - 1
                    break
            for k, (_, conts) in cont.items():
                assert 1 <= len(conts) <= G and len(set(conts)) == len(conts)
