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
