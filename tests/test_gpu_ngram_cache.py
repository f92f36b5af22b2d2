"""HIP hashed n-gram pool vs the CPU oracle (needs an MI355X).

Seeded n-gram streams (workloads/ngram.py) with repeated keys, repeated n-grams
and tokens outside [0, V) go through both. After every insert call the whole GPU
table is read back and compared with the oracle: each sequence's clock, and for
every held key its set, stamp and continuations (the way a key sits in is free,
but it must sit in its home set). Skipped counts and lookups of hit, evicted,
missing and out-of-range tokens are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import rejection_sampling_verify_sample_amd as rsv
from golden_io import load
from oracle import ngram
from workloads.ngram import lookup_tokens, ngram_steps

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"


def log(msg):
    print(f"[gpu-ngram-cache] {msg}", flush=True)


def gpu_state(cache: rsv.NgramCache):
    """(clocks, {(b, key): (set, stamp, continuations)}) read from the device table."""
    clocks, ents = cache.entries()
    return clocks, {k: (s, st, held) for k, (s, _w, st, held) in ents.items()}


def oracle_state(caches):
    clocks = [c.clock % 2 ** 32 for c in caches]
    out = {}
    for b, c in enumerate(caches):
        for k, (st, conts) in c.contents().items():
            out[(b, k)] = (ngram.cache_set(k, c.sets), st % 2 ** 32, conts)
    return clocks, out


def test_golden_sequences_on_gpu():
    for case in load("ngram_cache_worked.json")["cases"]:
        V, G, N, sets, ways = case["V"], case["G"], case["N"], case["sets"], case["ways"]
        B = len(case["steps"][0]["ngrams"])
        log(f"golden case {case['name']}")
        cache = rsv.NgramCache(B, V, G, N, sets, ways, DEV)
        for st in case["steps"]:
            sk = cache.insert(torch.tensor(st["ngrams"], dtype=torch.int32, device=DEV))
            assert sk.cpu().tolist() == st["expect_skipped"]
            _, ents = gpu_state(cache)
            for b in range(B):
                got = sorted([k, stamp, [list(c) for c in held]] for (bb, k), (_s, stamp, held) in ents.items()
                             if bb == b)
                assert got == st["expect_contents"][b], (case["name"], b)
        for lk in case["lookups"]:
            cand, count = cache.lookup(torch.tensor(lk["last"], dtype=torch.int32, device=DEV))
            assert count.cpu().tolist() == lk["expect_count"]
            assert cand.cpu().tolist() == lk["expect_cand"]


CASES = [
    # (B, W, N, V, G, sets, ways, steps, hot, bad)
    (4, 5, 4, 50, 7, 4, 2, 6, 0.6, 0.05),
    (32, 15, 5, 32000, 7, 512, 8, 5, 0.5, 0.02),     # the page's W=15, N=5 and G=7 at the greedy workload's B, V
    (3, 64, 2, 9, 1, 1, 3, 4, 0.8, 0.1),             # the largest window, one set, one slot per key
    (2, 64, 17, 200, 64, 2, 64, 3, 0.9, 0.05),       # the longest n-grams, the most slots, the most ways
    (5, 1, 3, 7, 2, 1, 1, 12, 0.5, 0.2),             # one n-gram per call into a one-entry table
    (6, 0, 3, 7, 2, 4, 2, 1, 0.5, 0.0),              # an empty call
    (3, 33, 6, 40, 5, 8, 1, 6, 0.3, 0.3),            # direct-mapped: evictions inside every call
    (2, 40, 3, 1000, 3, 1, 64, 8, 0.2, 0.05),        # fully associative over 64 ways, evictions among them
    (4, 20, 4, 152064, 7, 1 << 16, 4, 3, 0.5, 0.02), # a 152064-token vocabulary over 65536 sets
    (256, 15, 5, 152064, 7, 512, 8, 3, 0.5, 0.02),   # the bench's large leg: B=256 V=152064, 512 sets x 8 ways
]


@pytest.mark.parametrize("B,W,N,V,G,sets,ways,steps,hot,bad", CASES)
def test_cache_matches_oracle(B, W, N, V, G, sets, ways, steps, hot, bad):
    log(f"B={B} W={W} N={N} V={V} G={G} sets={sets} ways={ways} steps={steps}")
    stream = ngram_steps(13, steps, B, W, N, V, hot=hot, n_hot=5, repeat=0.4, bad=bad)
    cache = rsv.NgramCache(B, V, G, N, sets, ways, DEV)
    oc = ngram.new_caches(B, V, G, N, sets, ways)
    for i, st in enumerate(stream):
        sk = cache.insert(torch.from_numpy(st).to(DEV))
        osk = ngram.pool_insert(oc, st)
        assert np.array_equal(sk.cpu().numpy(), osk), f"skipped counts differ at step {i}"
        assert gpu_state(cache) == oracle_state(oc), f"table differs after step {i}"
        last = lookup_tokens(i, B, V, stream[: i + 1])
        cand, count = cache.lookup(torch.from_numpy(last).to(DEV))
        ocand, ocount = ngram.pool_lookup(oc, last)
        assert np.array_equal(count.cpu().numpy(), ocount), f"counts differ at step {i}"
        assert np.array_equal(cand.cpu().numpy(), ocand), f"candidates differ at step {i}"


def test_the_most_sets():
    """2^24 sets of one way (one 201 MB table): hashes reach the top set."""
    B, V, G, N, sets, ways = 1, 1 << 30, 1, 2, 1 << 24, 1
    rng = np.random.default_rng(3)
    keys = rng.integers(0, V, 64)
    keys[0] = 0
    keys[1] = V - 1
    st = np.stack([keys, rng.integers(0, V, 64)], axis=1)[None].astype(np.int32)
    log("sets=2^24 ways=1")
    cache = rsv.NgramCache(B, V, G, N, sets, ways, DEV)
    oc = ngram.new_caches(B, V, G, N, sets, ways)
    cache.insert(torch.from_numpy(st).to(DEV))
    ngram.pool_insert(oc, st)
    assert gpu_state(cache) == oracle_state(oc)
    assert max(ngram.cache_set(int(k), sets) for k in keys) > sets - (sets >> 3)
    cand, count = cache.lookup(torch.from_numpy(keys[:1].astype(np.int32)).to(DEV))
    ocand, ocount = ngram.pool_lookup(oc, keys[:1].astype(np.int32))
    assert np.array_equal(cand.cpu().numpy(), ocand) and np.array_equal(count.cpu().numpy(), ocount)


def test_clock_wraps():
    """Clocks set 5 short of 2^32 before the first insert: stamps and ages taken modulo 2^32."""
    B, W, N, V, G, sets, ways = 3, 12, 3, 30, 2, 2, 2
    stream = ngram_steps(17, 4, B, W, N, V, hot=0.5, n_hot=6, repeat=0.3, bad=0.1)
    cache = rsv.NgramCache(B, V, G, N, sets, ways, DEV)
    start = 2 ** 32 - 5
    view = cache.buffer[: B * cache.seq_elems].view(B, cache.seq_elems)
    view[:, 0] = start - 2 ** 32  # the same 32 bits as an int32
    oc = ngram.new_caches(B, V, G, N, sets, ways)
    for c in oc:
        c.clock = start
    log("clock wrap")
    for i, st in enumerate(stream):
        cache.insert(torch.from_numpy(st).to(DEV))
        ngram.pool_insert(oc, st)
        assert gpu_state(cache) == oracle_state(oc), f"table differs after step {i}"
    assert all(c.clock > 2 ** 32 for c in oc)


def test_without_overflow_equals_the_direct_pool():
    """With room for every key the hashed pool's lookups equal the direct pool's (both on the GPU)."""
    B, W, N, V, G = 8, 15, 5, 64, 7
    stream = ngram_steps(19, 6, B, W, N, V, hot=0.5, n_hot=4, repeat=0.4, bad=0.05)
    cache = rsv.NgramCache(B, V, G, N, 16, 64, DEV)
    pool = rsv.NgramPool(B, V, G, N, DEV)
    for i, st in enumerate(stream):
        t = torch.from_numpy(st).to(DEV)
        assert torch.equal(cache.insert(t), pool.insert(t))
        last = torch.from_numpy(lookup_tokens(i, B, V, stream[: i + 1])).to(DEV)
        c1, n1 = cache.lookup(last)
        c2, n2 = pool.lookup(last)
        assert torch.equal(c1, c2) and torch.equal(n1, n2), f"step {i}"
