"""HIP n-gram pool vs the CPU oracle (needs an MI355X).

Seeded n-gram streams (workloads/ngram.py) with repeated keys, repeated
n-grams and tokens outside [0, V) go through both; after every insert call the
GPU pool's whole table is compared with the oracle's buckets, the skipped
counts bit for bit, and lookups of hit, missing and out-of-range tokens.
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
    print(f"[gpu-ngram] {msg}", flush=True)


def table_as_buckets(pool: rsv.NgramPool) -> dict:
    t = pool.table().cpu().numpy()
    out = {}
    for b, k in zip(*np.nonzero(t[:, :, 0, 0] >= 0)):
        slots = t[b, k]
        held = [tuple(int(x) for x in row) for row in slots if row[0] >= 0]
        # slots are compacted: every empty slot comes after the held ones and is -1 throughout
        assert np.all(slots[len(held):] == -1)
        out[(int(b), int(k))] = held
    return out


def test_golden_sequences_on_gpu():
    for case in load("ngram_worked.json")["cases"]:
        V, G, N = case["V"], case["G"], case["N"]
        B = len(case["steps"][0]["ngrams"])
        pool = rsv.NgramPool(B, V, G, N, DEV)
        for st in case["steps"]:
            sk = pool.insert(torch.tensor(st["ngrams"], dtype=torch.int32, device=DEV))
            assert sk.cpu().tolist() == st["expect_skipped"]
        for lk in case["lookups"]:
            cand, count = pool.lookup(torch.tensor(lk["last"], dtype=torch.int32, device=DEV))
            assert count.cpu().tolist() == lk["expect_count"]
            assert cand.cpu().tolist() == lk["expect_cand"]


CASES = [
    # (B, W, N, V, G, steps, hot, bad)
    (4, 5, 4, 50, 7, 6, 0.6, 0.05),
    (32, 15, 5, 32000, 7, 5, 0.5, 0.02),    # the page's W=15, N=5 and G=7, the greedy workload's V and B
    (3, 64, 2, 9, 1, 4, 0.8, 0.1),          # the largest window, N=2, one slot per key
    (2, 64, 17, 20, 64, 3, 0.9, 0.05),      # the longest n-grams, the most slots
    (5, 1, 3, 7, 2, 12, 0.5, 0.2),          # one n-gram per call
    (6, 0, 3, 7, 2, 1, 0.5, 0.0),           # an empty call
    (3, 33, 6, 5, 5, 6, 0.0, 0.3),          # a tiny vocabulary: every key collides
]


@pytest.mark.parametrize("B,W,N,V,G,steps,hot,bad", CASES, ids=lambda x: str(x))
def test_pool_matches_oracle(B, W, N, V, G, steps, hot, bad):
    log(f"case B={B} W={W} N={N} V={V} G={G}")
    stream = ngram_steps(11, steps, B, W, N, V, hot=hot, n_hot=4, repeat=0.4, bad=bad)
    pool = rsv.NgramPool(B, V, G, N, DEV)
    opools = ngram.new_pools(B, V, G, N)
    for i, st in enumerate(stream):
        sk = pool.insert(torch.from_numpy(st).to(DEV))
        osk = ngram.pool_insert(opools, st)
        torch.cuda.synchronize()
        assert np.array_equal(sk.cpu().numpy(), osk), f"skipped counts differ at step {i}"
        assert table_as_buckets(pool) == ngram.pool_contents(opools), f"pool contents differ after step {i}"
        last = lookup_tokens(i, B, V, stream[: i + 1])
        cand, count = pool.lookup(torch.from_numpy(last).to(DEV))
        ocand, ocount = ngram.pool_lookup(opools, last)
        torch.cuda.synchronize()
        assert np.array_equal(count.cpu().numpy(), ocount)
        assert np.array_equal(cand.cpu().numpy(), ocand)


@pytest.mark.parametrize("kind", ["direct", "hashed"])
def test_lookup_feeds_the_greedy_verify(kind):
    """Candidates from the pool (direct table, or the hashed one with 4 sets of 2 ways) verified
    against logits whose argmax follows one of them."""
    B, G, N, V = 8, 4, 5, 300
    pool = rsv.NgramPool(B, V, G, N, DEV) if kind == "direct" else rsv.NgramCache(B, V, G, N, 4, 2, DEV)
    rng = np.random.default_rng(5)
    grams = rng.integers(0, V, size=(B, G, N)).astype(np.int32)
    grams[:, :, 0] = np.arange(B)[:, None] % V  # every sequence's grams share its last token
    pool.insert(torch.from_numpy(grams).to(DEV))
    last = torch.from_numpy((np.arange(B) % V).astype(np.int32)).to(DEV)
    cand, count = pool.lookup(last)
    torch.cuda.synchronize()
    assert count.cpu().tolist() == [G] * B
    c = cand.cpu().numpy()
    logits = rng.normal(size=(B, G, N, V)).astype(np.float32)
    # candidate 1 of every row matches the argmax for 2 positions, the others not at all
    for b in range(B):
        for g in range(G):
            for i in range(N - 1):
                logits[b, g, i, c[b, g, i]] = 50.0 if (g == 1 and i < 2) else -50.0
    out = rsv.verify_greedy(torch.from_numpy(logits).to(DEV), cand)
    torch.cuda.synchronize()
    assert out.accept_len.cpu().tolist() == [2] * B and out.best.cpu().tolist() == [1] * B
