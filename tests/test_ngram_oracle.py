"""The n-gram pool oracles (direct and hashed) against their pins, and planted mistakes they must fail (CPU only)."""
import importlib.util
import os
import sys

import pytest

import pins_ngram
from oracle import ngram

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "ngram.py")
CHECKS = [pins_ngram.check_golden_ngram, pins_ngram.check_ngram_history_replay, pins_ngram.check_ngram_invariants]
CACHE_CHECKS = [pins_ngram.check_golden_cache, pins_ngram.check_cache_hash, pins_ngram.check_cache_history_replay,
                pins_ngram.check_cache_equals_pool_without_overflow, pins_ngram.check_cache_invariants]


def test_golden_ngram_sequences():
    pins_ngram.check_golden_ngram(ngram)


def test_history_replay_agrees():
    pins_ngram.check_ngram_history_replay(ngram)


def test_invariants():
    pins_ngram.check_ngram_invariants(ngram)


def test_cache_golden_sequences():
    pins_ngram.check_golden_cache(ngram)


def test_cache_hash():
    pins_ngram.check_cache_hash(ngram)


def test_cache_history_replay_agrees():
    pins_ngram.check_cache_history_replay(ngram)


def test_cache_equals_pool_without_overflow():
    pins_ngram.check_cache_equals_pool_without_overflow(ngram)


def test_cache_invariants():
    pins_ngram.check_cache_invariants(ngram)


MUTATIONS = [
    ("a held continuation is stored twice", "        if cont in held:\n            held.remove(cont)\n", ""),
    ("a held continuation keeps its old place",
     "        if cont in held:\n            held.remove(cont)\n        held.insert(0, cont)\n",
     "        if cont not in held:\n            held.insert(0, cont)\n"),
    ("the newest is dropped when full", "        held.insert(0, cont)\n        del held[self.G:]\n",
     "        held.insert(0, cont)\n        del held[self.G - 1:self.G]\n        del held[self.G:]\n"),
    ("one continuation too many kept", "del held[self.G:]", "del held[self.G + 1:]"),
    ("oldest first", "held.insert(0, cont)", "held.append(cont)"),
    ("the key is the last token", "key, cont = toks[0], tuple(toks[1:])", "key, cont = toks[-1], tuple(toks[:-1])"),
    ("token V accepted", "if any(t < 0 or t >= self.V for t in toks):", "if any(t < 0 or t > self.V for t in toks):"),
    ("negative tokens accepted", "if any(t < 0 or t >= self.V for t in toks):", "if any(t >= self.V for t in toks):"),
    ("window inserted in reverse", "        for w in range(W):\n            if not pools[b].insert(ngrams[b, w]):",
     "        for w in reversed(range(W)):\n            if not pools[b].insert(ngrams[b, w]):"),
    ("lookup count off by one", "        count[b] = len(found)\n", "        count[b] = min(len(found) + 1, G)\n"),
]


CACHE_SECTION = "# " + "-" * 64 + " the hashed pool"

# Mistakes in the hashed pool; the within-key ones are planted in its class alone, so the
# hashed pool's own pins must catch them.
CACHE_MUTATIONS = [
    ("the newest key is evicted", "oldest = min(entries, key=lambda k: entries[k][0])",
     "oldest = max(entries, key=lambda k: entries[k][0])"),
    ("the smallest key is evicted", "oldest = min(entries, key=lambda k: entries[k][0])", "oldest = min(entries)"),
    ("a hit does not refresh the stamp", "        ent[0] = stamp\n", ""),
    ("a set holds one key too many", "if len(entries) == self.ways:", "if len(entries) == self.ways + 1:"),
    ("a set holds one key too few", "if len(entries) == self.ways:", "if len(entries) >= self.ways - 1 and entries:"),
    ("an evicted key keeps its continuations",
     "                del entries[oldest]\n            entries[key] = [stamp, []]\n",
     "                self.ghost = getattr(self, 'ghost', {})\n"
     "                self.ghost[oldest] = entries.pop(oldest)[1]\n"
     "            entries[key] = [stamp, getattr(self, 'ghost', {}).get(key, [])]\n"),
    ("the hash takes the low bits", ">> (32 - bits)", "& ((1 << bits) - 1)"),
    ("the hash is the key modulo the sets", "return ((int(key) * GOLDEN32) % (1 << 32)) >> (32 - bits)",
     "return int(key) % sets"),
    ("the hash constant is the nearby prime", "GOLDEN32 = 2654435769", "GOLDEN32 = 2654435761"),
    ("skipped n-grams advance the clock",
     "        if any(t < 0 or t >= self.V for t in toks):\n            return False\n"
     "        key, cont = toks[0], tuple(toks[1:])\n        stamp = self.clock\n        self.clock += 1\n",
     "        stamp = self.clock\n        self.clock += 1\n"
     "        if any(t < 0 or t >= self.V for t in toks):\n            return False\n"
     "        key, cont = toks[0], tuple(toks[1:])\n"),
    ("a held continuation is stored twice", "        if cont in held:\n            held.remove(cont)\n", ""),
    ("oldest continuation first", "held.insert(0, cont)", "held.append(cont)"),
    ("one continuation too many kept", "del held[self.G:]", "del held[self.G + 1:]"),
    ("the key is the last token", "key, cont = toks[0], tuple(toks[1:])", "key, cont = toks[-1], tuple(toks[:-1])"),
    ("token V accepted", "if any(t < 0 or t >= self.V for t in toks):", "if any(t < 0 or t > self.V for t in toks):"),
    ("lookup in set zero", "ent = self.table[cache_set(token, self.sets)].get(token)",
     "ent = self.table[0].get(token)"),
]


def _mutant(name, old, new, after=None):
    """The oracle module with `old` replaced by `new` (only past the line `after`, when given)."""
    src = open(SRC, encoding="utf-8").read()
    cut = src.index(after) if after is not None else 0
    head, tail = src[:cut], src[cut:]
    assert tail.count(old) >= 1, f"mutation '{name}' does not apply"
    modname = "ngram_mutant_" + "".join(ch if ch.isalnum() else "_" for ch in name)
    spec = importlib.util.spec_from_loader(modname, loader=None)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[modname] = mod
    exec(compile(head + tail.replace(old, new), f"<{modname}>", "exec"), mod.__dict__)
    return mod


def _expect_caught(mod, name, checks):
    try:
        for check in checks:
            try:
                check(mod)
            except Exception:
                return
        pytest.fail(f"planted mistake '{name}' passed every pin")
    finally:
        sys.modules.pop(mod.__name__, None)


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_reject_planted_mistake(name, old, new):
    _expect_caught(_mutant(name, old, new), name, CHECKS)


@pytest.mark.parametrize("name,old,new", CACHE_MUTATIONS, ids=[m[0] for m in CACHE_MUTATIONS])
def test_cache_pins_reject_planted_mistake(name, old, new):
    _expect_caught(_mutant(name, old, new, after=CACHE_SECTION), name, CACHE_CHECKS)


def test_unmutated_copy_passes():
    mod = _mutant("control", "import numpy as np", "import numpy as np")
    try:
        for check in CHECKS + CACHE_CHECKS:
            check(mod)
    finally:
        sys.modules.pop(mod.__name__, None)
