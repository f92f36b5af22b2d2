"""The n-gram pool oracle against its pins, and planted mistakes it must fail (CPU only)."""
import importlib.util
import os
import sys

import pytest

import pins_ngram
from oracle import ngram

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "ngram.py")
CHECKS = [pins_ngram.check_golden_ngram, pins_ngram.check_ngram_history_replay, pins_ngram.check_ngram_invariants]


def test_golden_ngram_sequences():
    pins_ngram.check_golden_ngram(ngram)


def test_history_replay_agrees():
    pins_ngram.check_ngram_history_replay(ngram)


def test_invariants():
    pins_ngram.check_ngram_invariants(ngram)


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


def _mutant(name, old, new):
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) >= 1, f"mutation '{name}' does not apply"
    modname = "ngram_mutant_" + "".join(ch if ch.isalnum() else "_" for ch in name)
    spec = importlib.util.spec_from_loader(modname, loader=None)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[modname] = mod
    exec(compile(src.replace(old, new), f"<{modname}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_reject_planted_mistake(name, old, new):
    mod = _mutant(name, old, new)
    try:
        for check in CHECKS:
            try:
                check(mod)
            except Exception:
                return
        pytest.fail(f"planted mistake '{name}' passed every pin")
    finally:
        sys.modules.pop(mod.__name__, None)


def test_unmutated_copy_passes():
    mod = _mutant("control", "import numpy as np", "import numpy as np")
    try:
        for check in CHECKS:
            check(mod)
    finally:
        sys.modules.pop(mod.__name__, None)
