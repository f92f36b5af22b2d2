"""Load the hand-worked fixtures under tests/golden/ into arrays."""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    with open(os.path.join(GOLDEN_DIR, name), encoding="utf-8") as f:
        return json.load(f)


def logits_from_probs(probs: list[str], T: float) -> np.ndarray:
    """Logits T*ln(p) (ln 0 = -inf) so that softmax(logits / T) = p."""
    out = []
    for s in probs:
        p = Fraction(s)
        out.append(-math.inf if p == 0 else T * math.log(float(p)))
    return np.array(out, dtype=np.float64)


def probs_from_case(case: dict) -> np.ndarray:
    """The case's hand-derived p_i(x_i), q_i(x_i) as a [1, K, 2] float array (null -> NaN)."""
    return np.array([[[math.nan if v is None else float(Fraction(v)) for v in pair] for pair in case["probs"]]],
                    dtype=np.float64)


def sample_case(case: dict) -> dict:
    T = float(case["T"])
    K = len(case["x"])
    target = np.stack([logits_from_probs(row, T) for row in case["p"]])[None]
    draft = np.stack([logits_from_probs(row, T) for row in case["q"]])[None]
    assert target.shape[1] == K + 1 and draft.shape[1] == K
    uni = np.zeros((1, K + 1, 2), dtype=np.float32)
    uni[0, :, 0] = case["r"]
    uni[0, :, 1] = case["u"]
    return dict(target=target, draft=draft, tokens=np.array([case["x"]], dtype=np.int32), uniforms=uni, T=T,
                expect_tokens=np.array([case["tokens"]], dtype=np.int32),
                expect_n=np.array([case["n_accepted"]], dtype=np.int32), expect_probs=probs_from_case(case),
                name=case["name"])


def greedy_case(case: dict) -> dict:
    rows = [[[(-math.inf if v is None else float(v)) for v in r] for r in g] for g in case["logits"]]
    logits = np.array(rows, dtype=np.float64)[None]
    cand = np.array(case["cand"], dtype=np.int32)[None]
    return dict(logits=logits, cand=cand, expect_tokens=np.array([case["tokens"]], dtype=np.int32),
                expect_len=np.array([case["accept_len"]], dtype=np.int32),
                expect_best=np.array([case["best"]], dtype=np.int32), name=case["name"])


def filtered_case(case: dict) -> dict:
    c = sample_case(case)
    c["top_k"] = np.array([int(case["top_k"])], dtype=np.int32)
    c["top_p"] = np.array([float(case["top_p"])], dtype=np.float32)
    c["expect_kept"] = np.array([case["kept"]], dtype=np.int64)
    return c


def ngram_sample_case(case: dict) -> dict:
    rows = [[[(-math.inf if v is None else float(v)) for v in r] for r in g] for g in case["logits"]]
    return dict(logits=np.array(rows, dtype=np.float64)[None], cand=np.array(case["cand"], dtype=np.int32)[None],
                uniforms=np.array(case["uniforms"], dtype=np.float64)[None], T=float(case["T"]),
                expect_tokens=np.array([case["tokens"]], dtype=np.int32),
                expect_len=np.array([case["accept_len"]], dtype=np.int32),
                expect_rows=np.array([case["rows"]], dtype=np.int32), name=case["name"])
