"""Plant plausible mistakes in copies of the oracle; the pins must reject every copy (CPU only).

Each mutation edits the oracle's source text (a dropped term, a wrong sign,
index or operand, a flipped comparison), loads it as a separate module and runs
the pin checks until one fails. A mutation that passes every pin would mean
the pins cannot see that kind of mistake.
"""
import importlib.util
import os
import sys

import pytest

import pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "verify.py")

MUTATIONS = [
    ("accept compares with <=", "if r < alpha:", "if r <= alpha:"),
    ("ratio operands swapped", "return p_x / q_x", "return q_x / p_x"),
    ("no truncation to one", "if p_x >= q_x:\n        return 1.0\n", ""),
    ("residual sign flipped", "np.maximum(0.0, p_rej - q_rej)", "np.maximum(0.0, q_rej - p_rej)"),
    ("residual without the clamp", "np.maximum(0.0, p_rej - q_rej)", "(p_rej - q_rej)"),
    ("bonus from the wrong row", "softmax64(target[b, K], temperature)", "softmax64(target[b, K - 1], temperature)"),
    ("draw uses the accept uniform", "float(uniforms[b, n, 1])", "float(uniforms[b, n, 0])"),
    ("draw uses position 0's uniform", "float(uniforms[b, n, 1])", "float(uniforms[b, 0, 1])"),
    ("draw boundary inclusive", "np.nonzero(c > tau)", "np.nonzero(c >= tau)"),
    ("softmax not normalised", "return e / np.sum(e)", "return e"),
    ("temperature multiplies", "/ temperature64(temperature)", "* temperature64(temperature)"),
    ("temperature ignored", "/ temperature64(temperature)", "/ 1.0"),
    ("draw not scaled by Z", "tau = float(u) * Z", "tau = float(u)"),
    ("accepted prefix shifted", "tokens[b, :n] = draft_tokens[b, :n]", "tokens[b, :n] = draft_tokens[b, ::-1][:n]"),
    ("rejection position off by one", "n = i                              #", "n = min(i + 1, K)                  #"),
    ("no zero-mass fallback", "if np.sum(w) == 0.0:", "if False:"),
    ("greedy match test inverted", "cand[b, g, L[g]] == amax[b, g, L[g]]", "cand[b, g, L[g]] != amax[b, g, L[g]]"),
    ("greedy highest candidate wins ties", "best = int(np.argmax(L))", "best = int(len(L) - 1 - np.argmax(L[::-1]))"),
    ("greedy extra token from the wrong row", "amax[b, best, Lb]", "amax[b, best, max(Lb - 1, 0)]"),
    ("greedy argmax highest index on ties",
     "return int(np.argmax(np.asarray(row, dtype=np.float64)))",
     "return int(len(row) - 1 - np.argmax(np.asarray(row, dtype=np.float64)[::-1]))"),
    ("greedy counts one position too many", "while L[g] < N - 1 and", "while L[g] < N and"),
    ("top-k drops the ties of the k-th value", "keep = x >= kth", "keep = x > kth"),
    ("top-k threshold off by one", "kth = np.sort(x)[V - k]", "kth = np.sort(x)[max(V - k - 1, 0)]"),
    ("top-p counts the entry's own group", "above = np.where(start > 0, csum[np.maximum(start - 1, 0)], 0.0)",
     "above = csum"),
    ("top-p ignores the temperature", "z = x / temperature64(temperature)\n        e = np.where(keep",
     "z = x\n        e = np.where(keep"),
    ("top-p over the whole row, not the top-k set",
     "e = np.where(keep, np.exp(z - np.max(z)), 0.0)\n        Z", "e = np.exp(z - np.max(z))\n        Z"),
    ("top-p without the largest group", "kept_s = keep[order] & (top | (above < p * Z))",
     "kept_s = keep[order] & (above < p * Z)"),
    ("filtered law renormalised over the whole row",
     "e = np.where(keep, np.exp(z - np.max(z)), 0.0)\n    return e / np.sum(e)",
     "e = np.exp(z - np.max(z))\n    return np.where(keep, e, 0.0) / np.sum(e)"),
    ("draft rows not filtered",
     "keeps = [filter_keep(r, temperature, int(top_k[b]), float(top_p[b])) for r in rows]",
     "keeps = [filter_keep(r, temperature, int(top_k[b]) if j <= K else 0, float(top_p[b]) if j <= K else 1.0)"
     " for j, r in enumerate(rows)]"),
    ("bonus row not filtered",
     "keeps = [filter_keep(r, temperature, int(top_k[b]), float(top_p[b])) for r in rows]",
     "keeps = [filter_keep(r, temperature, int(top_k[b]) if j != K else 0, float(top_p[b]) if j != K else 1.0)"
     " for j, r in enumerate(rows)]"),
]

MUTATIONS += [
    ("token probabilities p/q swapped", "    return p, q\n", "    return q, p\n"),
    ("token probabilities from the next target row", "probs[b, i] = token_probs(target[b, i], draft[b, i],",
     "probs[b, i] = token_probs(target[b, i + 1], draft[b, i],"),
    ("token probabilities of the previous draft token", "int(draft_tokens[b, i]), temperature)",
     "int(draft_tokens[b, max(i - 1, 0)]), temperature)"),
    ("token probability not normalised", "p = float(softmax64(target_row, temperature)[x])",
     "p = float(np.exp(np.asarray(target_row, dtype=np.float64)[x] / temperature64(temperature)))"),
    ("an invalid draft row blanks p too", 'if row_is_valid(target_row) else float("nan")',
     'if row_is_valid(target_row) and row_is_valid(draft_row) else float("nan")'),
    ("filtered token probabilities not renormalised", "probs[b, i, side] = float(law(j)[x])",
     "probs[b, i, side] = float(softmax64(rows[j], temperature)[x]) if keeps[j].keep[x] else 0.0"),
    ("filtered token probabilities p/q swapped", "for side, j in ((0, i), (1, K + 1 + i)):",
     "for side, j in ((1, i), (0, K + 1 + i)):"),
]

MUTATIONS += [
    ("n-gram: no renormalisation after a rejection",
     "alpha = float(live[x]) / left if left > 0.0 else 0.0", "alpha = float(p[x])"),
    ("n-gram: a rejected token keeps its mass", "                live[x] = 0.0                               # residual",
     "                pass                                        # residual"),
    ("n-gram: the highest active candidate's rows", "            g0 = active[0]\n", "            g0 = active[-1]\n"),
    ("n-gram: the prefix filter ignored",
     "            active = [h for h in active if int(cand[b, h, i]) == accepted]", "            active = active"),
    ("n-gram: accept compares with <=", "                if r < alpha:                               # accept iff r",
     "                if r <= alpha:                              # accept iff r"),
    ("n-gram: the draw reads candidate 0's accept uniform", "float(uniforms[b, len(prefix), G])",
     "float(uniforms[b, len(prefix), 0])"),
    ("n-gram: accept uniforms indexed by try order, not candidate",
     "                r = float(uniforms[b, i, h])", "                r = float(uniforms[b, i, active.index(h)])"),
    ("n-gram: the bonus from the first row", "            if i == N - 1:                                  # every",
     "            if i == N - 1 and False:                        # every"),
]

CHECKS = [
    pins.check_golden_sample,
    pins.check_token_probs,
    pins.check_golden_greedy,
    pins.check_softmax_closed_forms,
    pins.check_acceptance_special_cases,
    pins.check_inverse_cdf,
    pins.check_faults,
    pins.check_greedy_argmax_brute_force,
    pins.check_exact_law_on_grid,
    pins.check_acceptance_is_one_minus_tv,
    pins.check_tokens_per_round,
    pins.check_golden_filtered,
    pins.check_filter_top_k_by_rank,
    pins.check_filter_top_p_nucleus,
    pins.check_filter_special_cases,
    pins.check_filters_off_match_plain,
    pins.check_filtered_exact_law,
    pins.check_golden_ngram_sample,
    pins.check_ngram_sample_g1_matches_sample,
    pins.check_ngram_sample_exact_law,
]


def _mutant(name: str, old: str, new: str):
    with open(ORACLE_SRC, encoding="utf-8") as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation '{name}' does not apply: text not found"
    src = src.replace(old, new)
    modname = "oracle_mutant_" + "".join(ch if ch.isalnum() else "_" for ch in name)
    spec = importlib.util.spec_from_loader(modname, loader=None)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[modname] = mod
    exec(compile(src, f"<{modname}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_reject_planted_mistake(name, old, new):
    mod = _mutant(name, old, new)
    try:
        for check in CHECKS:
            try:
                check(mod)
            except Exception:
                return  # caught
        pytest.fail(f"planted mistake '{name}' passed every pin")
    finally:
        sys.modules.pop(mod.__name__, None)


def test_unmutated_copy_passes_every_pin():
    """Control: a copy loaded the same way, with no edit, passes all the checks."""
    mod = _mutant("control", "import numpy as np", "import numpy as np")
    try:
        for check in CHECKS:
            check(mod)
    finally:
        sys.modules.pop(mod.__name__, None)
