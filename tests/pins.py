"""Checks that pin the CPU oracle to facts fixed outside itself.

Every check takes the oracle module as its argument, so the same checks run
against the real oracle (tests/test_oracle_pins.py) and against copies with a
planted mistake (tests/test_pin_mutations.py), which they must reject.

Sources of the pinned facts (page title, section):
  Speculative Decoding —— LLM推理优化技术（一）: §2.2 the output law of the
    accept/resample rule is exactly p; §2.4 E[accept] = 1 - TV(p, q);
    §3.1 tokens per round (1 - a^(K+1)) / (1 - a).
  Lookahead Decoding 完全拆解:Jacobi 迭代与 N-gram 池: eq. (5), the expected
    tokens per step with b disjoint candidates of gamma tokens each; section
    "采样模式的验证": greedy-drafted (one-hot) candidates keep the target's law
    under a full sampling verification.
  kwkr.cn/news/620797 notes §3.4: top-k / top-p must truncate the draft and
    the target side alike, and the correction is drawn inside the kept set.
  Hand-worked rounds in tests/golden/ (derivations stored beside them).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
from scipy import special, stats

from golden_io import filtered_case, greedy_case, load, logits_from_probs, ngram_sample_case, sample_case
from workloads import make_greedy_inputs, verify_uniforms


# --------------------------------------------------------------------------- golden

def check_golden_sample(orc) -> None:
    for case in load("sample_worked.json")["cases"]:
        c = sample_case(case)
        res = orc.oracle_sample(c["target"], c["draft"], c["tokens"], c["uniforms"], c["T"])
        assert np.array_equal(res.tokens, c["expect_tokens"]), (c["name"], res.tokens, c["expect_tokens"])
        assert np.array_equal(res.n_accepted, c["expect_n"]), (c["name"], res.n_accepted, c["expect_n"])


def check_golden_greedy(orc) -> None:
    for case in load("greedy_worked.json")["cases"]:
        c = greedy_case(case)
        res = orc.oracle_greedy(c["logits"], c["cand"])
        assert np.array_equal(res.tokens, c["expect_tokens"]), (c["name"], res.tokens)
        assert np.array_equal(res.accept_len, c["expect_len"]), (c["name"], res.accept_len)
        assert np.array_equal(res.best, c["expect_best"]), (c["name"], res.best)


def _same_probs(got: np.ndarray, expect: np.ndarray, what) -> None:
    assert np.array_equal(np.isnan(got), np.isnan(expect)), (what, "NaN pattern", got, expect)
    fin = ~np.isnan(expect)
    assert np.allclose(got[fin], expect[fin], rtol=1e-12, atol=1e-15), (what, got, expect)


def check_token_probs(orc) -> None:
    """The out_probs values p_i(x_i), q_i(x_i): the two numbers alpha is formed from (§2.1).

    Pinned three ways: the hand-derived values of every golden round (plain and
    filtered: the filtered values are those of the renormalised kept laws);
    closed forms on rows with one raised logit per position, distinct on every
    row, so a swapped pair, a value from the wrong row or of the wrong token, or
    an unnormalised value shows; and the per-side reading of a value that does
    not exist -- p_i(x_i) depends on target row i and x_i alone, q_i(x_i) on draft
    row i and x_i alone, so a row with no finite logit blanks only its own side,
    and a token outside the vocabulary blanks both.
    """
    for case in load("sample_worked.json")["cases"]:
        c = sample_case(case)
        res = orc.oracle_sample(c["target"], c["draft"], c["tokens"], c["uniforms"], c["T"])
        _same_probs(res.probs, c["expect_probs"], c["name"])
    for case in load("filtered_worked.json")["cases"]:
        c = filtered_case(case)
        res = orc.oracle_sample_filtered(c["target"], c["draft"], c["tokens"], c["uniforms"], c["T"],
                                         c["top_k"], c["top_p"])
        _same_probs(res.probs, c["expect_probs"], c["name"])
    # closed forms: target row i is a_i at x_i over V-1 zeros, draft row i is d_i at x_i
    # over zeros, so p_i(x_i) = e^(a_i/T) / (e^(a_i/T) + V - 1) and likewise q_i(x_i)
    V, K, T = 37, 5, 0.8
    T64 = float(np.float32(T))
    a = np.array([1.5, -0.5, 3.0, 0.25, 2.0, 0.75])       # K + 1 target rows (row K: the bonus row)
    d = np.array([0.5, 2.5, -1.0, 1.75, -0.25])
    x = np.array([[3, 11, 0, 36, 20]], dtype=np.int32)
    tgt = np.zeros((1, K + 1, V))
    drf = np.zeros((1, K, V))
    for i in range(K):
        tgt[0, i, x[0, i]] = a[i]
        drf[0, i, x[0, i]] = d[i]
    tgt[0, K, 7] = a[K]
    uni = np.full((1, K + 1, 2), 0.5, dtype=np.float32)

    def closed(v):
        return math.exp(v / T64) / (math.exp(v / T64) + V - 1)

    expect = np.array([[[closed(a[i]), closed(d[i])] for i in range(K)]])
    res = orc.oracle_sample(tgt, drf, x, uni, T)
    _same_probs(res.probs, expect, "closed forms")
    # with every raised logit above the zeros, top-k = 1 keeps only the raised entry: every value is 1
    up_t, up_d = np.abs(tgt) + (tgt != 0) * 0.5, np.abs(drf) + (drf != 0) * 0.5
    res = orc.oracle_sample_filtered(up_t, up_d, x, uni, T, np.array([1]), np.array([1.0], dtype=np.float32))
    _same_probs(res.probs, np.ones((1, K, 2)), "top-k 1")
    # per-side blanks: target row 1 and draft row 3 hold no finite logit; token 4 is outside [0, V)
    tgt2, drf2, x2 = tgt.copy(), drf.copy(), x.copy()
    tgt2[0, 1, :] = -np.inf
    drf2[0, 3, :] = -np.inf
    x2[0, 4] = V
    expect2 = expect.copy()
    expect2[0, 1, 0] = np.nan
    expect2[0, 3, 1] = np.nan
    expect2[0, 4, :] = np.nan
    res = orc.oracle_sample(tgt2, drf2, x2, uni, T)
    _same_probs(res.probs, expect2, "per-side blanks")
    res = orc.oracle_sample_filtered(tgt2, drf2, x2, uni, T, np.array([0]), np.array([1.0], dtype=np.float32))
    _same_probs(res.probs, expect2, "per-side blanks, filters off")


# --------------------------------------------------------------------------- closed forms

def check_softmax_closed_forms(orc) -> None:
    # equal logits: 1/V
    for V in (1, 3, 1000):
        p = orc.softmax64(np.full(V, 2.5), 0.7)
        assert np.allclose(p, 1.0 / V, rtol=1e-14, atol=0)
    # one logit a above V-1 zeros: e^(a/T) / (e^(a/T) + V - 1)
    for a, V, T in ((3.0, 10, 1.0), (-2.0, 7, 0.5), (40.0, 128256, 2.0)):
        x = np.zeros(V)
        x[V // 2] = a
        T64 = float(np.float32(T))
        expect = math.exp(a / T64) / (math.exp(a / T64) + V - 1)
        p = orc.softmax64(x, T)
        assert abs(p[V // 2] - expect) <= 1e-14 * expect
        assert abs(p[0] - 1.0 / (math.exp(a / T64) + V - 1)) <= 1e-14 * p[0]
    # -inf entries carry no mass; the rest renormalise
    p = orc.softmax64(np.array([0.0, -np.inf, 0.0, -np.inf]), 1.0)
    assert np.array_equal(p, [0.5, 0.0, 0.5, 0.0])
    # special case that reduces to a library routine: scipy's softmax of x / T,
    # with T the float32 value the caller passes
    rng = np.random.default_rng(7)
    for T in (1.0, 0.7, 0.8, 1.3):
        x = rng.normal(0, 3, 5000)
        ref = special.softmax(x / float(np.float32(T)))
        assert np.allclose(orc.softmax64(x, T), ref, rtol=1e-12, atol=1e-300)


def check_acceptance_special_cases(orc) -> None:
    a = orc.acceptance_probability
    assert a(0.5, 0.25) == 1.0 and a(0.25, 0.25) == 1.0
    assert a(0.125, 0.5) == 0.25
    assert a(0.0, 0.5) == 0.0 and a(0.0, 0.0) == 0.0
    assert a(0.3, 0.0) == 1.0
    rng = np.random.default_rng(11)
    V, K = 50, 3
    # p == q at every position: every draft is accepted for any r < 1
    tgt = rng.normal(0, 2, (8, K + 1, V))
    drf = tgt[:, :K].copy()
    toks = rng.integers(0, V, (8, K)).astype(np.int32)
    uni = np.full((8, K + 1, 2), 1.0 - 2.0 ** -24, dtype=np.float32)
    res = orc.oracle_sample(tgt, drf, toks, uni, 1.0)
    assert np.all(res.n_accepted == K)
    assert np.array_equal(res.tokens[:, :K], toks)
    # one-hot q at x: alpha = p(x). Target uniform on 4 tokens holding x, so p(x) = 1/4.
    tgt = np.full((2, 2, 8), -np.inf)
    tgt[:, :, :4] = 0.0
    drf = np.full((2, 1, 8), -np.inf)
    drf[:, 0, 2] = 5.0
    toks = np.array([[2], [2]], dtype=np.int32)
    uni = np.zeros((2, 2, 2), dtype=np.float32)
    uni[0, 0, 0] = 0.25 - 2.0 ** -24      # just below alpha: accept
    uni[1, 0, 0] = 0.25                   # on alpha: reject
    res = orc.oracle_sample(tgt, drf, toks, uni, 1.0)
    assert res.n_accepted.tolist() == [1, 0]
    # one-hot p at y, draft token x != y: alpha = 0 and the residual is all on y
    tgt = np.full((3, 2, 6), -np.inf)
    tgt[:, 0, 4] = 1.0
    tgt[:, 1, :] = 0.0
    drf = rng.normal(0, 1, (3, 1, 6))
    toks = np.array([[0], [1], [5]], dtype=np.int32)
    uni = np.zeros((3, 2, 2), dtype=np.float32)
    uni[:, 0, 1] = [0.0, 0.5, 1.0 - 2.0 ** -24]
    res = orc.oracle_sample(tgt, drf, toks, uni, 1.0)
    assert res.n_accepted.tolist() == [0, 0, 0]
    assert res.tokens[:, 0].tolist() == [4, 4, 4]


def check_inverse_cdf(orc) -> None:
    # uniform weights on 2^m tokens: C_k = (k+1)/2^m exactly; u = k/2^m selects k
    for m in (1, 3, 6):
        n = 2 ** m
        w = np.full(n, 1.0 / n)
        for k in range(n):
            assert orc.inverse_cdf_draw(w, k / n)[0] == k
            assert orc.inverse_cdf_draw(w, (k + 0.5) / n)[0] == k
    # zero-mass tokens are never drawn, even when u*Z lands on their boundary
    w = np.array([0.0, 1.0, 0.0, 1.0, 0.0])
    assert orc.inverse_cdf_draw(w, 0.0)[0] == 1
    assert orc.inverse_cdf_draw(w, 0.5)[0] == 3
    assert orc.inverse_cdf_draw(w, 1.0 - 2.0 ** -24)[0] == 3
    # unnormalised weights: the draw compares u*Z with the running sums
    w = np.array([1.0, 2.0, 1.0])
    assert [orc.inverse_cdf_draw(w, u)[0] for u in (0.0, 0.24, 0.25, 0.74, 0.75)] == [0, 0, 1, 1, 2]
    # the margin is the distance of u from the ends of the chosen interval of the
    # normalised CDF: here [1/4, 3/4) for u = 0.3, so 0.05
    k, Z, margin = orc.inverse_cdf_draw(w, 0.3)
    assert k == 1 and Z == 4.0 and abs(margin - 0.05) < 1e-15


# --------------------------------------------------------------------------- exact law on a grid

GRID_PAIRS = [
    # (p0, q0, p1): dyadic laws; every alpha and every w/Z is a multiple of 1/64
    (["1/2", "1/4", "1/8", "1/8"], ["1/8", "1/8", "1/4", "1/2"], ["1/16", "3/16", "1/4", "1/2"]),
    (["1/2", "1/2", "0", "0"], ["0", "0", "3/4", "1/4"], ["1/4", "1/4", "1/4", "1/4"]),
    (["3/8", "1/8", "1/2", "0"], ["3/8", "1/8", "1/2", "0"], ["0", "0", "1/8", "7/8"]),
    (["0", "5/16", "1/4", "1/16", "3/8", "0"], ["1/8", "1/16", "1/2", "1/16", "1/8", "1/8"],
     ["1/2", "0", "0", "0", "0", "1/2"]),
]


def check_exact_law_on_grid(orc, pairs=GRID_PAIRS, grid: int = 64) -> None:
    """Theorem of Speculative Decoding -- LLM推理优化技术（一） §2.2: the emitted token has law p exactly.

    K = 1. The draft token x runs over q's support with weight q(x) (exact), the
    accept uniform r and the draw uniform u over the midpoints of a 1/grid mesh.
    All boundaries are multiples of 1/grid, so each mesh cell lies on one side
    of each boundary and the mesh integral is exact. Checked exactly in
    rationals: P(first token = y) = p0(y); P(all accepted) = 1 - TV(p0, q0)
    (§2.4); P(all accepted, bonus = y) = (1 - TV) p1(y) (§2.3 step 4). The
    bonus uniform is 1 - u, so a draw that read the wrong position's uniform
    would show up as a mirrored law.
    """
    mids = (np.arange(grid) + 0.5) / grid
    for p0s, q0s, p1s in pairs:
        p0 = [Fraction(s) for s in p0s]
        q0 = [Fraction(s) for s in q0s]
        p1 = [Fraction(s) for s in p1s]
        V = len(p0)
        xs = [x for x in range(V) if q0[x] > 0]
        rr, uu = np.meshgrid(mids, mids, indexing="ij")
        rr, uu = rr.ravel(), uu.ravel()
        cells = rr.size
        B = len(xs) * cells
        tgt = np.stack([logits_from_probs(p0s, 1.0), logits_from_probs(p1s, 1.0)])
        tgt = np.broadcast_to(tgt, (B, 2, V))
        drf = np.broadcast_to(logits_from_probs(q0s, 1.0), (B, 1, V))
        toks = np.repeat(np.array(xs, dtype=np.int32), cells)[:, None]
        uni = np.zeros((B, 2, 2), dtype=np.float64)
        uni[:, 0, 0] = np.tile(rr, len(xs))
        uni[:, 0, 1] = np.tile(uu, len(xs))
        uni[:, 1, 1] = 1.0 - np.tile(uu, len(xs))
        res = orc.oracle_sample(tgt, drf, toks, uni, 1.0, with_probs=False)
        first = np.zeros(V, dtype=object)
        bonus = np.zeros(V, dtype=object)
        accepted = Fraction(0)
        for j, x in enumerate(xs):
            sl = slice(j * cells, (j + 1) * cells)
            wgt = q0[x] / cells
            t0 = res.tokens[sl, 0]
            n = res.n_accepted[sl]
            assert np.all(n >= 0)
            for y in range(V):
                first[y] += wgt * int(np.sum(t0 == y))
                bonus[y] += wgt * int(np.sum((n == 1) & (res.tokens[sl, 1] == y)))
            accepted += wgt * int(np.sum(n == 1))
        tv = sum(abs(a - b) for a, b in zip(p0, q0)) / 2
        assert list(first) == p0, ("first-token law", list(first), p0)
        assert accepted == 1 - tv, ("acceptance", accepted, 1 - tv)
        assert list(bonus) == [(1 - tv) * v for v in p1], ("bonus law", list(bonus))


# --------------------------------------------------------------------------- statistics

def _sample_from(q: np.ndarray, rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.choice(q.shape[-1], size=n, p=q / q.sum()).astype(np.int32)


CHI_V = (2, 5, 16)
CHI_CHUNK = 50000


def _chisquare_laws(V: int):
    """(target logits, draft logits) of the chi-square law for vocabulary V (fixed seeds)."""
    rng = np.random.default_rng([2024, V])
    lt = rng.normal(0, 1.5, V)
    ld = rng.normal(0, 1.5, V)
    if V == 16:                       # disjoint-ish supports: part of the target mass where q has none
        ld[:4] = -np.inf
    return lt, ld


def chisquare_counts(orc, V: int, chunk: int, n: int) -> np.ndarray:
    """Histogram of the emitted token over n verify rows (K = 1) of chunk `chunk` of the V-token law."""
    lt, ld = _chisquare_laws(V)
    q = special.softmax(ld)
    toks = _sample_from(q, np.random.default_rng([2025, V, chunk]), n)[:, None]
    tgt = np.broadcast_to(np.stack([lt, lt]), (n, 2, V))
    drf = np.broadcast_to(ld, (n, 1, V))
    uni = verify_uniforms(100 + V, chunk, n, 1)
    res = orc.oracle_sample(tgt, drf, toks, uni, 1.0, with_probs=False)
    return np.bincount(res.tokens[:, 0], minlength=V)


def check_chisquare_law(orc, trials: int = 30000, map_fn=map) -> None:
    """Output law = p (§2.2) by chi-square on non-dyadic laws; p-value >= 1e-3.

    `trials` rows per vocabulary, in chunks of CHI_CHUNK (each with its own
    seeds); `map_fn` maps chisquare_counts over (V, chunk, n) argument tuples, so
    a caller can spread the chunks over worker processes.
    """
    for V in CHI_V:
        jobs = [(V, c, min(CHI_CHUNK, trials - c * CHI_CHUNK)) for c in range((trials + CHI_CHUNK - 1) // CHI_CHUNK)]
        counts = sum(map_fn(lambda a: chisquare_counts(orc, *a), jobs)) if map_fn is map else sum(map_fn(jobs))
        lt, _ = _chisquare_laws(V)
        p = special.softmax(lt)
        pv = stats.chisquare(counts, p * trials).pvalue
        assert pv >= 1e-3, (V, trials, pv)


def _fixed_tv_rows(rng, V: int, K: int, alpha: float):
    """Logit rows with TV(p_i, q_i) = 1 - alpha at every position: q = (1-e) p + e delta_k."""
    tgt = np.empty((K + 1, V))
    drf = np.empty((K, V))
    qs = []
    for i in range(K + 1):
        p = rng.dirichlet(np.ones(V))
        tgt[i] = np.log(p)
        if i < K:
            k = int(np.argmin(p))
            eps = (1.0 - alpha) / (1.0 - p[k])
            q = (1.0 - eps) * p
            q[k] += eps
            drf[i] = np.log(q)
            qs.append(q)
    return tgt, drf, qs


def check_acceptance_is_one_minus_tv(orc, trials: int = 20000) -> None:
    """E[accept at i | position i reached] = 1 - TV(p_i, q_i) (§2.4), within 5 sigma."""
    rng = np.random.default_rng(99)
    V, K = 8, 4
    tgt = rng.normal(0, 1.2, (K + 1, V))
    drf = tgt[:K] + rng.normal(0, [[0.3], [0.8], [1.5], [3.0]], (K, V))
    p = special.softmax(tgt[:K], axis=1)
    q = special.softmax(drf, axis=1)
    tv = 0.5 * np.abs(p - q).sum(axis=1)
    toks = np.stack([_sample_from(q[i], rng, trials) for i in range(K)], axis=1)
    uni = verify_uniforms(5, 0, trials, K)
    res = orc.oracle_sample(np.broadcast_to(tgt, (trials, K + 1, V)), np.broadcast_to(drf, (trials, K, V)),
                            toks, uni, 1.0, with_probs=False)
    n = res.n_accepted
    for i in range(K):
        reached = n >= i
        acc = n[reached] > i
        m = reached.sum()
        expect = 1.0 - tv[i]
        sd = math.sqrt(expect * (1 - expect) / m)
        assert abs(acc.mean() - expect) <= 5 * sd, (i, acc.mean(), expect, sd)


def tokens_per_round(alpha: float, K: int) -> float:
    """(1 - a^(K+1)) / (1 - a) (Speculative Decoding -- LLM推理优化技术（一） §3.1)."""
    return (1.0 - alpha ** (K + 1)) / (1.0 - alpha)


def check_tokens_per_round(orc, trials: int = 8000) -> None:
    rng = np.random.default_rng(31)
    V = 8
    for K, alpha in ((3, 0.5), (5, 0.8), (7, 0.9)):
        tgt, drf, qs = _fixed_tv_rows(rng, V, K, alpha)
        toks = np.stack([_sample_from(qs[i], rng, trials) for i in range(K)], axis=1)
        uni = verify_uniforms(77 + K, 0, trials, K)
        res = orc.oracle_sample(np.broadcast_to(tgt, (trials, K + 1, V)), np.broadcast_to(drf, (trials, K, V)),
                                toks, uni, 1.0, with_probs=False)
        got = res.n_accepted + 1
        expect = tokens_per_round(alpha, K)
        sd = got.std() / math.sqrt(trials)
        assert abs(got.mean() - expect) <= 5 * sd, (K, alpha, got.mean(), expect, sd)


def lookahead_eq5(alpha: float, gamma: int, b: int) -> float:
    """E(#tokens) = (gamma+1) - sum_{i=1..gamma} (1 - alpha^i)^b (Lookahead Decoding 完全拆解, eq. (5))."""
    return (gamma + 1) - sum((1.0 - alpha ** i) ** b for i in range(1, gamma + 1))


def check_greedy_eq5(orc, B: int = 6000) -> None:
    """Mean accepted length + 1 over B rows of G disjoint candidates matches eq. (5), within 5 sigma.

    float32 logits (no bf16 ties), so a candidate token matches the argmax with
    probability alpha = 0.6 + 0.4/V, independently per position and candidate.
    """
    G, N, V = 7, 5, 64
    g = make_greedy_inputs(0, B=B, G=G, N=N, V=V, dtype="f32", seed=3)
    res = orc.oracle_greedy(g.logits_f32(), g.cand)
    got = res.accept_len + 1
    alpha = 0.6 + 0.4 / V
    expect = lookahead_eq5(alpha, N - 1, G)
    sd = got.std() / math.sqrt(B)
    assert abs(got.mean() - expect) <= 5 * sd, (got.mean(), expect, sd)
    p_full = 1.0 - (1.0 - alpha ** (N - 1)) ** G
    frac = np.mean(res.accept_len == N - 1)
    assert abs(frac - p_full) <= 5 * math.sqrt(p_full * (1 - p_full) / B), (frac, p_full)


def check_greedy_argmax_brute_force(orc) -> None:
    """Lowest-index argmax checked against a plain scan on small rows with many ties."""
    rng = np.random.default_rng(5)
    for _ in range(300):
        V = int(rng.integers(1, 12))
        row = rng.integers(-3, 3, V).astype(np.float64)
        row[rng.random(V) < 0.2] = -np.inf
        if not np.any(np.isfinite(row)):
            continue
        best, best_v = 0, row[0]
        for v in range(1, V):
            if row[v] > best_v:
                best, best_v = v, row[v]
        assert orc.first_argmax(row) == best


def check_faults(orc) -> None:
    """Fault reading: only consulted rows can fault; a fault gives n = -1 and all tokens -1."""
    V, K = 6, 2
    tgt = np.zeros((4, K + 1, V))
    drf = np.zeros((4, K, V))
    drf[:, 0, 3:] = -np.inf                 # q0 uniform on {0,1,2}
    toks = np.array([[4, 0], [0, 0], [0, 0], [0, 0]], dtype=np.int32)
    uni = np.zeros((4, K + 1, 2), dtype=np.float32)
    # row 0: x0 = 4 has q0 = 0 and p0 = 1/6 > 0: alpha = 1 -> accepted, x1 fine -> n = 2
    # row 1: draft row 1 all -inf -> consulted at i = 1 (x0 accepted) -> fault
    drf[1, 1, :] = -np.inf
    # row 2: x0 rejected (target mass 0 at x0) -> draft row 1 never consulted -> no fault
    tgt[2, 0, 0] = -np.inf
    drf[2, 1, :] = -np.inf
    # row 3: all accepted, bonus row all -inf -> fault
    tgt[3, K, :] = -np.inf
    res = orc.oracle_sample(tgt, drf, toks, uni, 1.0)
    assert res.n_accepted.tolist() == [2, -1, 0, -1]
    assert np.all(res.tokens[[1, 3]] == -1)
    assert res.tokens[0, :2].tolist() == [4, 0] and 0 <= res.tokens[0, 2] < V
    assert res.tokens[2, 1:].tolist() == [-1, -1] and res.tokens[2, 0] in (1, 2, 3, 4, 5)


# --------------------------------------------------------------------------- top-k / top-p filtering

def check_golden_filtered(orc) -> None:
    for case in load("filtered_worked.json")["cases"]:
        c = filtered_case(case)
        res = orc.oracle_sample_filtered(c["target"], c["draft"], c["tokens"], c["uniforms"], c["T"],
                                         c["top_k"], c["top_p"])
        assert np.array_equal(res.tokens, c["expect_tokens"]), (c["name"], res.tokens)
        assert np.array_equal(res.n_accepted, c["expect_n"]), (c["name"], res.n_accepted)
        assert np.array_equal(res.kept, c["expect_kept"]), (c["name"], res.kept)


def _rank_keep(x: np.ndarray, k: int) -> np.ndarray:
    """Brute force: keep v iff fewer than k entries are strictly larger."""
    return np.array([np.sum(x > x[v]) < k for v in range(x.size)])


def check_filter_top_k_by_rank(orc) -> None:
    """top-k against a counting brute force on small rows full of ties and -inf."""
    rng = np.random.default_rng(17)
    for _ in range(400):
        V = int(rng.integers(1, 14))
        x = rng.integers(-3, 4, V).astype(np.float64)
        x[rng.random(V) < 0.15] = -np.inf
        k = int(rng.integers(-1, V + 2))
        kr = orc.filter_keep(x, 1.0, k, 1.0)
        if not np.any(np.isfinite(x)):
            assert not kr.keep.any()
            continue
        expect = _rank_keep(x, k) if 0 < k < V else np.ones(V, dtype=bool)
        assert np.array_equal(kr.keep, expect), (x, k, kr.keep)
        assert kr.margin == np.inf
        if 0 < k < V and np.unique(x).size == V:
            assert kr.keep.sum() == k        # distinct values: exactly k


def check_filter_top_p_nucleus(orc) -> None:
    """top-p against the nucleus definition in exact rationals.

    Laws are small integer weights w (zero weight = -inf logit), taken at
    temperature 1 and 1/2 (logits T ln w, so the tempered law is w itself).
    The nucleus: among the thresholds t (distinct kept values, high to low) the
    first whose set {w >= t} reaches mass >= p of the top-k set; the row's
    largest group is kept whatever p is. Cases closer than 1e-9 to a boundary
    are skipped (the oracle is float64).
    """
    rng = np.random.default_rng(23)
    checked = 0
    for _ in range(600):
        V = int(rng.integers(1, 10))
        w = rng.integers(0, 6, V)
        if w.max() == 0:
            continue
        T = float(rng.choice([1.0, 0.5]))
        x = np.array([T * math.log(v) if v > 0 else -math.inf for v in w])
        k = int(rng.integers(0, V + 1))
        p = float(np.float32(rng.choice([0.0, 0.1, 0.3, 0.5, 0.7, 0.9, 0.95, rng.random()])))
        topk = _rank_keep(x, k) if 0 < k < V else np.ones(V, dtype=bool)
        ws = [Fraction(int(v)) if topk[i] else Fraction(0) for i, v in enumerate(w)]
        Z = sum(ws)
        P = Fraction(p)
        vals = sorted({int(w[i]) for i in range(V) if topk[i]}, reverse=True)
        chosen = vals[0]
        near = False
        for t in vals:
            mass = sum(ws[i] for i in range(V) if topk[i] and w[i] >= t) / Z
            if abs(mass - P) < Fraction(1, 10 ** 9):
                near = True
            chosen = t
            if mass >= P:
                break
        if near:
            continue
        expect = np.array([bool(topk[i]) and int(w[i]) >= chosen for i in range(V)])
        kr = orc.filter_keep(x, T, k, p)
        assert np.array_equal(kr.keep, expect), (w.tolist(), T, k, p, kr.keep, expect)
        checked += 1
    assert checked > 300


def check_filter_special_cases(orc) -> None:
    rng = np.random.default_rng(29)
    for _ in range(100):
        V = int(rng.integers(2, 40))
        x = np.round(rng.normal(0, 2, V), 1)
        x[rng.random(V) < 0.1] = -np.inf
        if not np.any(np.isfinite(x)):
            continue
        top = x == np.max(x)
        T = float(rng.choice([0.5, 1.0, 1.7]))
        # k = 1 and p -> 0 both keep exactly the entries of the largest logit
        assert np.array_equal(orc.filter_keep(x, T, 1, 1.0).keep, top)
        assert np.array_equal(orc.filter_keep(x, T, 0, 1e-30).keep, top)
        assert np.array_equal(orc.filter_keep(x, T, 0, 0.0).keep, top)
        # off: k <= 0 or k >= V, p >= 1 or NaN
        for k, p in ((0, 1.0), (V, 1.0), (-3, 2.0), (V + 5, float("nan"))):
            assert orc.filter_keep(x, T, k, p).keep.all()
        # nested: smaller k or smaller p keeps a subset
        prev = np.ones(V, dtype=bool)
        for k in range(V, 0, -1):
            cur = orc.filter_keep(x, T, k, 1.0).keep
            assert np.all(cur <= prev)
            prev = cur
        prev = np.ones(V, dtype=bool)
        for p in (0.99, 0.9, 0.7, 0.5, 0.2, 0.01):
            cur = orc.filter_keep(x, T, 0, p).keep
            assert np.all(cur <= prev) and cur[top].all()
            prev = cur
        # top-p never keeps an entry without mass
        assert not np.any(orc.filter_keep(x, T, 0, 0.999).keep & np.isneginf(x))
        # the kept mass of a top-p cut reaches p; without its lowest kept group it does not
        kr = orc.filter_keep(x, T, 0, 0.8)
        pz = special.softmax(np.where(np.isneginf(x), -np.inf, x / T))
        low = x == np.min(x[kr.keep])
        assert pz[kr.keep].sum() >= 0.8 - 1e-12 or kr.keep.all()
        assert pz[kr.keep & ~low].sum() < 0.8 + 1e-12
    assert not orc.filter_keep(np.full(5, -np.inf), 1.0, 2, 0.5).keep.any()
    # temperature matters to top-p, not to top-k: a cut that moves with T
    x = np.log(np.array([4.0, 2.0, 2.0, 1.0, 1.0]))
    assert orc.filter_keep(x, 1.0, 0, 0.7).keep.tolist() == [True, True, True, False, False]
    assert orc.filter_keep(x, 0.5, 0, 0.7).keep.tolist() == [True, True, True, False, False]
    assert orc.filter_keep(x, 0.25, 0, 0.7).keep.tolist() == [True, False, False, False, False]
    assert orc.filter_keep(x, 0.25, 3, 1.0).keep.tolist() == [True, True, True, False, False]


def check_filters_off_match_plain(orc) -> None:
    """With both filters off the filtered verify is the plain verify, output for output."""
    rng = np.random.default_rng(31)
    B, K, V = 40, 3, 30
    tgt = rng.normal(0, 2, (B, K + 1, V))
    drf = tgt[:, :K] + rng.normal(0, 1, (B, K, V))
    tgt[rng.random(tgt.shape) < 0.05] = -np.inf
    toks = rng.integers(0, V, (B, K)).astype(np.int32)
    uni = verify_uniforms(9, 0, B, K)
    plain = orc.oracle_sample(tgt, drf, toks, uni, 0.8)
    for k, p in ((0, 1.0), (V, 1.5)):
        f = orc.oracle_sample_filtered(tgt, drf, toks, uni, 0.8, np.full(B, k), np.full(B, p, dtype=np.float32))
        assert np.array_equal(f.tokens, plain.tokens) and np.array_equal(f.n_accepted, plain.n_accepted)
        assert np.allclose(f.probs, plain.probs, rtol=1e-12, atol=0, equal_nan=True)
        assert np.all(f.kept == V)


FILTER_GRID_CASES = [
    # (T, top_k, top_p, target row 0, draft row 0, bonus row; then the filtered laws p'0, q'0, p'1 by hand)
    (1.0, 0, 0.7, ["2/5", "1/5", "1/5", "1/10", "1/10", "0"], ["1/5", "0", "1/5", "2/5", "1/10", "1/10"],
     ["1/10", "1/10", "2/5", "1/5", "1/5", "0"],
     ["1/2", "1/4", "1/4", "0", "0", "0"], ["1/4", "0", "1/4", "1/2", "0", "0"], ["0", "0", "1/2", "1/4", "1/4", "0"]),
    (0.5, 2, 1.0, ["1/4", "1/8", "1/8", "1/4", "1/8", "1/8"], ["3/8", "3/8", "1/8", "1/16", "1/16", "0"],
     ["1/8", "1/8", "1/8", "1/8", "1/4", "1/4"],
     ["1/2", "0", "0", "1/2", "0", "0"], ["1/2", "1/2", "0", "0", "0", "0"], ["0", "0", "0", "0", "1/2", "1/2"]),
    (1.0, 3, 0.6, ["1/2", "1/8", "1/4", "1/16", "1/16", "0"], ["1/4", "1/4", "1/4", "1/8", "1/8", "0"],
     ["1/8", "1/8", "1/8", "1/8", "1/4", "1/4"],
     ["2/3", "0", "1/3", "0", "0", "0"], ["1/3", "1/3", "1/3", "0", "0", "0"],
     ["1/8", "1/8", "1/8", "1/8", "1/4", "1/4"]),
    (0.8, 0, 0.45, ["1/2", "1/4", "1/4", "0"], ["1/8", "1/8", "1/4", "1/2"], ["1/4", "1/4", "1/4", "1/4"],
     ["1", "0", "0", "0"], ["0", "0", "0", "1"], ["1/4", "1/4", "1/4", "1/4"]),
]


def check_filtered_exact_law(orc, grid: int = 48) -> None:
    """The theorem of §2.2 on the filtered laws: the emitted token has law p' exactly.

    As check_exact_law_on_grid, with K = 1 and a filter on every row; the draft
    token runs over q'0's support with weight q'0(x) (the draft samples its own
    filtered law). The filtered laws are worked out by hand from the unfiltered
    ones (comments in FILTER_GRID_CASES), not by the oracle: P(first = y) =
    p'0(y), P(accepted) = 1 - TV(p'0, q'0), P(accepted, bonus = y) = (1 - TV) p'1(y).
    Every boundary is a multiple of 1/48, so the mesh integral is exact.
    """
    mids = (np.arange(grid) + 0.5) / grid
    for T, k, p, t0s, d0s, t1s, e0s, eq0s, e1s in FILTER_GRID_CASES:
        pf0 = [Fraction(s) for s in e0s]
        qf0 = [Fraction(s) for s in eq0s]
        pf1 = [Fraction(s) for s in e1s]
        V = len(pf0)
        xs = [x for x in range(V) if qf0[x] > 0]
        rr, uu = np.meshgrid(mids, mids, indexing="ij")
        rr, uu = rr.ravel(), uu.ravel()
        cells = rr.size
        B = len(xs) * cells
        tgt = np.broadcast_to(np.stack([logits_from_probs(t0s, T), logits_from_probs(t1s, T)]), (B, 2, V))
        drf = np.broadcast_to(logits_from_probs(d0s, T), (B, 1, V))
        toks = np.repeat(np.array(xs, dtype=np.int32), cells)[:, None]
        uni = np.zeros((B, 2, 2), dtype=np.float64)
        uni[:, 0, 0] = np.tile(rr, len(xs))
        uni[:, 0, 1] = np.tile(uu, len(xs))
        uni[:, 1, 1] = 1.0 - np.tile(uu, len(xs))
        res = orc.oracle_sample_filtered(tgt, drf, toks, uni, T, np.full(B, k), np.full(B, p, dtype=np.float32),
                                         with_probs=False)
        first = [Fraction(0)] * V
        bonus = [Fraction(0)] * V
        accepted = Fraction(0)
        for j, x in enumerate(xs):
            sl = slice(j * cells, (j + 1) * cells)
            wgt = qf0[x] / cells
            t0 = res.tokens[sl, 0]
            n = res.n_accepted[sl]
            assert np.all(n >= 0)
            for y in range(V):
                first[y] += wgt * int(np.sum(t0 == y))
                bonus[y] += wgt * int(np.sum((n == 1) & (res.tokens[sl, 1] == y)))
            accepted += wgt * int(np.sum(n == 1))
        tv = sum(abs(a - b) for a, b in zip(pf0, qf0)) / 2
        assert first == pf0, ("filtered first-token law", T, k, p, first, pf0)
        assert accepted == 1 - tv, ("filtered acceptance", accepted, 1 - tv)
        assert bonus == [(1 - tv) * v for v in pf1], ("filtered bonus law", bonus)


# --------------------------------------------------------------------------- sampling verify of one-hot n-grams

def check_golden_ngram_sample(orc) -> None:
    for case in load("ngram_sample_worked.json")["cases"]:
        c = ngram_sample_case(case)
        res = orc.oracle_ngram_sample(c["logits"], c["cand"], c["uniforms"], c["T"])
        assert np.array_equal(res.tokens, c["expect_tokens"]), (c["name"], res.tokens, c["expect_tokens"])
        assert np.array_equal(res.accept_len, c["expect_len"]), (c["name"], res.accept_len)
        assert np.array_equal(res.rows, c["expect_rows"]), (c["name"], res.rows)


def check_ngram_sample_g1_matches_sample(orc) -> None:
    """One candidate drafted greedily is speculative decoding with a one-hot draft law
    ([SD] §2.1 with q = delta_x): the n-gram verify must give oracle_sample's outputs
    when the draft rows are one-hot at the candidate tokens and the uniforms map
    [b,i,0] -> r_i, [b,i,G] -> u_i."""
    rng = np.random.default_rng(77)
    for B, N, V, T, scale in ((300, 5, 40, 1.0, 1.5), (200, 3, 7, 0.7, 3.0), (100, 9, 300, 1.3, 2.0)):
        logits = rng.normal(0.0, scale, size=(B, 1, N, V))
        # candidate tokens: the target's argmax half the time (so walks go deep), else uniform
        amax = np.argmax(logits[:, 0, : N - 1], axis=-1)
        cand = np.where(rng.random((B, N - 1)) < 0.5, amax, rng.integers(0, V, size=(B, N - 1)))[:, None]
        cand = cand.astype(np.int32)
        uni = rng.random((B, N, 2))
        res = orc.oracle_ngram_sample(logits, cand, uni, T)
        draft = np.full((B, N - 1, V), -np.inf)
        for b in range(B):
            draft[b, np.arange(N - 1), cand[b, 0]] = 0.0
        su = np.zeros((B, N, 2))
        su[:, :, 0] = uni[:, :, 0]
        su[:, :, 1] = uni[:, :, 1]
        ref = orc.oracle_sample(logits[:, 0], draft, cand[:, 0], su, T, with_probs=False)
        assert np.array_equal(res.accept_len, ref.n_accepted), (B, N, V)
        assert np.array_equal(res.tokens, ref.tokens), (B, N, V)


# (p0, candidate tokens at position 0, bonus law of each candidate's row 1, mesh);
# every acceptance probability after renormalisation and every cumulative draw
# weight (as a fraction of the remaining mass) is a multiple of 1/mesh, so the mesh
# of uniforms integrates the walk exactly
NGRAM_LAW_DESIGNS = [
    (["1/2", "1/4", "1/8", "1/8"], [0, 1], [["1/2", "1/2", "0", "0"], ["0", "0", "1/2", "1/2"]], 8),
    (["1/2", "1/4", "1/8", "1/8"], [0, 1, 2], [["1/2", "1/2", "0", "0"], ["0", "0", "1/2", "1/2"],
                                              ["1/4", "1/4", "1/4", "1/4"]], 8),
    (["0", "1/2", "1/2", "0"], [1, 1, 2], [["1", "0", "0", "0"], ["0", "1", "0", "0"], ["0", "0", "1/4", "3/4"]], 8),
    (["1/2", "1/4", "1/4", "0"], [3, 0], [["1/4", "1/4", "1/2", "0"], ["0", "1/2", "0", "1/2"]], 8),
    (["1/2", "1/4", "1/8", "1/8"], [0, 0], [["1/2", "0", "1/2", "0"], ["0", "0", "0", "1"]], 8),
    # thirds: after 2 is rejected from the uniform law the rest holds 3/4 (draw weights 1/3, 2/3)
    (["1/4", "1/4", "1/4", "1/4"], [2, 2], [["1/2", "0", "1/2", "0"], ["0", "0", "0", "1"]], 12),
    (["1/4", "1/4", "1/4", "1/4"], [0, 1], [["1/4", "1/4", "1/4", "1/4"], ["1/2", "1/2", "0", "0"]], 12),
]


def check_ngram_sample_exact_law(orc, designs=NGRAM_LAW_DESIGNS) -> None:
    """The sampling verify of one-hot candidates keeps the target's law ([LA] "采样模式的验证";
    the one-candidate case is [SD] §2.2's theorem with q = delta_x). N = 2: the G
    accept uniforms and the draw uniform run over the midpoints of a 1/grid mesh
    (the bonus uniform is 1 - u). Exactly in rationals:
      P(first token = y) = p0(y);
      P(first token x accepted, bonus y) = P(x accepted) * p1[g(x)](y), g(x) the lowest
      candidate proposing x (its row is the one the bonus reads).
    """
    from itertools import product
    for p0s, toks, p1s, grid in designs:
        mids = (np.arange(grid) + 0.5) / grid
        G = len(toks)
        V = len(p0s)
        p0 = [Fraction(x) for x in p0s]
        p1 = [[Fraction(x) for x in r] for r in p1s]
        cells = np.array(list(product(range(grid), repeat=G + 1)))
        Bn = len(cells)
        logits = np.zeros((Bn, G, 2, V))
        for g in range(G):
            logits[:, g, 0] = logits_from_probs(p0s, 1.0)
            logits[:, g, 1] = logits_from_probs(p1s[g], 1.0)
        cand = np.broadcast_to(np.array(toks, dtype=np.int32)[None, :, None], (Bn, G, 1)).copy()
        uni = np.zeros((Bn, 2, G + 1))
        uni[:, 0, :G] = mids[cells[:, :G]]
        uni[:, 0, G] = mids[cells[:, G]]
        uni[:, 1, G] = 1.0 - mids[cells[:, G]]
        res = orc.oracle_ngram_sample(logits, cand, uni, 1.0)
        assert np.all(res.accept_len >= 0)
        w = Fraction(1, Bn)
        first = [w * int(np.sum(res.tokens[:, 0] == y)) for y in range(V)]
        assert first == p0, ("first-token law", toks, first, p0)
        for x in set(toks):
            acc = res.accept_len == 1
            px = w * int(np.sum(acc & (res.tokens[:, 0] == x)))
            gx = toks.index(x)
            for y in range(V):
                got = w * int(np.sum(acc & (res.tokens[:, 0] == x) & (res.tokens[:, 1] == y)))
                assert got == px * p1[gx][y], ("bonus law", toks, x, y, got, px * p1[gx][y])
