"""CPU oracle of the speculative-decoding verify step: plain, slow, float64.

TEST INFRASTRUCTURE. Only the tests, the package's smoke check and the bench's
CPU-baseline leg may import or run this module. The product path never does:
it shares no code with the HIP library, and the library does not import it.

Sources (page title, section):
  [SD]  Speculative Decoding —— LLM推理优化技术（一） (hustzhy.cn):
        §2.1 acceptance probability min(1, p/q) and the residual law
        norm(max(0, p - q)); §2.2 proof that the output law is p; §2.3 the
        multi-token rule (stop at the first rejection, bonus token when all K
        are accepted); §2.4 E[accept] = 1 - TV(p, q); §3.1 tokens per round;
        §4 code: temperature divides the logits, a fresh uniform per accept
        test, fall back to p when the residual mass is zero.
  [KW]  kwkr.cn/news/620797 engineering notes: §3.1 the verify steps in order
        (accept iff r < alpha, reject iff r >= alpha, residual re-normalised,
        bonus from the target's last row); §3.2 truncate alpha to 1 when
        p >= q without dividing; probabilities in fp32 at least; §3.4 the same
        temperature on both sides.
  [SS]  EMNLP'23 | ... Self-Speculative Decoding 原理详解: §2.2 alpha_t and the
        resample law, stated a second time.
  [LA]  Lookahead Decoding 完全拆解:Jacobi 迭代与 N-gram 池 ...: eq. (1)
        greedy decoding is an argmax per position; section
        "验证分支:输出分布不变性": under greedy decoding a candidate's i-th
        token must equal the argmax at position i, the longest matched prefix
        among the candidates wins, and one extra token follows it.

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * no epsilon in p/q or in the residual normalisation (the pages' code adds
    1e-10; the method's definition has none);
  * alpha = 0 when p(x) = 0; otherwise alpha = 1 when p(x) >= q(x) (this
    covers q(x) = 0), else p(x)/q(x);
  * inverse-CDF draw: the smallest k with C_k > u * Z, C_k the running sum of
    the unnormalised weights w; if rounding leaves no such k, the last index
    with w > 0;
  * residual mass Z == 0 falls back to sampling p (as [SD] §4's code does);
  * the temperature is the float32 value the caller passes, widened to float64;
  * a data fault (draft token outside [0, V), or a consulted logit row with no
    finite entry) gives n_accepted = -1 and all output tokens -1; a row is
    consulted when the walk over positions reaches it (target and draft rows
    0..n, and the bonus row when n = K);
  * greedy ties: the lowest vocabulary index attains the argmax; among
    candidates with the longest prefix, the lowest candidate index wins.
Margins (distance of a uniform from the boundary that decided it) are
returned so that the parity tests can exclude the ambiguous cases. Both are
distances on the unit interval the uniform lives on: |r - alpha| for an
accept test, and for a draw the distance of u from the ends of the chosen
token's interval of the normalised CDF C_k / Z (the residual law is
norm(max(0, p - q)), [SD] §2.1, so its CDF boundaries are the C_k / Z).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def temperature64(temperature: float) -> float:
    """The temperature the verify step uses: the float32 value, widened to float64."""
    return float(np.float32(temperature))


def softmax64(logits: np.ndarray, temperature: float) -> np.ndarray:
    """p = softmax(logits / T) in float64, computed as exp(z - max z) / sum ([SD] §4, [KW] §3.4).

    Entries equal to -inf get probability 0. The row must hold a finite entry.
    """
    z = np.asarray(logits, dtype=np.float64) / temperature64(temperature)
    m = np.max(z)
    if not np.isfinite(m):
        raise ValueError("softmax64: row has no finite logit")
    e = np.exp(z - m)
    return e / np.sum(e)


def row_is_valid(logits: np.ndarray) -> bool:
    """A consulted logit row must hold at least one finite entry."""
    return bool(np.any(np.isfinite(np.asarray(logits, dtype=np.float64))))


def acceptance_probability(p_x: float, q_x: float) -> float:
    """alpha = min(1, p(x)/q(x)) ([SD] §2.1, [SS] §2.2), truncated to 1 without dividing when p >= q ([KW] §3.2)."""
    if p_x == 0.0:
        return 0.0
    if p_x >= q_x:
        return 1.0
    return p_x / q_x


def inverse_cdf_draw(w: np.ndarray, u: float) -> tuple[int, float, float]:
    """Draw from the weights w (not necessarily normalised) with the uniform u.

    Returns (k, Z, margin): k = min{k : C_k > u Z} with C_k = sum_{v <= k} w_v and
    Z = sum w; margin = distance of u from the nearer end of k's interval
    [C_{k-1} / Z, C_k / Z) of the normalised CDF.
    """
    c = np.cumsum(np.asarray(w, dtype=np.float64))
    Z = float(c[-1])
    tau = float(u) * Z
    hits = np.nonzero(c > tau)[0]
    if hits.size:
        k = int(hits[0])
    else:
        k = int(np.nonzero(np.asarray(w) > 0)[0][-1])
    lo = float(c[k - 1]) if k > 0 else 0.0
    margin = min(abs(tau - lo), abs(float(c[k]) - tau)) / Z
    return k, Z, margin


@dataclass
class SampleResult:
    tokens: np.ndarray          # [B, K+1] int32; first n+1 valid, rest -1
    n_accepted: np.ndarray      # [B] int32; -1 marks a data fault
    probs: np.ndarray           # [B, K, 2] float64: p_i(x_i), q_i(x_i) (nan where undefined, each by its own row)
    accept_margin: np.ndarray   # [B, K] |r_i - alpha_i| for evaluated tests, +inf otherwise
    draw_margin: np.ndarray     # [B] margin of the resample / bonus draw (+inf on a fault)
    residual_mass: np.ndarray   # [B] Z of the draw (1 for a bonus draw; nan on a fault)
    fallback: np.ndarray        # [B] bool: residual mass was zero and p was sampled instead

    def min_margin(self) -> np.ndarray:
        """Per row, the smallest margin over every decision the row took."""
        return np.minimum(self.accept_margin.min(axis=1, initial=np.inf), self.draw_margin)


def token_probs(target_row: np.ndarray, draft_row: np.ndarray, x: int, temperature: float) -> tuple[float, float]:
    """(p(x), q(x)) for one position; each is nan when x is out of range or its own row has no finite logit."""
    V = target_row.shape[-1]
    if not (0 <= x < V):
        return float("nan"), float("nan")
    p = float(softmax64(target_row, temperature)[x]) if row_is_valid(target_row) else float("nan")
    q = float(softmax64(draft_row, temperature)[x]) if row_is_valid(draft_row) else float("nan")
    return p, q


def oracle_sample(target: np.ndarray, draft: np.ndarray, draft_tokens: np.ndarray,
                  uniforms: np.ndarray, temperature: float, *, with_probs: bool = True) -> SampleResult:
    """Rejection-sampling verify of B independent rows ([SD] §2.1-2.3, [KW] §3.1).

    target [B, K+1, V] and draft [B, K, V] are logit values (any float dtype; bf16
    inputs must be widened by the caller); target row i is the distribution for
    draft token i and row K is the bonus row. draft_tokens [B, K]; uniforms
    [B, K+1, 2] with [b,i,0] the accept uniform r_i and [b,i,1] the draw uniform u_i.
    """
    target = np.asarray(target)
    draft = np.asarray(draft)
    B, K, V = draft.shape
    assert target.shape == (B, K + 1, V), "target must be [B, K+1, V]"
    assert draft_tokens.shape == (B, K) and uniforms.shape == (B, K + 1, 2)
    tokens = np.full((B, K + 1), -1, dtype=np.int32)
    n_acc = np.zeros(B, dtype=np.int32)
    probs = np.full((B, K, 2), np.nan)
    acc_margin = np.full((B, K), np.inf)
    draw_margin = np.full(B, np.inf)
    zmass = np.full(B, np.nan)
    fallback = np.zeros(B, dtype=bool)

    for b in range(B):
        if with_probs:
            for i in range(K):
                probs[b, i] = token_probs(target[b, i], draft[b, i], int(draft_tokens[b, i]), temperature)
        fault = False
        n = K
        p_rej = q_rej = None
        for i in range(K):
            x = int(draft_tokens[b, i])
            if not (0 <= x < V) or not row_is_valid(target[b, i]) or not row_is_valid(draft[b, i]):
                fault = True
                break
            p = softmax64(target[b, i], temperature)
            q = softmax64(draft[b, i], temperature)
            alpha = acceptance_probability(float(p[x]), float(q[x]))
            r = float(uniforms[b, i, 0])
            acc_margin[b, i] = abs(r - alpha)
            if r < alpha:                      # accept iff r < alpha ([KW] §3.1)
                continue
            n = i                              # first rejection: stop here ([SD] §2.3)
            p_rej, q_rej = p, q
            break
        if not fault and n == K and not row_is_valid(target[b, K]):
            fault = True
        if fault:
            n_acc[b] = -1
            acc_margin[b] = np.inf
            continue
        if n < K:
            w = np.maximum(0.0, p_rej - q_rej)          # residual law ([SD] §2.1)
            if np.sum(w) == 0.0:                        # zero residual mass: sample p ([SD] §4 code)
                w = p_rej
                fallback[b] = True
        else:
            w = softmax64(target[b, K], temperature)    # bonus draw from the last row ([SD] §2.3 step 4)
        k, Z, margin = inverse_cdf_draw(w, float(uniforms[b, n, 1]))
        tokens[b, :n] = draft_tokens[b, :n]
        tokens[b, n] = k
        n_acc[b] = n
        draw_margin[b] = margin
        zmass[b] = Z
    return SampleResult(tokens, n_acc, probs, acc_margin, draw_margin, zmass, fallback)


@dataclass
class GreedyResult:
    tokens: np.ndarray       # [B, N]: matched prefix, then the argmax after it, rest -1
    accept_len: np.ndarray   # [B]: L in [0, N-1]; -1 marks a data fault
    best: np.ndarray         # [B]: winning candidate (lowest index among the longest); -1 on a fault
    argmax: np.ndarray       # [B, G, N]: per-row argmax (lowest index on ties); -1 for a row with no finite entry


def first_argmax(row: np.ndarray) -> int:
    """Lowest index attaining the maximum of the row, values compared exactly ([LA] eq. (1))."""
    return int(np.argmax(np.asarray(row, dtype=np.float64)))


def oracle_greedy(logits: np.ndarray, cand: np.ndarray) -> GreedyResult:
    """Greedy longest-prefix verify over G disjoint candidates ([LA] "验证分支:输出分布不变性").

    logits [B, G, N, V] (row i of candidate g predicts cand[b,g,i]; row N-1 is the
    bonus row); cand [B, G, N-1]. No temperature: greedy decoding is the argmax.
    """
    logits = np.asarray(logits)
    B, G, N, V = logits.shape
    assert cand.shape == (B, G, N - 1)
    tokens = np.full((B, N), -1, dtype=np.int32)
    acc_len = np.full(B, -1, dtype=np.int32)
    best_out = np.full(B, -1, dtype=np.int32)
    amax = np.full((B, G, N), -1, dtype=np.int32)
    for b in range(B):
        fault = bool(np.any((cand[b] < 0) | (cand[b] >= V)))
        for g in range(G):
            for i in range(N):
                if row_is_valid(logits[b, g, i]):
                    amax[b, g, i] = first_argmax(logits[b, g, i])
                else:
                    fault = True
        if fault:
            continue
        L = np.zeros(G, dtype=np.int64)
        for g in range(G):
            while L[g] < N - 1 and cand[b, g, L[g]] == amax[b, g, L[g]]:
                L[g] += 1
        best = int(np.argmax(L))          # lowest g among the longest prefixes
        Lb = int(L[best])
        tokens[b, :Lb] = cand[b, best, :Lb]
        tokens[b, Lb] = amax[b, best, Lb]  # the extra token after the matched prefix
        acc_len[b] = Lb
        best_out[b] = best
    return GreedyResult(tokens, acc_len, best_out, amax)


# --------------------------------------------------------------------------- sampling verify of greedy-drafted n-grams
#
# [LA] "采样模式的验证": the lookahead branch drafts its n-grams greedily, so each
# candidate token comes from a one-hot law q = delta_x and only the token id is
# kept; the verify side still runs a full sampling verification (the paper's
# Algorithm 4, not printed on the page). Reading: the rule of [SD] §2.1 with
# q = delta_x accepts x with probability min(1, p(x)/1) = p(x), and on rejection
# the residual norm(max(0, p - delta_x)) is p with x removed, renormalised. With
# G disjoint candidates ([LA] "验证分支"), at each position the candidates whose
# prefix matches the tokens accepted so far ("active") are tried in index order,
# each rejection removing its token from the current law:
#   * the law of position i is the target row i of the lowest-index active
#     candidate (every active candidate has the same prefix);
#   * candidate h's token x is accepted iff r < p_cur(x), r = uniforms[b, i, h],
#     p_cur = p with the tokens rejected so far at this position removed,
#     renormalised (a token already rejected has p_cur(x) = 0);
#   * on acceptance, the candidates whose token at i is x stay active and the walk
#     moves to position i + 1; after N-1 accepted tokens a bonus token is drawn
#     from row N-1 of the lowest-index active candidate with uniforms[b, N-1, G];
#   * when every active candidate is rejected, the token is drawn from p_cur with
#     uniforms[b, i, G] by the inverse-CDF rule of oracle_sample (zero remaining
#     mass falls back to p), and the walk stops.
# A candidate token outside [0, V), or a consulted row with no finite logit, is a
# data fault of the batch row.

@dataclass
class NgramSampleResult:
    tokens: np.ndarray         # [B, N]: accepted tokens, then the drawn one, rest -1
    accept_len: np.ndarray     # [B]: L in [0, N-1]; -1 marks a data fault
    rows: np.ndarray           # [B]: candidate whose rows the final draw used; -1 on a fault
    accept_margin: np.ndarray  # [B]: smallest |r - p_cur(x)| over the tries taken (+inf if none)
    draw_margin: np.ndarray    # [B]: margin of the draw (+inf on a fault)
    residual_mass: np.ndarray  # [B]: mass the draw's weights carry (1 for the bonus; nan on a fault)

    def min_margin(self) -> np.ndarray:
        return np.minimum(self.accept_margin, self.draw_margin)


def oracle_ngram_sample(logits: np.ndarray, cand: np.ndarray, uniforms: np.ndarray,
                        temperature: float) -> NgramSampleResult:
    """Sampling verify of G greedy-drafted candidate n-grams ([LA] "采样模式的验证", [SD] §2.1).

    logits [B, G, N, V]: row i of candidate g is the target's law after the
    candidate's first i tokens (row N-1 the bonus row); cand [B, G, N-1];
    uniforms [B, N, G+1]: [b, i, h] accepts candidate h at position i, [b, i, G]
    is the draw uniform of position i.
    """
    logits = np.asarray(logits)
    B, G, N, V = logits.shape
    assert cand.shape == (B, G, N - 1) and uniforms.shape == (B, N, G + 1)
    tokens = np.full((B, N), -1, dtype=np.int32)
    acc_len = np.full(B, -1, dtype=np.int32)
    rows_out = np.full(B, -1, dtype=np.int32)
    acc_margin = np.full(B, np.inf)
    draw_margin = np.full(B, np.inf)
    zmass = np.full(B, np.nan)
    for b in range(B):
        if np.any((cand[b] < 0) | (cand[b] >= V)):
            continue
        active = list(range(G))
        prefix: list[int] = []
        margin = np.inf
        fault = False
        while True:
            g0 = active[0]
            i = len(prefix)
            if not row_is_valid(logits[b, g0, i]):
                fault = True
                break
            p = softmax64(logits[b, g0, i], temperature)
            if i == N - 1:                                  # every candidate token accepted: bonus draw
                w = p
                break
            live = p.copy()                                 # p_cur, unnormalised
            accepted = None
            for h in active:
                x = int(cand[b, h, i])
                left = float(np.sum(live))
                alpha = float(live[x]) / left if left > 0.0 else 0.0   # p_cur(x) / q(x), q = delta_x
                r = float(uniforms[b, i, h])
                margin = min(margin, abs(r - alpha))
                if r < alpha:                               # accept iff r < alpha ([KW] §3.1)
                    accepted = x
                    break
                live[x] = 0.0                               # residual: max(0, p_cur - delta_x)
            if accepted is None:
                w = live if np.sum(live) > 0.0 else p       # zero remaining mass: sample p
                break
            prefix.append(accepted)
            active = [h for h in active if int(cand[b, h, i]) == accepted]
        if fault:
            continue
        k, Z, dmargin = inverse_cdf_draw(w, float(uniforms[b, len(prefix), G]))
        L = len(prefix)
        tokens[b, :L] = prefix
        tokens[b, L] = k
        acc_len[b] = L
        rows_out[b] = active[0]
        acc_margin[b] = margin
        draw_margin[b] = dmargin
        zmass[b] = Z
    return NgramSampleResult(tokens, acc_len, rows_out, acc_margin, draw_margin, zmass)


# --------------------------------------------------------------------------- top-k / top-p consistent verify
#
# [KW] §3.4: the temperature rescales both sides before p and q are formed; a
# top-p (or top-k) truncation must use the same threshold on the draft and the
# target side, and the correction is drawn only inside the truncated set.
# Readings where the notes are silent (listed with their reasons in the design
# notes of the repository):
#   * top-k then top-p, each on the row's tempered law, top-p on the law left
#     by top-k and renormalised (the order of the usual sampling pipeline);
#   * top-k (0 < k < V) keeps every entry with fewer than k entries strictly
#     above it, so all ties of the k-th largest logit stay; k <= 0 or k >= V
#     turns it off;
#   * top-p (p < 1) keeps an entry when the mass of kept entries with a strictly
#     larger logit is below p, and always keeps the entries of the row's largest
#     logit (so p <= 0 keeps only those); p >= 1 or NaN turns it off; p is the
#     float32 value the caller passes;
#   * p', q' are the kept probabilities renormalised; the verify then runs on
#     p', q' unchanged (a draft token outside the draft's kept set has q' = 0, so
#     alpha = 1 when p' > 0);
#   * a row with no finite logit keeps nothing.

def top_p64(top_p: float) -> float:
    """The top-p the verify step uses: the float32 value, widened to float64."""
    return float(np.float32(top_p))


@dataclass
class KeepResult:
    keep: np.ndarray   # [V] bool: the entries the row keeps
    margin: float      # |p - mass| of the top-p decisions at the cut, in the top-k law's probability; +inf if no top-p cut


def filter_keep(logits: np.ndarray, temperature: float, top_k: int, top_p: float) -> KeepResult:
    """Entries a logit row keeps under top-k, then top-p on the renormalised top-k law ([KW] §3.4)."""
    x = np.asarray(logits, dtype=np.float64)
    V = x.shape[-1]
    if not np.any(np.isfinite(x)):
        return KeepResult(np.zeros(V, dtype=bool), np.inf)
    keep = np.ones(V, dtype=bool)
    k = int(top_k)
    if 0 < k < V:
        kth = np.sort(x)[V - k]            # the k-th largest logit, counting repeats
        keep = x >= kth
    p = top_p64(top_p)
    margin = np.inf
    if p < 1.0:                            # False for NaN: no top-p
        z = x / temperature64(temperature)
        e = np.where(keep, np.exp(z - np.max(z)), 0.0)
        Z = float(np.sum(e))
        order = np.argsort(-x, kind="stable")
        xs, es = x[order], e[order]
        csum = np.cumsum(es)
        # first position of each entry's group of equal logits in the descending order
        start = np.searchsorted(-xs, -xs, side="left")
        above = np.where(start > 0, csum[np.maximum(start - 1, 0)], 0.0)   # mass strictly above
        top = xs == xs[0]
        kept_s = keep[order] & (top | (above < p * Z))
        J = int(np.sum(kept_s))            # the kept entries form a prefix of the order
        m_in = np.inf if top[J - 1] else p * Z - above[J - 1]
        m_out = np.inf
        if J < V and keep[order][J]:       # the first entry dropped by top-p rather than by top-k
            m_out = above[J] - p * Z
        margin = min(m_in, m_out) / Z
        keep = np.zeros(V, dtype=bool)
        keep[order] = kept_s
    return KeepResult(keep, margin)


def filtered_softmax64(logits: np.ndarray, temperature: float, keep: np.ndarray) -> np.ndarray:
    """softmax(logits / T) restricted to `keep` and renormalised over it."""
    z = np.asarray(logits, dtype=np.float64) / temperature64(temperature)
    e = np.where(keep, np.exp(z - np.max(z)), 0.0)
    return e / np.sum(e)


@dataclass
class FilteredResult(SampleResult):
    kept: np.ndarray = None           # [B, 2K+1] kept entries: target rows 0..K, then draft rows 0..K-1
    filter_margin: np.ndarray = None  # [B, 2K+1] top-p margin of each row (+inf without a top-p cut)
    consulted: np.ndarray = None      # [B, 2K+1] bool: the walk read this row's law

    def min_margin(self) -> np.ndarray:
        fm = np.where(self.consulted, self.filter_margin, np.inf).min(axis=1, initial=np.inf)
        return np.minimum(SampleResult.min_margin(self), fm)


def oracle_sample_filtered(target: np.ndarray, draft: np.ndarray, draft_tokens: np.ndarray, uniforms: np.ndarray,
                           temperature: float, top_k: np.ndarray, top_p: np.ndarray, *,
                           with_probs: bool = True) -> FilteredResult:
    """Rejection-sampling verify on top-k / top-p filtered laws p', q' ([KW] §3.4, [SD] §2.1-2.3).

    Shapes as in oracle_sample; top_k [B] int and top_p [B] float hold the
    filter of each batch row, applied alike to its target and draft rows.
    """
    target = np.asarray(target)
    draft = np.asarray(draft)
    B, K, V = draft.shape
    assert target.shape == (B, K + 1, V) and draft_tokens.shape == (B, K) and uniforms.shape == (B, K + 1, 2)
    top_k = np.asarray(top_k).reshape(B)
    top_p = np.asarray(top_p).reshape(B)
    tokens = np.full((B, K + 1), -1, dtype=np.int32)
    n_acc = np.zeros(B, dtype=np.int32)
    probs = np.full((B, K, 2), np.nan)
    acc_margin = np.full((B, K), np.inf)
    draw_margin = np.full(B, np.inf)
    zmass = np.full(B, np.nan)
    fallback = np.zeros(B, dtype=bool)
    kept = np.zeros((B, 2 * K + 1), dtype=np.int64)
    fmargin = np.full((B, 2 * K + 1), np.inf)
    consulted = np.zeros((B, 2 * K + 1), dtype=bool)

    for b in range(B):
        rows = [target[b, i] for i in range(K + 1)] + [draft[b, i] for i in range(K)]
        keeps = [filter_keep(r, temperature, int(top_k[b]), float(top_p[b])) for r in rows]
        for j, kr in enumerate(keeps):
            kept[b, j] = int(np.sum(kr.keep))
            fmargin[b, j] = kr.margin

        def law(j):
            return filtered_softmax64(rows[j], temperature, keeps[j].keep)

        if with_probs:
            for i in range(K):
                x = int(draft_tokens[b, i])
                if 0 <= x < V:
                    for side, j in ((0, i), (1, K + 1 + i)):
                        if row_is_valid(rows[j]):
                            probs[b, i, side] = float(law(j)[x])
        fault = False
        n = K
        p_rej = q_rej = None
        for i in range(K):
            x = int(draft_tokens[b, i])
            if not (0 <= x < V) or not row_is_valid(rows[i]) or not row_is_valid(rows[K + 1 + i]):
                fault = True
                break
            consulted[b, i] = consulted[b, K + 1 + i] = True
            p = law(i)
            q = law(K + 1 + i)
            alpha = acceptance_probability(float(p[x]), float(q[x]))
            r = float(uniforms[b, i, 0])
            acc_margin[b, i] = abs(r - alpha)
            if r < alpha:
                continue
            n = i
            p_rej, q_rej = p, q
            break
        if not fault and n == K and not row_is_valid(rows[K]):
            fault = True
        if fault:
            n_acc[b] = -1
            acc_margin[b] = np.inf
            consulted[b] = False
            continue
        if n < K:
            w = np.maximum(0.0, p_rej - q_rej)   # residual of the filtered laws: inside p's kept set
            if np.sum(w) == 0.0:
                w = p_rej
                fallback[b] = True
        else:
            consulted[b, K] = True
            w = law(K)                           # bonus from the filtered last row
        k, Z, margin = inverse_cdf_draw(w, float(uniforms[b, n, 1]))
        tokens[b, :n] = draft_tokens[b, :n]
        tokens[b, n] = k
        n_acc[b] = n
        draw_margin[b] = margin
        zmass[b] = Z
    return FilteredResult(tokens, n_acc, probs, acc_margin, draw_margin, zmass, fallback,
                          kept=kept, filter_margin=fmargin, consulted=consulted)
