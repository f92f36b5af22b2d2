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
returned so that the parity tests can exclude the ambiguous cases; draw
margins are measured in probability mass, on the unnormalised cumulative
weights that u * Z is compared with.
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
    Z = sum w; margin = distance of u Z from the nearer boundary of k's interval.
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
    margin = min(abs(tau - lo), abs(float(c[k]) - tau))
    return k, Z, margin


@dataclass
class SampleResult:
    tokens: np.ndarray          # [B, K+1] int32; first n+1 valid, rest -1
    n_accepted: np.ndarray      # [B] int32; -1 marks a data fault
    probs: np.ndarray           # [B, K, 2] float64: p_i(x_i), q_i(x_i) (nan where undefined)
    accept_margin: np.ndarray   # [B, K] |r_i - alpha_i| for evaluated tests, +inf otherwise
    draw_margin: np.ndarray     # [B] margin of the resample / bonus draw (+inf on a fault)
    residual_mass: np.ndarray   # [B] Z of the draw (1 for a bonus draw; nan on a fault)
    fallback: np.ndarray        # [B] bool: residual mass was zero and p was sampled instead

    def min_margin(self) -> np.ndarray:
        """Per row, the smallest margin over every decision the row took."""
        return np.minimum(self.accept_margin.min(axis=1, initial=np.inf), self.draw_margin)


def token_probs(target_row: np.ndarray, draft_row: np.ndarray, x: int, temperature: float) -> tuple[float, float]:
    """(p(x), q(x)) for one position; nan when a row is invalid or x is out of range."""
    V = target_row.shape[-1]
    if not (0 <= x < V) or not row_is_valid(target_row) or not row_is_valid(draft_row):
        return float("nan"), float("nan")
    return float(softmax64(target_row, temperature)[x]), float(softmax64(draft_row, temperature)[x])


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
