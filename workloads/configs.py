"""Seeded synthetic inputs shaped like the workloads of the speculative-decoding pages.

This module only builds inputs: logits, draft tokens and uniforms. It holds no
step of the verify method itself (no softmax, ratio, residual, CDF search or
argmax over a verified row). Both the CPU oracle and the HIP path receive the
same arrays from here.

Five workloads (sizes from the task's configuration list; value laws chosen to
match the pages' acceptance ranges: 0.6-0.8 for a same-family draft in
Speculative Decoding -- LLM推理优化技术（一） §2.4, >70% vs ~40% in the kwkr.cn
notes §2, greedy n-gram candidates in Lookahead Decoding 完全拆解, section
"验证分支:输出分布不变性"):

  1  B=1,   K=4, V=32000,  fp32, T=1.0  target N(0,2^2); draft = target + N(0,0.5^2)
  2  B=8,   K=5, V=32000,  bf16, T=0.7  Zipf-like: per (b,i) a random permutation pi,
                                        logit[pi(r)] = -1.1 ln r + N(0,0.3^2); draft = target + N(0,1)
  3  B=64,  K=8, V=128256, bf16, T=1.0  target N(0,3^2); sigma_b ~ U[0.2,2.0] per batch row;
                                        draft = target + N(0,sigma_b^2)
  4  B=256, K=4, V=152064, fp32, T=0.8  rows b < B/2 peaked: N(0,1) + 12 on one token t*;
                                        rows b >= B/2 flat: N(0,0.5^2); draft = target + N(0,0.8^2);
                                        in 10% of peaked positions the draft logits of t* and of a
                                        uniformly chosen other token are swapped (draft top-1 != target top-1)
  5  greedy B=32, G=7, N=5, V=32000, bf16 logits [B,G,N,V] i.i.d. N(0,2^2);
                                        cand[b,g,i] = the row's maximiser w.p. 0.6, else uniform on [0,V)

Draft tokens are drawn from q = softmax(draft/T), evaluated on the stored
(bf16-rounded where applicable) draft values, with the Gumbel-max construction
(x = the index maximising draft/T + Gumbel noise): drawing drafts is the draft
model's job, outside the verify step, and this way the generator shares no
arithmetic with the verify path's softmax or inverse-CDF draw.

Greedy rows place the row maximum by construction: the maximum of V i.i.d.
N(0,s^2) values is drawn from its own law (P(max <= m) = Phi(m/s)^V), the other
V-1 values from N(0,s^2) truncated below it, and the maximum is put at a
uniformly chosen position. That is the same joint law as V i.i.d. draws, and the
maximiser is known without searching the row. After bf16 rounding another value
can tie with the maximum (a few % of rows at V=32000), which exercises the
lowest-index tie rule.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
from scipy.special import ndtri

from .bf16 import bf16_bits_to_f32, f32_to_bf16_bits
from .philox import ngram_uniforms, verify_uniforms

F32 = "f32"
BF16 = "bf16"


@dataclass
class SampleInputs:
    """Inputs of one sampling verify round.

    target: [B, K+1, V] float32 values, or uint16 bf16 bit patterns when dtype == "bf16"
    draft:  [B, K, V]   same storage as target
    draft_tokens: [B, K] int32; uniforms: [B, K+1, 2] float32; temperature: float
    """
    target: np.ndarray
    draft: np.ndarray
    dtype: str
    draft_tokens: np.ndarray
    uniforms: np.ndarray
    temperature: float
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def shape(self) -> tuple[int, int, int]:
        B, K, V = self.draft.shape
        return B, K, V

    def target_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.target) if self.dtype == BF16 else self.target

    def draft_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.draft) if self.dtype == BF16 else self.draft


@dataclass
class GreedyInputs:
    """Inputs of one greedy verify round: logits [B, G, N, V] (bf16 bits or float32), cand [B, G, N-1]."""
    logits: np.ndarray
    dtype: str
    cand: np.ndarray
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def shape(self) -> tuple[int, int, int, int]:
        return self.logits.shape  # type: ignore[return-value]

    def logits_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.logits) if self.dtype == BF16 else self.logits


SAMPLE_CONFIGS = {
    1: dict(B=1, K=4, V=32000, dtype=F32, T=1.0),
    2: dict(B=8, K=5, V=32000, dtype=BF16, T=0.7),
    3: dict(B=64, K=8, V=128256, dtype=BF16, T=1.0),
    4: dict(B=256, K=4, V=152064, dtype=F32, T=0.8),
}
GREEDY_CONFIGS = {5: dict(B=32, G=7, N=5, V=32000, dtype=BF16)}
WORKLOAD_NAMES = {
    1: "B=1 K=4 V=32000 fp32 T=1.0, normal logits",
    2: "B=8 K=5 V=32000 bf16 T=0.7, Zipf logits",
    3: "B=64 K=8 V=128256 bf16 T=1.0, normal logits, per-row draft noise",
    4: "B=256 K=4 V=152064 fp32 T=0.8, half peaked / half flat",
    5: "greedy B=32 G=7 N=5 V=32000 bf16, i.i.d. normal logits",
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == BF16 else x


def _gumbel_draft_tokens(draft_vals: np.ndarray, T: float, rng: np.random.Generator) -> np.ndarray:
    """Draw x[b,i] ~ softmax(draft[b,i]/T) with the Gumbel-max construction (float64)."""
    B, K, V = draft_vals.shape
    out = np.empty((B, K), dtype=np.int32)
    Tf = float(np.float32(T))
    for b in range(B):
        g = -np.log(-np.log(rng.random((K, V))))
        score = draft_vals[b].astype(np.float64) / Tf + g
        out[b] = np.argmax(score, axis=1)
    return out


def _logits_cfg1(rng, B, K, V):
    tgt = rng.standard_normal((B, K + 1, V), dtype=np.float32) * np.float32(2.0)
    drf = tgt[:, :K] + rng.standard_normal((B, K, V), dtype=np.float32) * np.float32(0.5)
    return tgt, drf, {}


def _logits_cfg2(rng, B, K, V):
    ranks = np.arange(1, V + 1, dtype=np.float64)
    base = (-1.1 * np.log(ranks)).astype(np.float32)
    tgt = np.empty((B, K + 1, V), dtype=np.float32)
    for b in range(B):
        for i in range(K + 1):
            perm = rng.permutation(V)
            row = base + rng.standard_normal(V, dtype=np.float32) * np.float32(0.3)
            tgt[b, i, perm] = row
    drf = tgt[:, :K] + rng.standard_normal((B, K, V), dtype=np.float32)
    return tgt, drf, {}


def _logits_cfg3(rng, B, K, V):
    sigma = rng.uniform(0.2, 2.0, size=B).astype(np.float32)
    tgt = rng.standard_normal((B, K + 1, V), dtype=np.float32) * np.float32(3.0)
    drf = np.empty((B, K, V), dtype=np.float32)
    for b in range(B):
        drf[b] = tgt[b, :K] + rng.standard_normal((K, V), dtype=np.float32) * sigma[b]
    return tgt, drf, {"draft_sigma": sigma}


def _logits_cfg4(rng, B, K, V):
    half = B // 2
    tgt = np.empty((B, K + 1, V), dtype=np.float32)
    peak_tok = rng.integers(0, V, size=(B, K + 1))
    for b in range(B):
        if b < half:
            tgt[b] = rng.standard_normal((K + 1, V), dtype=np.float32)
            tgt[b, np.arange(K + 1), peak_tok[b]] += np.float32(12.0)
        else:
            tgt[b] = rng.standard_normal((K + 1, V), dtype=np.float32) * np.float32(0.5)
    drf = tgt[:, :K] + rng.standard_normal((B, K, V), dtype=np.float32) * np.float32(0.8)
    forced = np.zeros((B, K), dtype=bool)
    for b in range(half):
        for i in range(K):
            if rng.random() < 0.1:
                t = peak_tok[b, i]
                j = (t + 1 + rng.integers(0, V - 1)) % V  # uniform over the other V-1 tokens
                drf[b, i, t], drf[b, i, j] = drf[b, i, j], drf[b, i, t]
                forced[b, i] = True
    return tgt, drf, {"peak_token": peak_tok, "forced_disagree": forced}


_SAMPLE_LAWS = {1: _logits_cfg1, 2: _logits_cfg2, 3: _logits_cfg3, 4: _logits_cfg4}


def make_sample_inputs(cfg: int, rnd: int = 0, *, B: int | None = None, K: int | None = None,
                       V: int | None = None, seed: int = 0, dtype: str | None = None,
                       temperature: float | None = None) -> SampleInputs:
    """Inputs of verify round `rnd` of sampling workload `cfg` (1-4), optionally resized.

    Resizing keeps the workload's value law; the parity tests use it to get
    small cases that still span several tiles and a ragged tail.
    """
    c = dict(SAMPLE_CONFIGS[cfg])
    B = c["B"] if B is None else B
    K = c["K"] if K is None else K
    V = c["V"] if V is None else V
    dt = c["dtype"] if dtype is None else dtype
    T = c["T"] if temperature is None else temperature
    rng = _rng(seed, cfg, rnd, 0)
    tgt, drf, meta = _SAMPLE_LAWS[cfg](rng, B, K, V)
    tgt_s, drf_s = _store(tgt, dt), _store(drf, dt)
    drf_vals = bf16_bits_to_f32(drf_s) if dt == BF16 else drf_s
    tokens = _gumbel_draft_tokens(drf_vals, T, _rng(seed, cfg, rnd, 1))
    uni = verify_uniforms(seed, rnd, B, K)
    return SampleInputs(tgt_s, drf_s, dt, tokens, uni, float(T),
                        name=f"cfg{cfg} B={B} K={K} V={V} {dt} T={T} round={rnd}", meta=meta)


def _rows_with_placed_max(rng: np.random.Generator, R: int, V: int, scale: float):
    """R rows of V i.i.d. N(0, scale^2) values, each with its maximum at a known, uniform position."""
    lu = np.log(rng.random(R))
    upper = -np.expm1(lu / V)                       # 1 - Phi(max/scale)
    mx = -ndtri(upper)                              # max / scale
    phi_mx = np.exp(lu / V)                         # Phi(max/scale)
    rest = ndtri(rng.random((R, V - 1)) * phi_mx[:, None])  # truncated below the max
    pos = rng.integers(0, V, size=R)
    rows = np.empty((R, V), dtype=np.float64)
    for r in range(R):
        p = pos[r]
        rows[r, :p] = rest[r, :p]
        rows[r, p] = mx[r]
        rows[r, p + 1:] = rest[r, p:]
    return (rows * scale).astype(np.float32), pos


def make_greedy_inputs(rnd: int = 0, *, B: int | None = None, G: int | None = None,
                       N: int | None = None, V: int | None = None, seed: int = 0,
                       dtype: str | None = None, match_prob: float = 0.6) -> GreedyInputs:
    """Inputs of greedy verify round `rnd` (workload 5), optionally resized."""
    c = dict(GREEDY_CONFIGS[5])
    B = c["B"] if B is None else B
    G = c["G"] if G is None else G
    N = c["N"] if N is None else N
    V = c["V"] if V is None else V
    dt = c["dtype"] if dtype is None else dtype
    rng = _rng(seed, 5, rnd, 0)
    rows, pos = _rows_with_placed_max(rng, B * G * N, V, 2.0)
    logits = _store(rows.reshape(B, G, N, V), dt)
    placed = pos.reshape(B, G, N)[:, :, : N - 1]
    hit = rng.random((B, G, N - 1)) < match_prob
    rand_tok = rng.integers(0, V, size=(B, G, N - 1))
    cand = np.where(hit, placed, rand_tok).astype(np.int32)
    return GreedyInputs(logits, dt, cand, name=f"cfg5 B={B} G={G} N={N} V={V} {dt} round={rnd}",
                        meta={"placed_max": pos.reshape(B, G, N)})


FILTER_TOP_K = (0, 1, 2, 5, 20, 50, 200, 1000)
FILTER_TOP_P = (1.0, 0.99, 0.95, 0.9, 0.8, 0.5, 0.2)


def make_filter_params(B: int, seed: int = 0, *, top_k: int | None = None, top_p: float | None = None,
                       V: int | None = None):
    """Per-batch-row top-k / top-p parameters: (top_k [B] int32, top_p [B] float32).

    With top_k / top_p given, every row gets that value. Otherwise each row
    draws k from FILTER_TOP_K (plus V - 1 and V when V is given, so the
    boundary of the off range is exercised) and p from FILTER_TOP_P,
    independently: some rows use neither filter, some one, some both.
    """
    rng = _rng(seed, 77, B)
    ks = list(FILTER_TOP_K) + ([V - 1, V] if V is not None else [])
    k = np.full(B, top_k, dtype=np.int32) if top_k is not None else rng.choice(ks, size=B).astype(np.int32)
    p = (np.full(B, top_p, dtype=np.float32) if top_p is not None
         else rng.choice(FILTER_TOP_P, size=B).astype(np.float32))
    return k, p


@dataclass
class NgramSampleInputs:
    logits: np.ndarray          # [B, G, N, V] float32 values, or bf16 bits (uint16)
    dtype: str
    cand: np.ndarray            # [B, G, N-1] int32
    uniforms: np.ndarray        # [B, N, G+1] float32
    temperature: float
    name: str = ""

    @property
    def shape(self):
        return self.logits.shape

    def logits_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.logits) if self.dtype == BF16 else self.logits


def make_ngram_sample_inputs(rnd: int = 0, *, B: int = 32, G: int = 7, N: int = 5, V: int = 32000,
                             dtype: str = BF16, T: float = 1.0, peak: float = 8.0, match_prob: float = 0.6,
                             seed: int = 0) -> NgramSampleInputs:
    """A sampling verify of greedy-drafted n-grams at the greedy workload's shape.

    Rows are N(0, 1) with one token raised by `peak` (placed uniformly), so the
    tempered law puts a visible mass on it (peak 8 at T = 1 over V = 32000: about
    0.08); a candidate token is the placed token with probability `match_prob`
    (the greedy draft saw the same peak), else uniform on [0, V). Uniforms from
    ngram_uniforms (Philox, seed, round).
    """
    rng = _rng(seed, 6, rnd, 0)
    n = B * G * N
    rows = rng.normal(0.0, 1.0, size=(n, V))
    pos = rng.integers(0, V, size=n)
    rows[np.arange(n), pos] += peak
    logits = _store(rows.reshape(B, G, N, V), dtype)
    placed = pos.reshape(B, G, N)[:, :, : N - 1]
    hit = rng.random((B, G, N - 1)) < match_prob
    cand = np.where(hit, placed, rng.integers(0, V, size=(B, G, N - 1))).astype(np.int32)
    uni = ngram_uniforms(seed, rnd, B, N, G)
    return NgramSampleInputs(logits, dtype, cand, uni, float(np.float32(T)),
                             name=f"ngram-sample B={B} G={G} N={N} V={V} {dtype} T={T} round={rnd}")
