"""HIP sampling verify of greedy-drafted n-gram candidates vs the CPU oracle (needs an MI355X).

Inputs: the hand-worked walks of tests/golden/ngram_sample_worked.json, and
seeded synthetic rounds (workloads.make_ngram_sample_inputs: peaked rows,
candidates that follow the peak with probability 0.6) in bf16 and fp32 at
several shapes, including one candidate, the most candidates, the shortest and
longest n-grams and vocabularies that are not a whole number of 16-byte vectors.
"""
import numpy as np
import pytest
import torch

import oracle
import rejection_sampling_verify_sample_amd as rsv
from golden_io import load, ngram_sample_case
from parity import ParityReport, compare_ngram_sample
from workloads import make_ngram_sample_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"


def log(msg):
    print(f"[gpu-ngram-sample] {msg}", flush=True)


def to_dev(s):
    lg = torch.from_numpy(s.logits).to(DEV)
    lg = lg.view(torch.bfloat16) if s.dtype == "bf16" else lg
    return lg, torch.from_numpy(s.cand).to(DEV), torch.from_numpy(s.uniforms).to(DEV)


def run(s):
    lg, cd, un = to_dev(s)
    out = rsv.verify_ngram_sample(lg, cd, un, s.temperature)
    torch.cuda.synchronize()
    return out.tokens.cpu().numpy(), out.accept_len.cpu().numpy(), out.rows.cpu().numpy()


@pytest.mark.parametrize("case", load("ngram_sample_worked.json")["cases"], ids=lambda c: c["name"])
def test_golden_walks_on_gpu(case):
    c = ngram_sample_case(case)
    lg = torch.from_numpy(c["logits"].astype(np.float32)).to(DEV)
    out = rsv.verify_ngram_sample(lg, torch.from_numpy(c["cand"]).to(DEV),
                                  torch.from_numpy(c["uniforms"].astype(np.float32)).to(DEV), c["T"])
    torch.cuda.synchronize()
    assert out.tokens.cpu().numpy().tolist() == c["expect_tokens"].tolist()
    assert out.accept_len.cpu().numpy().tolist() == c["expect_len"].tolist()
    assert out.rows.cpu().numpy().tolist() == c["expect_rows"].tolist()


CASES = [
    # (overrides, rounds)
    (dict(), 1),                                              # the bench shape: B=32 G=7 N=5 V=32000 bf16
    (dict(B=64, V=3001, dtype="f32", T=0.8), 2),              # fp32, odd V
    (dict(B=40, G=1, N=6, V=2000, peak=6.0), 2),              # one candidate
    (dict(B=8, G=64, N=3, V=1000, match_prob=0.9), 2),        # the most candidates, many duplicates
    (dict(B=16, G=3, N=2, V=500, peak=3.0), 3),               # the shortest n-grams: one try position + bonus
    (dict(B=4, G=2, N=65, V=300, peak=12.0, match_prob=0.97), 1),  # the longest n-grams, deep walks
    (dict(B=24, G=5, N=4, V=7, dtype="f32", peak=1.0), 3),    # V below one 16-byte vector
    (dict(B=6, G=4, N=4, V=152064, peak=10.0), 1),           # rows past 16 blocks: read block after block
    (dict(B=6, G=3, N=3, V=50021, dtype="f32", peak=8.0), 1),  # the same in fp32, odd V
]


@pytest.mark.parametrize("kw,rounds", CASES, ids=lambda x: str(x))
def test_parity_with_oracle(kw, rounds):
    rep = ParityReport()
    for rnd in range(rounds):
        s = make_ngram_sample_inputs(rnd, **kw)
        log(f"case {s.name}")
        tok, L, rows = run(s)
        res = oracle.oracle_ngram_sample(s.logits_f32(), s.cand, s.uniforms, s.temperature)
        rep.merge(compare_ngram_sample(s.cand, s.shape[3], res, tok, L, rows))
        log(f"  {rep.summary()} mean accepted {L.mean():.3f}")
    rep.check_accounting()


def test_one_candidate_matches_the_sample_verify_on_gpu():
    """G = 1 is speculative decoding with a one-hot draft row: both GPU paths agree bit for bit."""
    s = make_ngram_sample_inputs(3, B=48, G=1, N=6, V=4000, dtype="f32", peak=6.0)
    tok, L, _ = run(s)
    B, _, N, V = s.shape
    target = torch.from_numpy(s.logits_f32()[:, 0]).to(DEV)
    draft = torch.full((B, N - 1, V), float("-inf"))
    for b in range(B):
        draft[b, torch.arange(N - 1), torch.from_numpy(s.cand[b, 0]).long()] = 0.0
    uni = torch.zeros((B, N, 2))
    uni[:, :, 0] = torch.from_numpy(s.uniforms[:, :, 0])
    uni[:, :, 1] = torch.from_numpy(s.uniforms[:, :, 1])
    out = rsv.verify_sample(target, draft.to(DEV), torch.from_numpy(s.cand[:, 0].copy()).to(DEV), uni.to(DEV),
                            s.temperature)
    torch.cuda.synchronize()
    assert np.array_equal(out.num_accepted.cpu().numpy(), L)
    assert np.array_equal(out.tokens.cpu().numpy(), tok)


def test_first_token_law_chisquare():
    """The emitted first token follows the target's law (chi-square over 2e5 rows, V = 6, G = 3)."""
    from scipy import stats
    rng = np.random.default_rng(11)
    V, G, N, B = 6, 3, 2, 200000
    p0 = np.array([0.3, 0.05, 0.25, 0.1, 0.2, 0.1])
    logits = np.zeros((B, G, N, V), dtype=np.float32)
    logits[:, :, 0] = np.log(p0).astype(np.float32)
    logits[:, :, 1] = rng.normal(size=(1, G, V)).astype(np.float32)
    cand = np.broadcast_to(np.array([0, 2, 0], dtype=np.int32)[None, :, None], (B, G, 1)).copy()
    uni = rng.random((B, N, G + 1)).astype(np.float32)
    out = rsv.verify_ngram_sample(torch.from_numpy(logits).to(DEV), torch.from_numpy(cand).to(DEV),
                                  torch.from_numpy(uni).to(DEV), 1.0)
    torch.cuda.synchronize()
    first = out.tokens[:, 0].cpu().numpy()
    counts = np.bincount(first, minlength=V)
    p = np.exp(np.log(p0).astype(np.float32).astype(np.float64))
    p /= p.sum()
    chi = stats.chisquare(counts, B * p)
    log(f"first-token chi-square p-value {chi.pvalue:.3g}")
    assert chi.pvalue > 1e-3


def test_deterministic_and_workspace_reuse():
    """Repeated calls on one workspace give bitwise-identical outputs, also after a call
    of another shape has used it."""
    s = make_ngram_sample_inputs(0, peak=10.0)
    small = make_ngram_sample_inputs(1, B=3, G=2, N=3, V=1000, peak=10.0)
    lg, cd, un = to_dev(s)
    slg, scd, sun = to_dev(small)
    B, G, N, V = s.shape
    ws = torch.zeros(rsv.ngram_sample_workspace_size(B, G, N, V), dtype=torch.uint8, device=DEV)
    outs = []
    for rep in range(3):
        out = rsv.verify_ngram_sample(lg, cd, un, s.temperature, workspace=ws)
        outs.append((out.tokens.clone(), out.accept_len.clone(), out.rows.clone()))
        rsv.verify_ngram_sample(slg, scd, sun, small.temperature, workspace=ws)
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert all(torch.equal(a, b) for a, b in zip(outs[0], o))
