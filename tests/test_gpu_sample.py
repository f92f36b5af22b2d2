"""HIP sampling verify vs the CPU oracle (needs an MI355X).

Inputs are seeded and synthetic (workloads/), shaped like the five workloads;
the oracle receives the same arrays (bf16 values widened exactly to float).
"""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

import oracle
import rejection_sampling_verify_sample_amd as rsv
from golden_io import load, sample_case
from parity import AMBIGUOUS_RATE, ParityReport, compare_sample
from workloads import make_sample_inputs, verify_uniforms
from workloads.torch_io import sample_tensors

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"
REPORT_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out")


def log(msg):
    print(f"[gpu-sample] {msg}", flush=True)


def run_gpu(s, want_probs=True):
    t = sample_tensors(s, DEV)
    out = rsv.verify_sample(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"],
                            want_probs=want_probs)
    torch.cuda.synchronize()
    probs = out.probs.cpu().numpy() if want_probs else None
    return out.tokens.cpu().numpy(), out.num_accepted.cpu().numpy(), probs


def check_inputs(s, window=1e-6) -> ParityReport:
    log(f"case {s.name}")
    tok, n, probs = run_gpu(s)
    tgt, drf = s.target_f32(), s.draft_f32()
    res = oracle.oracle_sample(tgt, drf, s.draft_tokens, s.uniforms, s.temperature)
    rep = compare_sample(tgt, drf, s.draft_tokens, s.uniforms, s.temperature, res, tok, n, probs, window)
    log(f"  {rep.summary()}")
    return rep


def save_report(name, rep: ParityReport):
    os.makedirs(REPORT_DIR, exist_ok=True)
    path = os.path.join(REPORT_DIR, "parity_report.jsonl")
    with open(path, "a") as f:
        f.write(json.dumps({"case": name, "rows": rep.rows, "ambiguous": rep.ambiguous,
                            "ambiguous_agree": rep.ambiguous_agree}) + "\n")


# ------------------------------------------------------------------ hand-worked rounds

@pytest.mark.parametrize("case", load("sample_worked.json")["cases"], ids=lambda c: c["name"])
def test_golden_rounds_on_gpu(case):
    c = sample_case(case)
    log(f"golden {c['name']}")
    tgt = torch.from_numpy(c["target"].astype(np.float32)).to(DEV)
    drf = torch.from_numpy(c["draft"].astype(np.float32)).to(DEV)
    out = rsv.verify_sample(tgt, drf, torch.from_numpy(c["tokens"]).to(DEV),
                            torch.from_numpy(c["uniforms"]).to(DEV), c["T"], want_probs=True)
    torch.cuda.synchronize()
    assert out.tokens.cpu().numpy().tolist() == c["expect_tokens"].tolist()
    assert out.num_accepted.cpu().numpy().tolist() == c["expect_n"].tolist()
    # p_i(x_i), q_i(x_i) against the hand-derived values (NaN where a value does not exist)
    probs, expect = out.probs.cpu().numpy(), c["expect_probs"]
    assert np.array_equal(np.isnan(probs), np.isnan(expect))
    fin = ~np.isnan(expect)
    assert np.allclose(probs[fin], expect[fin], rtol=1e-4, atol=1e-5)


# ------------------------------------------------------------------ workloads at parity sizes

PARITY_CASES = [
    # (cfg, overrides, rounds): full sizes for 1 and 2; several tiles and ragged tails for 3 and 4
    (1, {}, 6),
    (2, {}, 4),
    (3, dict(B=8), 2),
    (3, dict(B=6, V=50001), 2),        # V odd: rows start at every 16-byte phase
    (4, dict(B=8), 1),
    (4, dict(B=6, V=40003), 1),
    (1, dict(B=5, K=1, V=7), 4),       # V smaller than one 16-byte vector
    (2, dict(B=4, K=64, V=3000), 1),   # the largest K: the ballot spans a whole wave
    (3, dict(B=7, K=0, V=1000), 2),    # K = 0: one draw from the bonus row
    (1, dict(B=1, K=1, V=300001), 2),  # two rows of 300k: 36 pass-1 segments each, merged in a loop
    (3, dict(B=2, K=2, V=1 << 20), 1), # rows of 2^20 bf16 entries over many segments and chunks
]


@pytest.mark.parametrize("cfg,kw,rounds", PARITY_CASES, ids=lambda x: str(x))
def test_parity_with_oracle(cfg, kw, rounds):
    rep = ParityReport()
    for rnd in range(rounds):
        rep.merge(check_inputs(make_sample_inputs(cfg, rnd, **kw)))
    save_report(f"cfg{cfg} {kw}", rep)
    rep.check_accounting(AMBIGUOUS_RATE[cfg])


@pytest.mark.parametrize("cfg,kw", [
    (2, dict(B=3000, V=4000)),
    (3, dict(B=1500, K=6, V=6000)),
    (4, dict(B=2000, V=3001)),
    (1, dict(B=2500, V=2000, dtype="bf16")),
], ids=lambda x: str(x))
def test_parity_many_rows(cfg, kw):
    """Thousands of rows of each value law: outside the window every row is bit-exact."""
    rep = check_inputs(make_sample_inputs(cfg, 7, **kw))
    save_report(f"cfg{cfg} many {kw}", rep)
    assert rep.rows == kw["B"]
    rep.check_accounting(AMBIGUOUS_RATE[cfg])


@pytest.mark.parametrize("cfg", [3, 4])
def test_parity_full_size(cfg):
    """The full workload in the bench's launch configuration, every row compared."""
    s = make_sample_inputs(cfg, 0)
    rep = check_inputs(s)
    save_report(f"cfg{cfg} full", rep)
    rep.check_accounting(AMBIGUOUS_RATE[cfg])


# ------------------------------------------------------------------ early exit (pass 1 in stages)

STAGED_CASES = [
    # (cfg, overrides, stage ends, rounds)
    (1, {}, [1, 2, 4], 3),
    (2, {}, [2, 5], 2),
    (3, dict(B=8), [2, 4, 8], 2),
    (3, dict(B=6, V=50001), [1, 8], 1),              # V odd: every 16-byte phase
    (4, dict(B=8), [1, 2, 3, 4], 1),
    (2, dict(B=4, K=64, V=3000), [8, 16, 32, 64], 1),  # the largest K, stages past one wave of positions
    (3, dict(B=7, K=0, V=1000), [], 1),               # K = 0: no stage, one draw from the bonus row
    (3, dict(B=16), [8], 1),                          # one stage: identical to the one-pass verify
    (3, {}, [2, 4, 8], 1),                            # the full workload in the bench's staged configuration
    (3, dict(B=48, V=4000), [3, 6, 8], 2),            # three stages, 48 batch rows
]


@pytest.mark.parametrize("cfg,kw,stages,rounds", STAGED_CASES, ids=lambda x: str(x))
def test_staged_parity_with_oracle(cfg, kw, stages, rounds):
    """Early exit gives the verify's outputs: tokens and counts under the parity rule,
    p_i(x_i), q_i(x_i) at every position the walk consulted, NaN after it (more than one stage)."""
    rep = ParityReport()
    for rnd in range(rounds):
        s = make_sample_inputs(cfg, rnd, **kw)
        log(f"staged {stages} case {s.name}")
        t = sample_tensors(s, DEV)
        out = rsv.verify_sample_staged(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"],
                                       stages, want_probs=True)
        torch.cuda.synchronize()
        tok, n, probs = out.tokens.cpu().numpy(), out.num_accepted.cpu().numpy(), out.probs.cpu().numpy()
        assert np.all(n >= 0), "these workloads hold no data fault"
        tgt, drf = s.target_f32(), s.draft_f32()
        res = oracle.oracle_sample(tgt, drf, s.draft_tokens, s.uniforms, s.temperature)
        if len(stages) > 1:
            past = np.arange(s.shape[1])[None, :] > n[:, None]
            assert np.all(np.isnan(probs[past])), "positions past the first rejection must be NaN"
            res = dataclasses.replace(res, probs=np.where(past[:, :, None], np.nan, res.probs))
        rep.merge(compare_sample(tgt, drf, s.draft_tokens, s.uniforms, s.temperature, res, tok, n, probs))
        log(f"  {rep.summary()}")
    save_report(f"staged {stages} cfg{cfg} {kw}", rep)
    rep.check_accounting(AMBIGUOUS_RATE[cfg])


@pytest.mark.parametrize("B", [32, 128])
def test_staged_matches_one_pass_on_the_gpu(B):
    """With the same segment counts the staged and the one-pass verify take the same
    row statistics, so every token and count agrees bit for bit."""
    s = make_sample_inputs(3, 1, B=B, V=20000)
    t = sample_tensors(s, DEV)
    os.environ["SPECVERIFY_S1"] = "1"
    try:
        b = rsv.verify_sample_staged(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"],
                                     [1, 3, 8])
        c = rsv.verify_sample(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"])
    finally:
        del os.environ["SPECVERIFY_S1"]
    torch.cuda.synchronize()
    assert torch.equal(b.tokens, c.tokens) and torch.equal(b.num_accepted, c.num_accepted)


# ------------------------------------------------------------------ edge cases

def _f32_inputs(target, draft, tokens, uni, T=1.0):
    return (torch.from_numpy(np.asarray(target, dtype=np.float32)).to(DEV),
            torch.from_numpy(np.asarray(draft, dtype=np.float32)).to(DEV),
            torch.from_numpy(np.asarray(tokens, dtype=np.int32)).to(DEV),
            torch.from_numpy(np.asarray(uni, dtype=np.float32)).to(DEV), T)


def test_dyadic_boundaries_exact():
    """Supports of size 2^m (logits 0 / -inf) make every p, q, alpha and C_k exact in fp32:
    u exactly on C_k must select k+1, and r exactly on alpha must reject."""
    log("dyadic boundaries")
    V, K = 64, 1
    rows = []
    for m in (0, 2, 4, 6):
        for k in range(0, 2 ** m, max(1, 2 ** m // 8)):
            rows.append((m, k))
    B = len(rows)
    tgt = np.full((B, K + 1, V), -np.inf)
    drf = np.full((B, K, V), -np.inf)
    tok = np.zeros((B, K), dtype=np.int32)
    uni = np.zeros((B, K + 1, 2), dtype=np.float32)
    for b, (m, k) in enumerate(rows):
        tgt[b, :, : 2 ** m] = 0.0          # p uniform on 2^m tokens (both rows)
        drf[b, 0, : 2 ** m] = 0.0          # q = p: accepted, then the bonus draw
        uni[b, 1, 1] = k / 2 ** m          # exactly on C_{k-1}: selects k
    out = rsv.verify_sample(*_f32_inputs(tgt, drf, tok, uni))
    torch.cuda.synchronize()
    assert out.num_accepted.cpu().tolist() == [1] * B
    assert out.tokens[:, 1].cpu().tolist() == [k for _, k in rows]
    # r exactly on alpha = 1/2 rejects; one 2^-24 below accepts
    tgt = np.full((2, 2, 8), -np.inf)
    tgt[:, :, :4] = 0.0
    drf = np.full((2, 1, 8), -np.inf)
    drf[:, 0, :2] = 0.0
    uni = np.zeros((2, 2, 2), dtype=np.float32)
    uni[0, 0, 0] = 0.5
    uni[1, 0, 0] = 0.5 - 2 ** -24
    uni[:, 0, 1] = 0.5                     # residual (0,0,1/4,1/4)/(1/2): u*Z = 1/4 = C_2 -> token 3
    out = rsv.verify_sample(*_f32_inputs(tgt, drf, np.zeros((2, 1)), uni))
    torch.cuda.synchronize()
    assert out.num_accepted.cpu().tolist() == [0, 1]
    assert out.tokens[0].cpu().tolist() == [3, -1]


def test_faults_and_masked_vocab():
    log("faults")
    V, K = 300, 2
    rng = np.random.default_rng(4)
    tgt = rng.normal(0, 1, (6, K + 1, V))
    drf = tgt[:, :K] + rng.normal(0, 0.3, (6, K, V))
    tgt[:, :, 250:] = -np.inf               # masked vocabulary
    drf[:, :, 250:] = -np.inf
    tok = np.array([[3, 4], [V, 0], [1, -1], [5, 6], [7, 8], [9, 10]], dtype=np.int32)
    uni = np.zeros((6, K + 1, 2), dtype=np.float32)
    uni[:, :, 1] = 0.37
    drf[3, 1, :] = -np.inf                  # consulted (r = 0 accepts position 0) -> fault
    tgt[4, K, :] = -np.inf                  # bonus row all -inf, reached only if both accept
    drf[4] = tgt[4, :K]                     # p = q -> both accept -> bonus row consulted -> fault
    tgt[5, 0, 9] = -np.inf                  # p(x0) = 0 -> reject at 0; row 5's later rows not consulted
    drf[5, 1, :] = -np.inf
    args = _f32_inputs(tgt, drf, tok, uni)
    out = rsv.verify_sample(*args, want_probs=True)
    torch.cuda.synchronize()
    res = oracle.oracle_sample(tgt, drf, tok, uni, 1.0)
    assert out.num_accepted.cpu().tolist() == res.n_accepted.tolist() == [res.n_accepted[0], -1, -1, -1, -1, 0]
    assert np.array_equal(out.tokens.cpu().numpy(), res.tokens)
    assert np.all(out.tokens.cpu().numpy()[1:5] == -1)
    assert 0 <= res.tokens[5, 0] < 250
    probs = out.probs.cpu().numpy()
    assert np.array_equal(np.isnan(probs), np.isnan(res.probs))   # each side NaN only by its own row
    fin = np.isfinite(res.probs)
    assert np.allclose(probs[fin], res.probs[fin], rtol=1e-4, atol=1e-5)


def test_zero_residual_falls_back_to_p():
    log("zero residual")
    V = 40
    tgt = np.full((3, 2, V), -np.inf)
    tgt[:, 0, :8] = np.linspace(0, 1, 8)
    tgt[:, 1, :] = 0.0
    drf = tgt[:, :1].copy()                 # p == q, and x has p(x) = q(x) = 0 -> alpha = 0
    tok = np.full((3, 1), 20, dtype=np.int32)
    uni = np.zeros((3, 2, 2), dtype=np.float32)
    uni[:, 0, 1] = [0.05, 0.5, 0.95]
    args = _f32_inputs(tgt, drf, tok, uni)
    out = rsv.verify_sample(*args)
    torch.cuda.synchronize()
    res = oracle.oracle_sample(tgt, drf, tok, uni, 1.0)
    assert res.fallback.all()
    assert np.array_equal(out.tokens.cpu().numpy(), res.tokens)
    assert out.num_accepted.cpu().tolist() == [0, 0, 0]


def test_temperatures():
    for T in (0.25, 0.7, 1.0, 1.6):
        s = make_sample_inputs(2, 9, B=6, V=5000, temperature=T)
        check_inputs(s)


def test_empty_batch_is_a_noop():
    t = torch.zeros((0, 3, 10), device=DEV)
    out = rsv.verify_sample(t, torch.zeros((0, 2, 10), device=DEV), torch.zeros((0, 2), dtype=torch.int32, device=DEV),
                            torch.zeros((0, 3, 2), device=DEV), 1.0)
    torch.cuda.synchronize()
    assert out.tokens.shape == (0, 3)


def test_deterministic_and_workspace_reuse():
    """Repeated calls on one workspace give bitwise-identical outputs (counters reset themselves)."""
    s = make_sample_inputs(3, 1, B=8, V=20000)
    t = sample_tensors(s, DEV)
    first = None
    for _ in range(5):
        out = rsv.verify_sample(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"],
                                want_probs=True)
        cur = (out.tokens.clone(), out.num_accepted.clone(), out.probs.clone())
        if first is None:
            first = cur
        else:
            assert all(torch.equal(a, b) for a, b in zip(first, cur))
    # a smaller call in between on the same stream, then the first again
    s2 = make_sample_inputs(1, 0, B=1, V=3000)
    run_gpu(s2)
    out = rsv.verify_sample(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"])
    torch.cuda.synchronize()
    assert torch.equal(out.tokens, first[0])


def test_graph_capture_replays():
    """The two launches captured in a HIP graph replay correctly, with eager work between replays."""
    s = make_sample_inputs(3, 2, B=8, V=30000)
    t = sample_tensors(s, DEV)
    B, K = s.draft_tokens.shape
    ws = torch.zeros(rsv.sample_workspace_size(B, K, s.shape[2]), dtype=torch.uint8, device=DEV)
    ot = torch.empty((B, K + 1), dtype=torch.int32, device=DEV)
    on = torch.empty((B,), dtype=torch.int32, device=DEV)
    eager = rsv.verify_sample(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        rsv.verify_sample(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"],
                          out_tokens=ot, out_num_accepted=on, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rsv.verify_sample(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"],
                          out_tokens=ot, out_num_accepted=on, workspace=ws)
    for rep in range(4):
        ot.fill_(-7)
        on.fill_(-7)
        _ = (t["target"].float().sum() * 0).item()   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ot, eager.tokens), f"replay {rep}"
        assert torch.equal(on, eager.num_accepted), f"replay {rep}"


def test_fill_uniforms_matches_reference_philox():
    for (seed, rnd, B, K) in ((0, 0, 64, 8), (12345678901234, 2 ** 40 + 7, 33, 5), (1, 1, 1, 0)):
        g = rsv.fill_uniforms(seed, rnd, B, K, device=DEV)
        torch.cuda.synchronize()
        assert np.array_equal(g.cpu().numpy(), verify_uniforms(seed, rnd, B, K))
