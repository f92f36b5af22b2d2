"""HIP top-k / top-p filtered verify vs the CPU oracle (needs an MI355X).

Inputs are the seeded synthetic workloads (workloads/) with per-batch-row filter
parameters (make_filter_params: a mix of k in {0,1,2,5,20,50,200,1000,V-1,V}
and p in {1,0.99,0.95,0.9,0.8,0.5,0.2}); the oracle receives the same arrays.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import rejection_sampling_verify_sample_amd as rsv
from golden_io import filtered_case, load
from parity import ParityReport, compare_filtered
from workloads import make_filter_params, make_sample_inputs
from workloads.torch_io import sample_tensors

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"
REPORT_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out")


def log(msg):
    print(f"[gpu-filtered] {msg}", flush=True)


def run_gpu(t, k, p, want_probs=True):
    kt = None if k is None else torch.from_numpy(np.asarray(k, dtype=np.int32)).to(DEV)
    pt = None if p is None else torch.from_numpy(np.asarray(p, dtype=np.float32)).to(DEV)
    out = rsv.verify_sample_filtered(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"],
                                     kt, pt, want_probs=want_probs, want_kept=True)
    torch.cuda.synchronize()
    return (out.tokens.cpu().numpy(), out.num_accepted.cpu().numpy(),
            out.probs.cpu().numpy() if want_probs else None, out.kept.cpu().numpy())


def check(s, k, p, name="") -> ParityReport:
    log(f"case {s.name} {name}")
    tok, n, probs, kept = run_gpu(sample_tensors(s, DEV), k, p)
    tgt, drf = s.target_f32(), s.draft_f32()
    B = s.shape[0]
    kk = np.zeros(B, dtype=np.int32) if k is None else np.asarray(k)
    pp = np.ones(B, dtype=np.float32) if p is None else np.asarray(p)
    res = oracle.oracle_sample_filtered(tgt, drf, s.draft_tokens, s.uniforms, s.temperature, kk, pp)
    rep = compare_filtered(tgt, drf, s.draft_tokens, s.uniforms, s.temperature, kk, pp, res, tok, n, probs, kept)
    log(f"  {rep.summary()}")
    return rep


def save_report(name, rep: ParityReport):
    os.makedirs(REPORT_DIR, exist_ok=True)
    with open(os.path.join(REPORT_DIR, "parity_report.jsonl"), "a") as f:
        f.write(json.dumps({"case": "filtered " + name, "rows": rep.rows, "ambiguous": rep.ambiguous,
                            "ambiguous_agree": rep.ambiguous_agree}) + "\n")


# ------------------------------------------------------------------ hand-worked rounds

@pytest.mark.parametrize("case", load("filtered_worked.json")["cases"], ids=lambda c: c["name"])
def test_golden_filtered_on_gpu(case):
    c = filtered_case(case)
    log(f"golden {c['name']}")
    t = dict(target=torch.from_numpy(c["target"].astype(np.float32)).to(DEV),
             draft=torch.from_numpy(c["draft"].astype(np.float32)).to(DEV),
             draft_tokens=torch.from_numpy(c["tokens"]).to(DEV),
             uniforms=torch.from_numpy(c["uniforms"]).to(DEV), temperature=c["T"])
    tok, n, probs, kept = run_gpu(t, c["top_k"], c["top_p"])
    assert tok.tolist() == c["expect_tokens"].tolist()
    assert n.tolist() == c["expect_n"].tolist()
    assert kept.tolist() == c["expect_kept"].tolist()
    res = oracle.oracle_sample_filtered(c["target"], c["draft"], c["tokens"], c["uniforms"], c["T"], c["top_k"],
                                        c["top_p"])
    assert np.allclose(probs, res.probs, rtol=1e-4, atol=1e-5, equal_nan=True), (probs, res.probs)
    # and against the hand-derived values of the renormalised kept laws
    assert np.allclose(probs, c["expect_probs"], rtol=1e-4, atol=1e-5, equal_nan=True), (probs, c["expect_probs"])


# ------------------------------------------------------------------ workloads with mixed filters

CASES = [
    (1, dict(B=6, V=5000)),
    (2, dict()),                          # full size: B=8 K=5 V=32000 bf16 T=0.7
    (3, dict(B=6, V=20001)),              # bf16, odd V: every 16-byte phase
    (4, dict(B=8, V=40003)),              # fp32 peaked and flat rows, three radix digits
    (3, dict(B=5, K=0, V=1000)),          # K = 0: the bonus row only
    (2, dict(B=3, K=64, V=3000)),         # the largest K
    (1, dict(B=4, K=2, V=7)),             # V smaller than a vector
    (3, dict(B=3, K=2, V=1 << 20)),       # rows of 2^20 bf16 entries under every filter route
]


@pytest.mark.parametrize("cfg,kw", CASES, ids=lambda x: str(x))
def test_filtered_parity_mixed(cfg, kw):
    rep = ParityReport()
    for rnd in range(2):
        s = make_sample_inputs(cfg, rnd, **kw)
        B, _, V = s.shape
        k, p = make_filter_params(B, seed=rnd, V=V)
        rep.merge(check(s, k, p))
    save_report(f"cfg{cfg} {kw}", rep)
    rep.check_accounting()


def test_filtered_parity_full_size_k50_p09():
    """The full B=64 K=8 V=128256 bf16 round with top-k 50, top-p 0.9 on every row, all rows compared."""
    s = make_sample_inputs(3, 0)
    k, p = make_filter_params(64, top_k=50, top_p=0.9)
    rep = check(s, k, p, "k50 p0.9")
    save_report("cfg3 full k50 p0.9", rep)
    rep.check_accounting()


def test_filtered_parity_full_size_p09():
    """The full B=64 K=8 V=128256 bf16 round with top-p 0.9 alone on every row (long bf16
    rows: the key-count route), all rows compared."""
    s = make_sample_inputs(3, 0)
    k, p = make_filter_params(64, top_k=0, top_p=0.9)
    rep = check(s, k, p, "p0.9")
    save_report("cfg3 full p0.9", rep)
    rep.check_accounting()


@pytest.fixture(scope="module")
def cfg4_full():
    return make_sample_inputs(4, 0)


@pytest.mark.parametrize("top_k,top_p", [(50, 0.9), (0, 0.9)])
def test_filtered_parity_full_size_fp32_sampled(cfg4_full, top_k, top_p):
    """The full B=256 K=4 V=152064 fp32 round (rows b < 128 peaked, the rest flat; flat
    rows with top-p alone take the two-read route) launched whole, as timed; 32 batch
    rows, 16 peaked and 16 flat, compared with the oracle run on those rows alone (a
    batch row's outputs depend only on its own rows)."""
    s = cfg4_full
    B = s.shape[0]
    k, p = make_filter_params(B, top_k=top_k, top_p=top_p)
    log(f"cfg4 full k={top_k} p={top_p}")
    tok, n, probs, kept = run_gpu(sample_tensors(s, DEV), k, p)
    idx = np.r_[0:8, 120:128, 128:136, B - 8:B]
    tgt, drf = s.target_f32()[idx], s.draft_f32()[idx]
    toks, uni = s.draft_tokens[idx], s.uniforms[idx]
    res = oracle.oracle_sample_filtered(tgt, drf, toks, uni, s.temperature, k[idx], p[idx])
    rep = compare_filtered(tgt, drf, toks, uni, s.temperature, k[idx], p[idx], res, tok[idx], n[idx], probs[idx],
                           kept[idx])
    log(f"  {rep.summary()}")
    save_report(f"cfg4 full sampled k{top_k} p{top_p}", rep)
    rep.check_accounting()


@pytest.mark.parametrize("k,p", [(None, None), (0, 1.0), (1, 1.0), (0, 1e-30), (0, float("nan")), (2000, 0.999),
                                 (7, 0.3), (0, 0.95)], ids=lambda x: str(x))
def test_filter_settings(k, p):
    s = make_sample_inputs(1, 3, B=6, V=2000)
    B = 6
    kk = None if k is None else np.full(B, k, dtype=np.int32)
    pp = None if p is None else np.full(B, p, dtype=np.float32)
    check(s, kk, pp, f"k={k} p={p}").check_accounting()


# ------------------------------------------------------------------ exact keys, ties and masks

def _f32_tensors(tgt, drf, toks, uni, T=1.0):
    return dict(target=torch.from_numpy(np.ascontiguousarray(tgt, dtype=np.float32)).to(DEV),
                draft=torch.from_numpy(np.ascontiguousarray(drf, dtype=np.float32)).to(DEV),
                draft_tokens=torch.from_numpy(np.asarray(toks, dtype=np.int32)).to(DEV),
                uniforms=torch.from_numpy(np.asarray(uni, dtype=np.float32)).to(DEV), temperature=T)


def test_top_k_resolves_adjacent_float_keys():
    """fp32 logits one ulp apart (all three radix digits matter) and bf16-style ties: top-k counts exact."""
    log("adjacent keys")
    rng = np.random.default_rng(3)
    B, K, V = 6, 1, 4099
    base = np.float32(1.5)
    vals = [base]
    for _ in range(V - 1):
        vals.append(np.nextafter(vals[-1], np.float32(2), dtype=np.float32))
    vals = np.array(vals, dtype=np.float32)
    tgt = np.empty((B, K + 1, V), dtype=np.float32)
    for b in range(B):
        for j in range(K + 1):
            tgt[b, j] = rng.permutation(vals)
    tgt[1] = np.round(tgt[1] * 4) / 4          # many ties
    tgt[2, :, : V // 2] = -np.inf              # masked half
    drf = tgt[:, :K].copy()
    toks = rng.integers(0, V, (B, K))
    uni = np.full((B, K + 1, 2), 0.5, dtype=np.float32)
    ks = np.array([1, 37, 4098, 1000, 3000, 2], dtype=np.int32)
    tok, n, _, kept = run_gpu(_f32_tensors(tgt, drf, toks, uni), ks, None, want_probs=False)
    res = oracle.oracle_sample_filtered(tgt, drf, toks, uni, 1.0, ks, np.ones(B, dtype=np.float32))
    assert np.array_equal(kept, res.kept), (kept, res.kept)
    assert np.array_equal(n, res.n_accepted)


def test_faults_and_empty_rows_filtered():
    log("faults")
    V, K = 300, 2
    rng = np.random.default_rng(4)
    tgt = rng.normal(0, 1, (4, K + 1, V))
    drf = tgt[:, :K] + rng.normal(0, 0.3, (4, K, V))
    toks = np.array([[3, 4], [V, 0], [1, 2], [5, 6]], dtype=np.int32)
    uni = np.zeros((4, K + 1, 2), dtype=np.float32)
    drf[2, 1, :] = -np.inf                   # consulted (r = 0 accepts at 0 when alpha > 0) -> fault, or not
    tgt[3, K, :] = -np.inf
    drf[3] = tgt[3, :K]
    t = _f32_tensors(tgt, drf, toks, uni)
    k = np.array([5, 5, 0, 0], dtype=np.int32)
    p = np.array([1.0, 0.9, 0.9, 0.5], dtype=np.float32)
    tok, n, probs, kept = run_gpu(t, k, p)
    res = oracle.oracle_sample_filtered(tgt, drf, toks, uni, 1.0, k, p)
    compare_filtered(tgt, drf, toks, uni, 1.0, k, p, res, tok, n, probs, kept).check_accounting()
    assert kept[3, K] == 0 and kept[2, K + 2] == 0


def test_filtered_is_deterministic():
    log("determinism")
    s = make_sample_inputs(4, 1, B=6, V=30000)
    k, p = make_filter_params(6, seed=5, V=30000)
    t = sample_tensors(s, DEV)
    a = run_gpu(t, k, p)
    b = run_gpu(t, k, p)
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True) if x.dtype.kind == "f" else np.array_equal(x, y)


def _bf16_tensors(tgt, drf, toks, uni, T=1.0):
    tb = torch.from_numpy(np.ascontiguousarray(tgt, dtype=np.float32)).to(torch.bfloat16)
    db = torch.from_numpy(np.ascontiguousarray(drf, dtype=np.float32)).to(torch.bfloat16)
    t = dict(target=tb.to(DEV), draft=db.to(DEV),
             draft_tokens=torch.from_numpy(np.asarray(toks, dtype=np.int32)).to(DEV),
             uniforms=torch.from_numpy(np.asarray(uni, dtype=np.float32)).to(DEV), temperature=T)
    return t, tb.float().numpy(), db.float().numpy()


@pytest.mark.parametrize("dtype,V", [("f32", 20011), ("bf16", 20011), ("f32", 3001), ("bf16", 3001)])
def test_one_pass_top_k_and_its_fallbacks(dtype, V):
    """Top-k with k <= 64 reads a row once into a candidate buffer; a row whose
    candidates overflow the buffer (ties at the top, ascending rows, -inf ties
    that top-k keeps) goes to the multi-pass select. At V = 3001 every row fits
    the buffer. Rows 0 and 7 hold only negative logits. Kept counts exact, the
    round against the oracle."""
    log(f"one-pass top-k {dtype} V={V}")
    rng = np.random.default_rng(11)
    B, K = 8, 1
    tgt = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    tgt[1, :, : V // 3] = 9.0                        # a third of the row tied at the maximum; k = 5 keeps them all
    tgt[2] = np.linspace(-10, 10, V, dtype=np.float32)[None]  # ascending: every entry beats the running bound
    tgt[3, :, 5:] = -np.inf                          # five finite entries; k = 10 keeps the -inf ties too
    tgt[4] = np.round(tgt[4] * 2) / 2                # coarse ties
    tgt[0] = -np.abs(tgt[0]) - 5.0                   # every logit negative: the k-th largest key
    tgt[7] = -np.abs(tgt[7]) - 0.5                   # has its sign bit clear (bf16: low half all ones)
    drf = (tgt[:, :K] + rng.normal(0, 0.5, (B, K, V))).astype(np.float32)
    toks = rng.integers(0, 5, (B, K))
    uni = rng.random((B, K + 1, 2)).astype(np.float32)
    ks = np.array([64, 5, 50, 10, 20, 65, 1, 64], dtype=np.int32)
    ps = np.array([1.0, 0.9, 1.0, 0.9, 0.8, 0.9, 1.0, 0.5], dtype=np.float32)
    if dtype == "f32":
        t, tg, dr = _f32_tensors(tgt, drf, toks, uni), tgt, drf
    else:
        t, tg, dr = _bf16_tensors(tgt, drf, toks, uni)
    tok, n, probs, kept = run_gpu(t, ks, ps)
    res = oracle.oracle_sample_filtered(tg, dr, toks, uni, 1.0, ks, ps)
    top_k_only = ps >= 1.0
    assert np.array_equal(kept[top_k_only], res.kept[top_k_only]), (kept, res.kept)
    compare_filtered(tg, dr, toks, uni, 1.0, ks, ps, res, tok, n, probs, kept).check_accounting()


def _run_multi_pass(t, k, p):
    """The same call with every row sent to the multi-pass select."""
    os.environ["SPECVERIFY_FILTER"] = "multi"
    try:
        return run_gpu(t, k, p)
    finally:
        del os.environ["SPECVERIFY_FILTER"]


@pytest.mark.parametrize("dtype,V", [("bf16", 128256), ("f32", 40003), ("bf16", 20011), ("f32", 8000),
                                     ("bf16", 3001)])
def test_one_read_top_p_and_large_top_k(dtype, V):
    """Top-p alone, and top-k with k > 64, read a row once: a bound from the first
    step of the read, the entries above it in a buffer, the cut there. Rows cover a
    buffer that holds the cut, a sample that puts the bound above the cut (its mass
    sits far below the sample's), rows too flat for the buffer (multi-pass select),
    ties, masked halves and all-negative rows; V at or below the buffer takes every
    entry. Kept counts and rounds against the oracle, and against the multi-pass
    select of the same rows."""
    log(f"one-read top-p / large top-k {dtype} V={V}")
    rng = np.random.default_rng(17)
    B, K = 10, 1
    tgt = (rng.normal(0, 3, (B, K + 1, V))).astype(np.float32)
    tgt[1] = np.float32(-20.0)                        # the sample's mass sits at 10, the row's at 5
    tgt[1, :, 64:74] = 10.0
    tgt[1, :, 20000 % V:] = np.where(rng.random((K + 1, V - 20000 % V)) < 0.8, 5.0, -20.0)
    tgt[2] = rng.normal(0, 0.3, (K + 1, V))           # flat: the nucleus is most of the row
    tgt[3] = np.round(tgt[3] * 2) / 2                 # ties
    tgt[4, :, : V // 2] = -np.inf                     # masked half
    tgt[5] = -np.abs(tgt[5]) - 1.0                    # every logit negative
    tgt[6] = np.sort(tgt[6], axis=-1)                 # ascending
    drf = (tgt[:, :K] + rng.normal(0, 0.5, (B, K, V))).astype(np.float32)
    drf[1] = tgt[1, :K]
    toks = rng.integers(0, V, (B, K))
    toks[1] = 70
    uni = rng.random((B, K + 1, 2)).astype(np.float32)
    ks = np.array([0, 0, 0, 0, 0, 0, 100, 1000, 5000, 300], dtype=np.int32)
    ps = np.array([0.9, 0.9, 0.95, 0.8, 0.5, 0.99, 1.0, 1.0, 0.9, 0.0], dtype=np.float32)
    if dtype == "f32":
        t, tg, dr = _f32_tensors(tgt, drf, toks, uni), tgt, drf
    else:
        t, tg, dr = _bf16_tensors(tgt, drf, toks, uni)
    tok, n, probs, kept = run_gpu(t, ks, ps)
    res = oracle.oracle_sample_filtered(tg, dr, toks, uni, 1.0, ks, ps)
    rep = compare_filtered(tg, dr, toks, uni, 1.0, ks, ps, res, tok, n, probs, kept)
    log(f"  {rep.summary()}")
    rep.check_accounting()
    top_k_only = ps >= 1.0
    assert np.array_equal(kept[top_k_only], res.kept[top_k_only]), (kept, res.kept)
    tok2, n2, probs2, kept2 = _run_multi_pass(t, ks, ps)
    sure = res.filter_margin >= 1e-6
    assert np.array_equal(kept[sure], kept2[sure]), (kept, kept2)
    same_rows = (res.min_margin() >= 1e-6)
    assert np.array_equal(tok[same_rows], tok2[same_rows]) and np.array_equal(n[same_rows], n2[same_rows])


@pytest.mark.parametrize("dtype,V", [("f32", 50021), ("bf16", 50021), ("f32", 152064)])
def test_filtered_residual_without_mass_draws_from_the_kept_target(dtype, V):
    """Draft rows equal to the target rows: the same filter keeps the same law on both
    sides (p' = q'), and a draft token outside the kept set is rejected (q'(x) = 0 and
    p'(x) = 0), leaving a residual with no mass, so the token is drawn from p'_n. The
    kept set spans many chunks of the row; the draws are compared with the oracle."""
    log(f"filtered zero residual {dtype} V={V}")
    rng = np.random.default_rng(23)
    B, K = 16, 2
    tgt = rng.normal(0, 1, (B, K + 1, V)).astype(np.float32)
    for b in range(B):
        for i in range(K + 1):
            hot = rng.choice(V, 40, replace=False)
            tgt[b, i, hot] = rng.uniform(7.0, 9.0, 40).astype(np.float32)
    drf = tgt[:, :K].copy()
    toks = np.zeros((B, K), dtype=np.int64)
    for b in range(B):
        for i in range(K):
            toks[b, i] = int(np.argmin(tgt[b, i]))  # never kept by top-p 0.9
    uni = rng.random((B, K + 1, 2)).astype(np.float32)
    ks = np.zeros(B, dtype=np.int32)
    ps = np.full(B, 0.9, dtype=np.float32)
    ps[::4] = 0.5
    if dtype == "f32":
        t, tg, dr = _f32_tensors(tgt, drf, toks, uni), tgt, drf
    else:
        t, tg, dr = _bf16_tensors(tgt, drf, toks, uni)
    tok, n, probs, kept = run_gpu(t, ks, ps)
    res = oracle.oracle_sample_filtered(tg, dr, toks, uni, 1.0, ks, ps)
    assert np.all(res.n_accepted == 0) and np.all(n == 0), (n, res.n_accepted)
    assert np.all(res.fallback), res.fallback  # the residual held no mass in every row
    rep = compare_filtered(tg, dr, toks, uni, 1.0, ks, ps, res, tok, n, probs, kept)
    log(f"  {rep.summary()}")
    rep.check_accounting()
    # every draw lands on a token the target's filter keeps at position 0
    for b in range(B):
        x0 = tg[b, 0]
        assert tok[b, 0] >= 0 and x0[tok[b, 0]] >= np.sort(x0)[-int(kept[b, 0])], (b, tok[b, 0])


def _million_entry_row(rng, V, T, n_top=20000):
    """A row of V entries whose nucleus is about n_top entries spread over 8 doublings of
    mass (more than the candidate buffer holds), above a tail of V - n_top entries that
    holds about 5% of the mass: the cut's band is narrow, the row long."""
    x = (T * np.log(0.0485) + rng.normal(0, 0.05, V)).astype(np.float32)
    top = rng.choice(V, n_top, replace=False)
    x[top] = rng.uniform(0.0, 8 * T * np.log(2.0), n_top).astype(np.float32)
    return x


def test_two_read_top_p_on_a_million_entry_fp32_row():
    """Top-p alone on fp32 rows of 2^20 entries whose nucleus outgrows the buffer but
    whose band fits it: the two-read route, whose second read moves its per-thread
    fp64 sums to 64-bit integers every 3,072 entries (more than 256 steps per thread
    here). Equal to the multi-pass select, and the oracle's round."""
    log("two-read top-p fp32 V=2^20")
    rng = np.random.default_rng(41)
    B, K, V, T = 2, 1, 1 << 20, 0.8
    tgt = np.stack([np.stack([_million_entry_row(rng, V, T) for _ in range(K + 1)]) for _ in range(B)])
    drf = (tgt[:, :K] + rng.normal(0, 0.05, (B, K, V))).astype(np.float32)
    toks = rng.integers(0, V, (B, K))
    uni = rng.random((B, K + 1, 2)).astype(np.float32)
    ks = np.zeros(B, dtype=np.int32)
    ps = np.array([0.9, 0.8], dtype=np.float32)
    t = _f32_tensors(tgt, drf, toks, uni, T=T)
    tok, n, probs, kept = run_gpu(t, ks, ps)
    tok2, n2, probs2, kept2 = _run_multi_pass(t, ks, ps)
    assert np.array_equal(kept, kept2), (kept, kept2)
    assert np.array_equal(tok, tok2) and np.array_equal(n, n2)
    assert np.all(kept > 6144)  # every nucleus outgrows the buffer
    res = oracle.oracle_sample_filtered(tgt, drf, toks, uni, T, ks, ps)
    rep = compare_filtered(tgt, drf, toks, uni, T, ks, ps, res, tok, n, probs, kept)
    log(f"  {rep.summary()}")
    rep.check_accounting()


def _crowd_ties_into_wave0(x, p, T, n_tie, rng):
    """A flat fp32 row whose top-p cut falls inside a block of n_tie equal entries, all
    placed where the second read hands them to wave 0 (16-byte vectors 0-63 of every
    256: entries whose index mod 1024 is below 256)."""
    V = x.size
    order = np.argsort(-x.astype(np.float64), kind="stable")
    m = np.exp((x[order].astype(np.float64) - x.max()) / T)
    kstar = int(np.searchsorted(np.cumsum(m) / m.sum(), p))
    lo = max(kstar - n_tie // 2, 0)
    vals = x[order].copy()
    vals[lo:lo + n_tie] = vals[kstar]                      # the block of ties around the cut
    wave0 = np.nonzero((np.arange(V) % 1024) < 256)[0]
    rest = np.setdiff1d(np.arange(V), wave0[:n_tie])
    out = np.empty_like(x)
    out[wave0[:n_tie]] = vals[lo:lo + n_tie]
    others = np.concatenate([vals[:lo], vals[lo + n_tie:]])
    out[rest] = others[rng.permutation(others.size)]
    return out, vals[kstar]


def test_two_read_band_held_by_one_wave():
    """The second read keeps the band's entries in four parts of the buffer, one per
    wave. Rows whose band (a block of 2500 ties at the cut) all falls to wave 0 overflow
    its part of 1536; they take the multi-pass select, so the round equals it, and the
    oracle's."""
    log("two-read band in one wave")
    rng = np.random.default_rng(37)
    B, K, V, T, p = 2, 1, 152064, 0.8, 0.9
    tgt = rng.normal(0, 0.5, (B, K + 1, V)).astype(np.float32)
    for b in range(B):
        for i in range(K + 1):
            tgt[b, i], tv = _crowd_ties_into_wave0(tgt[b, i], p, T, 2500, rng)
            m = np.exp((tgt[b, i].astype(np.float64) - tgt[b, i].max()) / T)
            above, at = m[tgt[b, i] > tv].sum(), m[tgt[b, i] == tv].sum()
            assert above < p * m.sum() <= above + at, "the cut must fall inside the block of ties"
    drf = tgt[:, :K].copy()
    drf[1] = tgt[1, :K] + rng.normal(0, 0.3, (K, V)).astype(np.float32)  # row 1: the draft side is not crowded
    toks = rng.integers(0, V, (B, K))
    uni = rng.random((B, K + 1, 2)).astype(np.float32)
    ks = np.zeros(B, dtype=np.int32)
    ps = np.full(B, p, dtype=np.float32)
    t = _f32_tensors(tgt, drf, toks, uni, T=T)
    tok, n, probs, kept = run_gpu(t, ks, ps)
    tok2, n2, probs2, kept2 = _run_multi_pass(t, ks, ps)
    assert np.array_equal(kept, kept2), (kept, kept2)
    assert np.array_equal(tok, tok2) and np.array_equal(n, n2)
    res = oracle.oracle_sample_filtered(tgt, drf, toks, uni, T, ks, ps)
    rep = compare_filtered(tgt, drf, toks, uni, T, ks, ps, res, tok, n, probs, kept)
    log(f"  {rep.summary()}")
    rep.check_accounting()


@pytest.mark.parametrize("V", [152064, 40003, 6145])
def test_two_read_top_p_on_long_fp32_rows(V):
    """Top-p alone on fp32 rows whose nucleus is larger than the candidate buffer (flat
    rows) takes two reads: counts per key half bound the cut to a band of keys, and the
    second read cuts there with exact masses. The kept counts, thresholds and the whole
    round equal the multi-pass select's bit for bit, and agree with the oracle."""
    log(f"two-read top-p fp32 V={V}")
    rng = np.random.default_rng(31)
    B, K = 8, 2
    tgt = rng.normal(0, 0.5, (B, K + 1, V)).astype(np.float32)    # flat: most of the row is kept
    tgt[1] = rng.normal(0, 1.0, (K + 1, V))
    tgt[2] = np.round(tgt[2] * 8) / 8                              # ties across the band
    tgt[3, :, : V // 3] = -np.inf                                  # masked third
    tgt[4] = -np.abs(tgt[4]) - 3.0                                 # every logit negative
    tgt[5, :, rng.choice(V, 3, replace=False)] = 6.0               # a few raised tokens on a flat row
    tgt[6] = rng.uniform(-1, 1, (K + 1, V))
    drf = (tgt[:, :K] + rng.normal(0, 0.3, (B, K, V))).astype(np.float32)
    toks = rng.integers(0, V, (B, K))
    uni = rng.random((B, K + 1, 2)).astype(np.float32)
    ks = np.zeros(B, dtype=np.int32)
    ps = np.array([0.9, 0.5, 0.9, 0.95, 0.99, 0.9, 0.999, 0.7], dtype=np.float32)
    t = _f32_tensors(tgt, drf, toks, uni, T=0.8)
    tok, n, probs, kept = run_gpu(t, ks, ps)
    tok2, n2, probs2, kept2 = _run_multi_pass(t, ks, ps)
    assert np.array_equal(kept, kept2), (kept, kept2)
    assert np.array_equal(tok, tok2) and np.array_equal(n, n2)
    res = oracle.oracle_sample_filtered(tgt, drf, toks, uni, 0.8, ks, ps)
    rep = compare_filtered(tgt, drf, toks, uni, 0.8, ks, ps, res, tok, n, probs, kept)
    log(f"  {rep.summary()}")
    rep.check_accounting()
