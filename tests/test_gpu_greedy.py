"""HIP greedy verify vs the CPU oracle: bit-exact (needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
import rejection_sampling_verify_sample_amd as rsv
from golden_io import greedy_case, load
from parity import compare_greedy
from workloads import bf16_round, make_greedy_inputs
from workloads.torch_io import greedy_tensors

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"


def log(msg):
    print(f"[gpu-greedy] {msg}", flush=True)


def run(logits: torch.Tensor, cand: torch.Tensor):
    out = rsv.verify_greedy(logits, cand)
    torch.cuda.synchronize()
    return out.tokens.cpu().numpy(), out.accept_len.cpu().numpy(), out.best.cpu().numpy()


def check(g):
    log(f"case {g.name}")
    t = greedy_tensors(g, DEV)
    tok, L, best = run(t["logits"], t["cand"])
    res = oracle.oracle_greedy(g.logits_f32(), g.cand)
    compare_greedy(res, tok, L, best)
    return res


@pytest.mark.parametrize("case", load("greedy_worked.json")["cases"], ids=lambda c: c["name"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_golden_rounds_on_gpu(case, dtype):
    c = greedy_case(case)
    logits = torch.from_numpy(c["logits"].astype(np.float32)).to(dtype).to(DEV)
    tok, L, best = run(logits, torch.from_numpy(c["cand"]).to(DEV))
    assert tok.tolist() == c["expect_tokens"].tolist()
    assert L.tolist() == c["expect_len"].tolist() and best.tolist() == c["expect_best"].tolist()


@pytest.mark.parametrize("rnd", range(3))
def test_full_workload(rnd):
    """B=32, G=7, N=5, V=32000 bf16: every row, bit-exact; bf16 ties occur in a few % of rows."""
    res = check(make_greedy_inputs(rnd))
    log(f"  mean accepted+1 = {(res.accept_len + 1).mean():.3f}")


@pytest.mark.parametrize("kw", [
    dict(B=5, G=1, N=2, V=7),            # plain greedy verify, V below one vector
    dict(B=3, G=9, N=65, V=1001),        # the longest candidates, ragged V
    dict(B=4, G=3, N=5, V=50001),        # rows at every 16-byte phase
    dict(B=2, G=700, N=6, V=300),        # many candidates: the epilogue loops over G
    dict(B=6, G=4, N=5, V=200000, dtype="f32"),
])
def test_shapes(kw):
    check(make_greedy_inputs(11, **kw))


def test_ties_across_segments():
    """Equal maxima placed in different segments and vector lanes: the lowest index must win."""
    log("ties")
    rng = np.random.default_rng(8)
    B, G, N, V = 2, 4, 3, 70001
    x = bf16_round(rng.normal(0, 1, (B, G, N, V)).astype(np.float32))
    positions = [(0, 5, V - 1), (1, 8191, 8192), (2, 35000, 69999), (3, 7, 8), (4, 0, 40000), (5, 16, 17)]
    flat = x.reshape(-1, V)
    for r, (_, a, b2) in enumerate(positions[: flat.shape[0]]):
        flat[r, a] = flat[r, b2] = 9.0
    flat[-1, :] = 2.0                       # a row of all-equal values: index 0
    cand = rng.integers(0, V, (B, G, N - 1)).astype(np.int32)
    cand[0, 0, 0] = 5
    cand[0, 0, 1] = 8191
    for dtype in (torch.float32, torch.bfloat16):
        t = torch.from_numpy(x).to(dtype).to(DEV)
        tok, L, best = run(t, torch.from_numpy(cand).to(DEV))
        res = oracle.oracle_greedy(x, cand)
        compare_greedy(res, tok, L, best)
        assert res.argmax.reshape(-1)[-1] == 0


def test_faults():
    log("faults")
    rng = np.random.default_rng(2)
    B, G, N, V = 4, 3, 4, 500
    x = rng.normal(0, 1, (B, G, N, V)).astype(np.float32)
    cand = rng.integers(0, V, (B, G, N - 1)).astype(np.int32)
    cand[1, 2, 2] = V                      # out of range
    cand[2, 0, 0] = -3
    x[3, 1, 2, :] = -np.inf                # a row with no finite logit
    x[0, :, :, 100:] = -np.inf             # masked vocabulary is fine
    tok, L, best = run(torch.from_numpy(x).to(DEV), torch.from_numpy(cand).to(DEV))
    res = oracle.oracle_greedy(x, cand)
    compare_greedy(res, tok, L, best)
    assert L.tolist()[1:] == [-1, -1, -1] and L[0] >= 0


def test_deterministic():
    g = make_greedy_inputs(4)
    t = greedy_tensors(g, DEV)
    a = run(t["logits"], t["cand"])
    for _ in range(3):
        b = run(t["logits"], t["cand"])
        assert all(np.array_equal(u, v) for u, v in zip(a, b))


@pytest.mark.parametrize("kw", [
    dict(B=32, G=7, N=5, V=32000),       # the workload's shape: 35 rows per batch row
    dict(B=9, G=16, N=4, V=3001),        # 64 rows: a full wave
    dict(B=5, G=1, N=17, V=2000),        # 16 candidate tokens: the wave select's longest
])
def test_wave_select_equals_workgroup_select(kw):
    """The one-wave select (G*N <= 64, N - 1 <= 16) and the workgroup select give the same
    outputs on the same argmax partials, faults included."""
    import os
    g = make_greedy_inputs(12, **kw)
    cand = g.cand.copy()
    cand[0, 0, 0] = kw["V"]              # a fault in batch row 0
    t = greedy_tensors(g, DEV)
    ct = torch.from_numpy(cand).to(DEV)
    a = run(t["logits"], ct)
    os.environ["SPECVERIFY_SELECT"] = "block"
    try:
        b = run(t["logits"], ct)
    finally:
        del os.environ["SPECVERIFY_SELECT"]
    assert all(np.array_equal(u, v) for u, v in zip(a, b))
    compare_greedy(oracle.oracle_greedy(g.logits_f32(), cand), *a)
