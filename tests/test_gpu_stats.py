"""The closed forms that pin the oracle, re-checked on the HIP path's own outputs (needs an MI355X).

Speculative Decoding -- LLM推理优化技术（一）: §2.2 the emitted token has law p;
§2.4 E[accept] = 1 - TV(p, q); §3.1 tokens per round (1 - a^(K+1)) / (1 - a).
Uniforms come from the device Philox (spec_fill_uniforms); draft tokens are
drawn from q on the host.
"""
import math

import numpy as np
import pytest
import torch
from scipy import special, stats

import rejection_sampling_verify_sample_amd as rsv
from pins import _fixed_tv_rows, tokens_per_round

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"


def log(msg):
    print(f"[gpu-stats] {msg}", flush=True)


def run(tgt_rows, drf_rows, tokens, seed, dtype=torch.float32, T=1.0):
    B, K = tokens.shape
    tgt = torch.from_numpy(np.ascontiguousarray(tgt_rows, dtype=np.float32)).to(dtype).to(DEV)
    drf = torch.from_numpy(np.ascontiguousarray(drf_rows, dtype=np.float32)).to(dtype).to(DEV)
    uni = rsv.fill_uniforms(seed, 0, B, K, device=DEV)
    out = rsv.verify_sample(tgt, drf, torch.from_numpy(tokens).to(DEV), uni, T)
    torch.cuda.synchronize()
    return out.tokens.cpu().numpy(), out.num_accepted.cpu().numpy()


@pytest.mark.parametrize("V", [2, 5, 16, 1000])
def test_output_law_is_p(V):
    """Chi-square of the emitted token against p over 10^6 verify rows (4 x 10^5 at V = 1000)."""
    log(f"chi-square V={V}")
    rng = np.random.default_rng(V)
    B = 1_000_000 if V <= 16 else 400_000
    lt = rng.normal(0, 1.5, V)
    ld = rng.normal(0, 1.5, V)
    if V >= 16:
        ld[: V // 4] = -np.inf
    p = special.softmax(lt)
    q = special.softmax(ld)
    tok = rng.choice(V, size=(B, 1), p=q).astype(np.int32)
    tgt = np.broadcast_to(np.stack([lt, rng.normal(0, 1, V)]), (B, 2, V))
    drf = np.broadcast_to(ld, (B, 1, V))
    out, n = run(tgt, drf, tok, seed=V)
    counts = np.bincount(out[:, 0], minlength=V)
    expect = p * B
    keep = expect >= 5
    f_obs = np.append(counts[keep], counts[~keep].sum())
    f_exp = np.append(expect[keep], expect[~keep].sum())
    if f_exp[-1] == 0:
        f_obs, f_exp = f_obs[:-1], f_exp[:-1]
    pv = stats.chisquare(f_obs, f_exp).pvalue
    log(f"  p-value {pv:.4f}")
    assert pv >= 1e-3


def test_acceptance_is_one_minus_tv():
    rng = np.random.default_rng(99)
    V, K, B = 50, 4, 400000
    tgt = rng.normal(0, 1.2, (K + 1, V))
    drf = tgt[:K] + rng.normal(0, [[0.3], [0.8], [1.5], [3.0]], (K, V))
    p = special.softmax(tgt[:K], axis=1)
    q = special.softmax(drf, axis=1)
    tv = 0.5 * np.abs(p - q).sum(axis=1)
    tok = np.stack([rng.choice(V, size=B, p=q[i]) for i in range(K)], axis=1).astype(np.int32)
    _, n = run(np.broadcast_to(tgt, (B, K + 1, V)), np.broadcast_to(drf, (B, K, V)), tok, seed=5)
    for i in range(K):
        reached = n >= i
        acc = (n[reached] > i).mean()
        sd = math.sqrt((1 - tv[i]) * tv[i] / reached.sum())
        log(f"  position {i}: accept {acc:.5f} vs 1-TV {1 - tv[i]:.5f}")
        assert abs(acc - (1 - tv[i])) <= 5 * sd


@pytest.mark.parametrize("K,alpha", [(3, 0.5), (5, 0.7), (5, 0.8), (7, 0.9), (8, 0.6)])
def test_tokens_per_round(K, alpha):
    rng = np.random.default_rng(K * 100 + int(alpha * 10))
    V, B = 16, 400000
    tgt, drf, qs = _fixed_tv_rows(rng, V, K, alpha)
    tok = np.stack([rng.choice(V, size=B, p=qs[i] / qs[i].sum()) for i in range(K)], axis=1).astype(np.int32)
    _, n = run(np.broadcast_to(tgt, (B, K + 1, V)), np.broadcast_to(drf, (B, K, V)), tok, seed=K)
    got = n + 1
    expect = tokens_per_round(alpha, K)
    log(f"  K={K} alpha={alpha}: {got.mean():.4f} vs {expect:.4f}")
    assert abs(got.mean() - expect) <= 5 * got.std() / math.sqrt(B)
