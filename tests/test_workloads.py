"""Input generators: Philox known answers, uniform layout, bf16 rounding, workload structure (no GPU)."""
import numpy as np
import pytest
import torch
from scipy import stats

from workloads import (SAMPLE_CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make_greedy_inputs,
                       make_sample_inputs, philox4x32_10, verify_uniforms)

# Known-answer vectors published with the Philox4x32-10 generator (Salmon et al., SC'11,
# "Parallel Random Numbers: As Easy as 1, 2, 3"; the Random123 distribution's kat_vectors).
PHILOX_KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,expect", PHILOX_KAT)
def test_philox_known_answers(ctr, key, expect):
    out = philox4x32_10(np.array(ctr, dtype=np.uint32), np.array(key, dtype=np.uint32))
    assert tuple(int(v) for v in out) == expect


def test_philox_batched_equals_scalar():
    rng = np.random.default_rng(0)
    ctr = rng.integers(0, 2 ** 32, (50, 4), dtype=np.uint64).astype(np.uint32)
    key = rng.integers(0, 2 ** 32, (50, 2), dtype=np.uint64).astype(np.uint32)
    batched = philox4x32_10(ctr, key)
    for j in range(50):
        assert np.array_equal(batched[j], philox4x32_10(ctr[j], key[j]))


def test_uniform_layout_grid_and_range():
    u = verify_uniforms(0, 3, 64, 8)
    assert u.shape == (64, 9, 2) and u.dtype == np.float32
    assert u.min() >= 0.0 and u.max() <= 1.0 - 2.0 ** -24
    assert np.all((u.astype(np.float64) * 2 ** 24) % 1 == 0)
    # counter layout: (i, b, round_lo, round_hi), key (seed_lo, seed_hi); word 0 -> r, word 1 -> u
    w = philox4x32_10(np.array([5, 17, 3, 0], dtype=np.uint32), np.array([0, 0], dtype=np.uint32))
    assert u[17, 5, 0] == (int(w[0]) >> 8) * 2.0 ** -24
    assert u[17, 5, 1] == (int(w[1]) >> 8) * 2.0 ** -24
    assert not np.array_equal(u, verify_uniforms(0, 4, 64, 8))
    assert not np.array_equal(u, verify_uniforms(1, 3, 64, 8))
    assert np.array_equal(u, verify_uniforms(0, 3, 64, 8))


def test_uniforms_are_uniform_and_uncorrelated():
    u = verify_uniforms(0, 0, 20000, 4).astype(np.float64).ravel()
    counts, _ = np.histogram(u, bins=64, range=(0, 1))
    assert stats.chisquare(counts).pvalue > 1e-3
    assert abs(np.corrcoef(u[:-1], u[1:])[0, 1]) < 5 / np.sqrt(u.size)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.normal(0, 3, 100000).astype(np.float32),
                        np.array([np.inf, -np.inf, 0.0, -0.0, 1.00390625, 1.01171875, 3.4e38], dtype=np.float32)])
    # include exact ties (halfway between two bf16 values)
    ties = (f32_to_bf16_bits(rng.normal(0, 1, 1000).astype(np.float32)).astype(np.uint32) << 16) | 0x8000
    x = np.concatenate([x, ties.view(np.float32)])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.uint16).numpy()
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_sample_workload_structure(cfg):
    c = SAMPLE_CONFIGS[cfg]
    B, K, V = min(c["B"], 6), c["K"], min(c["V"], 4096)
    s = make_sample_inputs(cfg, 0, B=B, V=V)
    assert s.shape == (B, K, V) and s.target.shape == (B, K + 1, V)
    assert s.dtype == c["dtype"]
    assert s.target.dtype == (np.uint16 if c["dtype"] == "bf16" else np.float32)
    assert s.draft_tokens.dtype == np.int32 and s.draft_tokens.min() >= 0 and s.draft_tokens.max() < V
    assert s.uniforms.shape == (B, K + 1, 2)
    s2 = make_sample_inputs(cfg, 0, B=B, V=V)
    assert np.array_equal(s.target, s2.target) and np.array_equal(s.draft_tokens, s2.draft_tokens)
    assert np.all(np.isfinite(s.target_f32())) and np.all(np.isfinite(s.draft_f32()))


def test_draft_tokens_follow_q():
    """Gumbel-max drafts have law softmax(draft/T): chi-square on one repeated row."""
    s = make_sample_inputs(1, 0, B=1, K=1, V=6)
    rows = np.repeat(s.draft, 20000, axis=0)
    from workloads.configs import _gumbel_draft_tokens
    toks = _gumbel_draft_tokens(rows, s.temperature, np.random.default_rng(9))
    z = rows[0, 0].astype(np.float64) / s.temperature
    q = np.exp(z - z.max())
    q /= q.sum()
    counts = np.bincount(toks[:, 0], minlength=6)
    assert stats.chisquare(counts, q * toks.shape[0]).pvalue > 1e-3


def test_cfg4_forced_disagreement():
    s = make_sample_inputs(4, 0, B=8, V=5000)
    tgt, drf = s.target_f32(), s.draft_f32()
    forced = s.meta["forced_disagree"]
    peak = s.meta["peak_token"]
    for b in range(4):
        for i in range(s.shape[1]):
            assert np.argmax(tgt[b, i]) == peak[b, i]
            assert (np.argmax(drf[b, i]) != peak[b, i]) == forced[b, i]


def test_greedy_workload_places_max():
    g = make_greedy_inputs(0, B=4, G=3, N=5, V=2000, dtype="f32")
    x = g.logits_f32()
    placed = g.meta["placed_max"]
    assert np.array_equal(np.argmax(x, axis=-1), placed)
    assert g.cand.shape == (4, 3, 4) and g.cand.min() >= 0 and g.cand.max() < 2000
    # law of the placed maximum: i.i.d. N(0, 2^2) rows, so x / 2 looks standard normal off the max
    rest = np.sort(x.reshape(-1, 2000), axis=1)[:, :-1].ravel() / 2.0
    assert stats.kstest(rest[::7], "norm").pvalue > 1e-4
