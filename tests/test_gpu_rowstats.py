"""Full-row probability parity (needs an MI355X).

spec_row_stats exports, for each logit row, the maximum m and the denominator S
the verify's streaming reduction computes, so that the row's law is
p_v = 2^(x_v c - fl32(m c)) / S with c = fl32(log2(e) / T). Every probability of
every target and draft row of the four sampling workloads, at full size, is
rebuilt from them and compared with the oracle's float64 softmax (rtol 1e-4,
atol 1e-5: the probability tolerance of the parity rule). The verify's own
p_i(x_i), q_i(x_i) must match the rebuilt rows at the draft tokens.
"""
import numpy as np
import pytest
import torch

import oracle
import rejection_sampling_verify_sample_amd as rsv
from parity import PROB_ATOL, PROB_RTOL
from workloads import make_sample_inputs
from workloads.torch_io import sample_tensors

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"


def log(msg):
    print(f"[gpu-rowstats] {msg}", flush=True)


def _c32(T: float) -> np.float32:
    """log2(e) / T rounded to fp32, with T the fp32 value passed (as the library forms it)."""
    return np.float32(1.4426950408889634074 / float(np.float32(T)))


def rebuilt(x: np.ndarray, m: np.ndarray, S: np.ndarray, T: float) -> np.ndarray:
    c = _c32(T)
    R = (m.astype(np.float32) * c).astype(np.float32)
    return np.exp2(x.astype(np.float64) * float(c) - R.astype(np.float64)[:, None]) / S[:, None]


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_every_probability_of_every_row(cfg):
    s = make_sample_inputs(cfg, 0)
    B, K, V = s.shape
    T = s.temperature
    log(f"workload {cfg}: B={B} K={K} V={V} {s.dtype}")
    t = sample_tensors(s, DEV)
    worst = 0.0
    for name, dev_rows, host in (("target", t["target"], s.target_f32()), ("draft", t["draft"], s.draft_f32())):
        rows = dev_rows.reshape(-1, V)
        m, S = rsv.row_stats(rows, T)
        torch.cuda.synchronize()
        m, S = m.cpu().numpy(), S.cpu().numpy()
        x = host.reshape(-1, V)
        assert np.array_equal(m, x.max(axis=1)), f"{name}: row maxima differ"
        for r0 in range(0, x.shape[0], 64):
            r1 = min(r0 + 64, x.shape[0])
            p = rebuilt(x[r0:r1], m[r0:r1], S[r0:r1], T)
            ref = np.stack([oracle.softmax64(x[r], T) for r in range(r0, r1)])
            ok = np.isclose(p, ref, rtol=PROB_RTOL, atol=PROB_ATOL)
            assert ok.all(), f"{name} rows {r0}..{r1}: {np.argwhere(~ok)[:5]}"
            worst = max(worst, float(np.max(np.abs(p - ref) / np.maximum(ref, 1e-30))))
    log(f"  largest relative difference {worst:.2e}")


def test_verify_probabilities_match_the_rebuilt_rows():
    """The verify's p_i(x_i), q_i(x_i) are the rebuilt rows' values at the draft tokens."""
    s = make_sample_inputs(3, 0)
    B, K, V = s.shape
    t = sample_tensors(s, DEV)
    out = rsv.verify_sample(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"],
                            want_probs=True)
    mt, St = rsv.row_stats(t["target"][:, :K].reshape(-1, V).contiguous(), s.temperature)
    mq, Sq = rsv.row_stats(t["draft"].reshape(-1, V), s.temperature)
    torch.cuda.synchronize()
    x = s.draft_tokens.reshape(-1)
    idx = np.arange(B * K)
    xt = s.target_f32()[:, :K].reshape(-1, V)[idx, x]
    xq = s.draft_f32().reshape(-1, V)[idx, x]
    c = _c32(s.temperature)
    pt = np.exp2(xt.astype(np.float64) * float(c) - (mt.cpu().numpy() * c).astype(np.float32)) / St.cpu().numpy()
    pq = np.exp2(xq.astype(np.float64) * float(c) - (mq.cpu().numpy() * c).astype(np.float32)) / Sq.cpu().numpy()
    probs = out.probs.cpu().numpy().reshape(-1, 2)
    assert np.allclose(probs[:, 0], pt, rtol=1e-5, atol=1e-7)
    assert np.allclose(probs[:, 1], pq, rtol=1e-5, atol=1e-7)


def test_row_stats_edge_rows():
    """Rows with -inf entries, one finite entry, no finite entry, and V below one 16-byte vector."""
    rows = np.array([[0.0, -np.inf, 2.0, -np.inf, 1.0],
                     [-np.inf, -np.inf, 3.5, -np.inf, -np.inf],
                     [-np.inf] * 5,
                     [1.0, 1.0, 1.0, 1.0, 1.0]], dtype=np.float32)
    for dtype in (torch.float32, torch.bfloat16):
        x = torch.from_numpy(rows).to(dtype).to(DEV)
        m, S = rsv.row_stats(x, 0.8)
        torch.cuda.synchronize()
        m, S = m.cpu().numpy(), S.cpu().numpy()
        assert m[2] == -np.inf and S[2] == 0.0
        xr = x.float().cpu().numpy()
        for r in (0, 1, 3):
            p = rebuilt(xr[r:r + 1], m[r:r + 1], S[r:r + 1], 0.8)[0]
            assert np.allclose(p, oracle.softmax64(xr[r], 0.8), rtol=1e-6, atol=1e-12)
