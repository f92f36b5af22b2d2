"""Every entry point captured in a HIP graph replays to its eager result (needs an MI355X).

The bench launches every leg from graphs; here each capture is replayed several
times with the program's own eager work and synchronisations between replays, and
every replay is compared bit for bit with the eager call on the same inputs. The
stateful n-gram pools are compared with the oracle after every replay (each replay
inserts the captured n-grams again).
"""
import numpy as np
import pytest
import torch

import rejection_sampling_verify_sample_amd as rsv
from oracle import ngram
from workloads import make_filter_params, make_greedy_inputs, make_ngram_sample_inputs, make_sample_inputs
from workloads.ngram import lookup_tokens, ngram_steps
from workloads.torch_io import greedy_tensors, sample_tensors

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"


def log(msg):
    print(f"[gpu-graphs] {msg}", flush=True)


def capture(fn):
    """fn() once on a side stream (allocations settle), then captured."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def replay_and_check(g, outs, want, fill=-7, reps=4, noise=None):
    for rep in range(reps):
        for o in outs:
            o.fill_(fill)
        if noise is not None:
            _ = (noise.float().sum() * 0).item()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o, w), f"replay {rep}"


def test_greedy_graph():
    log("greedy")
    g5 = make_greedy_inputs(1, B=8, G=5, N=4, V=20000)
    gt = greedy_tensors(g5, DEV)
    eager = rsv.verify_greedy(gt["logits"], gt["cand"])
    B, G, N, V = gt["logits"].shape
    ws = torch.zeros(rsv.greedy_workspace_size(B, G, N, V), dtype=torch.uint8, device=DEV)
    ot = torch.empty((B, N), dtype=torch.int32, device=DEV)
    ol = torch.empty((B,), dtype=torch.int32, device=DEV)
    ob = torch.empty((B,), dtype=torch.int32, device=DEV)
    g = capture(lambda: rsv.verify_greedy(gt["logits"], gt["cand"], out_tokens=ot, out_accept_len=ol, out_best=ob,
                                          workspace=ws))
    torch.cuda.synchronize()
    replay_and_check(g, [ot, ol, ob], [eager.tokens, eager.accept_len, eager.best], noise=gt["logits"])


@pytest.mark.parametrize("k,p", [(50, 0.9), (0, 0.9), (200, 1.0)])
def test_filtered_graph(k, p):
    log(f"filtered k={k} p={p}")
    s = make_sample_inputs(3, 1, B=8, V=40000)
    t = sample_tensors(s, DEV)
    B, K = s.draft_tokens.shape
    V = s.shape[2]
    fk, fp = make_filter_params(B, top_k=k, top_p=p)
    tk, tp = torch.from_numpy(fk).to(DEV), torch.from_numpy(fp).to(DEV)
    eager = rsv.verify_sample_filtered(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"],
                                       tk, tp, want_kept=True)
    ws = torch.zeros(rsv.sample_filtered_workspace_size(B, K, V), dtype=torch.uint8, device=DEV)
    ot = torch.empty((B, K + 1), dtype=torch.int32, device=DEV)
    on = torch.empty((B,), dtype=torch.int32, device=DEV)
    okept = torch.empty((B, 2 * K + 1), dtype=torch.int32, device=DEV)
    g = capture(lambda: rsv.verify_sample_filtered(t["target"], t["draft"], t["draft_tokens"], t["uniforms"],
                                                   t["temperature"], tk, tp, out_tokens=ot, out_num_accepted=on,
                                                   out_kept=okept, workspace=ws))
    torch.cuda.synchronize()
    replay_and_check(g, [ot, on, okept], [eager.tokens, eager.num_accepted, eager.kept], noise=t["target"])


def test_staged_graph():
    log("staged")
    s = make_sample_inputs(3, 2, B=8, V=30000)
    t = sample_tensors(s, DEV)
    B, K = s.draft_tokens.shape
    stages = [3, K]
    eager = rsv.verify_sample_staged(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"],
                                     stages)
    ws = torch.zeros(rsv.sample_workspace_size(B, K, s.shape[2]), dtype=torch.uint8, device=DEV)
    ot = torch.empty((B, K + 1), dtype=torch.int32, device=DEV)
    on = torch.empty((B,), dtype=torch.int32, device=DEV)
    g = capture(lambda: rsv.verify_sample_staged(t["target"], t["draft"], t["draft_tokens"], t["uniforms"],
                                                 t["temperature"], stages, out_tokens=ot, out_num_accepted=on,
                                                 workspace=ws))
    torch.cuda.synchronize()
    replay_and_check(g, [ot, on], [eager.tokens, eager.num_accepted], noise=t["target"])


def test_ngram_sample_graph():
    log("n-gram sampling")
    ns = make_ngram_sample_inputs(1, B=6, G=4, N=4, V=20000)
    lg = torch.from_numpy(ns.logits).to(DEV).view(torch.bfloat16)
    cand = torch.from_numpy(ns.cand).to(DEV)
    uni = torch.from_numpy(ns.uniforms).to(DEV)
    eager = rsv.verify_ngram_sample(lg, cand, uni, ns.temperature)
    B, G, N, V = ns.shape
    ws = torch.zeros(rsv.ngram_sample_workspace_size(B, G, N, V), dtype=torch.uint8, device=DEV)
    ot = torch.empty((B, N), dtype=torch.int32, device=DEV)
    ol = torch.empty((B,), dtype=torch.int32, device=DEV)
    orow = torch.empty((B,), dtype=torch.int32, device=DEV)
    g = capture(lambda: rsv.verify_ngram_sample(lg, cand, uni, ns.temperature, out_tokens=ot, out_accept_len=ol,
                                                out_rows=orow, workspace=ws))
    torch.cuda.synchronize()
    replay_and_check(g, [ot, ol, orow], [eager.tokens, eager.accept_len, eager.rows], noise=lg)


@pytest.mark.parametrize("kind", ["direct", "hashed"])
def test_pool_graph(kind):
    """insert + lookup captured once; every replay inserts the same n-grams again, and the
    lookups are compared with the oracle fed the same sequence of inserts."""
    log(f"pool {kind}")
    B, W, N, V, G = 6, 12, 4, 300, 3
    st = ngram_steps(29, 1, B, W, N, V, hot=0.6, n_hot=4, repeat=0.3, bad=0.1)[0]
    last = lookup_tokens(2, B, V, [st])
    if kind == "direct":
        pool = rsv.NgramPool(B, V, G, N, DEV)
        opools = ngram.new_pools(B, V, G, N)
    else:
        pool = rsv.NgramCache(B, V, G, N, 2, 2, DEV)
        opools = ngram.new_caches(B, V, G, N, 2, 2)
    grams = torch.from_numpy(st).to(DEV)
    lt = torch.from_numpy(last).to(DEV)
    sk = torch.empty((B,), dtype=torch.int32, device=DEV)
    cand = torch.empty((B, G, N - 1), dtype=torch.int32, device=DEV)
    count = torch.empty((B,), dtype=torch.int32, device=DEV)

    def step():
        pool.insert(grams, out_skipped=sk)
        pool.lookup(lt, out_cand=cand, out_count=count)

    g = capture(step)  # the side-stream call and the capture itself: one insert so far
    ngram.pool_insert(opools, st)
    torch.cuda.synchronize()
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        osk = ngram.pool_insert(opools, st)
        ocand, ocount = ngram.pool_lookup(opools, last)
        assert np.array_equal(sk.cpu().numpy(), osk), f"replay {rep}"
        assert np.array_equal(cand.cpu().numpy(), ocand) and np.array_equal(count.cpu().numpy(), ocount), \
            f"replay {rep}"
        if kind == "hashed":
            clocks, _ = pool.entries()
            assert clocks == [c.clock for c in opools], f"replay {rep}"
