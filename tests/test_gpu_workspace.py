"""The verify's workspace needs no initialisation (needs an MI355X).

The C ABI promises that a workspace carries partial results only between the
launches of one call: whatever it holds before a call (zeros, 0xFF, random bytes,
or what other entry points and other shapes left in it) must not change the
outputs. spec_verify_sample reads its pass-1 partials, decisions and chunk masses
only after the launch that writes them in the same call.
"""
import numpy as np
import pytest
import torch

import rejection_sampling_verify_sample_amd as rsv
from workloads import make_filter_params, make_greedy_inputs, make_sample_inputs
from workloads.torch_io import greedy_tensors, sample_tensors

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"


def log(msg):
    print(f"[gpu-workspace] {msg}", flush=True)


def _run(t, workspace=None):
    out = rsv.verify_sample(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"],
                            want_probs=True, workspace=workspace)
    torch.cuda.synchronize()
    return out.tokens.cpu().numpy(), out.num_accepted.cpu().numpy(), out.probs.cpu().numpy()


@pytest.mark.parametrize("fill", ["zeros", "ones", "random", "others"])
def test_workspace_contents_do_not_matter(fill):
    """A workspace full of zeros, of 0xFF, of random bytes, or last written by other
    entry points (greedy, filtered, staged, a different shape) gives the same outputs
    as a fresh one, call after call."""
    s = make_sample_inputs(3, 5, B=8, V=30000)
    log(f"{fill}: {s.name}")
    t = sample_tensors(s, DEV)
    B, K, V = s.shape
    ref = _run(t)
    nbytes = max(rsv.sample_workspace_size(B, K, V), rsv.sample_filtered_workspace_size(B, K, V), 1 << 22)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    if fill == "zeros":
        ws.zero_()
    elif fill == "ones":
        ws.fill_(255)
    elif fill == "random":
        ws.copy_(torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=torch.Generator().manual_seed(3)))
    else:
        g = make_greedy_inputs(0, B=4, G=3, N=5, V=3001)
        gt = greedy_tensors(g, DEV)
        rsv.verify_greedy(gt["logits"], gt["cand"], workspace=ws)
        k, p = make_filter_params(B, 0, top_k=50, top_p=0.9)
        rsv.verify_sample_filtered(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"],
                                   torch.from_numpy(k).to(DEV), torch.from_numpy(p).to(DEV), workspace=ws)
        rsv.verify_sample_staged(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"],
                                 [2, 8], workspace=ws)
        s2 = make_sample_inputs(3, 6, B=4, V=30000)
        _run(sample_tensors(s2, DEV), workspace=ws)
    for rep in range(3):
        got = _run(t, workspace=ws)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), f"{fill} call {rep}"
        assert np.array_equal(got[2], ref[2], equal_nan=True), f"{fill} call {rep}"


def test_alternating_inputs_on_one_workspace():
    """Two different rounds alternating on one workspace: nothing one call leaves is
    taken for the next call's."""
    sa = make_sample_inputs(3, 7, B=16, V=20000)
    sb = make_sample_inputs(3, 8, B=16, V=20000)
    ta, tb = sample_tensors(sa, DEV), sample_tensors(sb, DEV)
    ws = torch.zeros(rsv.sample_workspace_size(16, 8, 20000), dtype=torch.uint8, device=DEV)
    ra, rb = _run(ta), _run(tb)
    for _ in range(4):
        for t, r in ((ta, ra), (tb, rb)):
            got = _run(t, workspace=ws)
            assert np.array_equal(got[0], r[0]) and np.array_equal(got[1], r[1])


def test_batches_in_flight_on_streams():
    """Independent rounds in flight at once, one stream and one workspace each (the way a
    serving loop overlaps one batch's pass 2 and draw with another's pass 1): queued
    several times over without waiting, every stream's outputs equal the round's own
    outputs run alone."""
    specs = [make_sample_inputs(3, 20 + i, B=16, V=20000) for i in range(3)]
    ts = [sample_tensors(s, DEV) for s in specs]
    refs = [_run(t) for t in ts]
    streams = [torch.cuda.Stream() for _ in ts]
    wss = [torch.zeros(rsv.sample_workspace_size(16, 8, 20000), dtype=torch.uint8, device=DEV) for _ in ts]
    outs = [(torch.empty((16, 9), dtype=torch.int32, device=DEV), torch.empty((16,), dtype=torch.int32, device=DEV))
            for _ in ts]
    log("3 streams")
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    got = []
    for rep in range(6):
        for i, (t, st) in enumerate(zip(ts, streams)):
            with torch.cuda.stream(st):
                o = rsv.verify_sample(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"],
                                      out_tokens=outs[i][0], out_num_accepted=outs[i][1], workspace=wss[i])
                got.append((i, o.tokens.clone(), o.num_accepted.clone()))  # copies queued on the same stream
    torch.cuda.synchronize()
    for i, tok, n in got:
        assert np.array_equal(tok.cpu().numpy(), refs[i][0]) and np.array_equal(n.cpu().numpy(), refs[i][1]), i


def test_host_threads_each_on_their_stream():
    """Four host threads, each with its own stream and round, call the verify at once
    (ctypes releases the interpreter lock during the calls) with the binding's own
    per-stream workspaces: every call's outputs equal the round's outputs run alone."""
    import threading

    specs = [make_sample_inputs(3, 30 + i, B=8, V=20000) for i in range(4)]
    ts = [sample_tensors(s, DEV) for s in specs]
    refs = [_run(t) for t in ts]
    errors, done = [], []
    log("4 threads")

    def work(i):
        try:
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.default_stream())
            t = ts[i]
            with torch.cuda.stream(st):
                outs = [rsv.verify_sample(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"])
                        for _ in range(5)]
            st.synchronize()
            for o in outs:
                if not (np.array_equal(o.tokens.cpu().numpy(), refs[i][0])
                        and np.array_equal(o.num_accepted.cpu().numpy(), refs[i][1])):
                    errors.append(i)
            done.append(i)
        except Exception as e:  # reported below, in the test's own thread
            errors.append((i, repr(e)))

    torch.cuda.synchronize()
    th = [threading.Thread(target=work, args=(i,)) for i in range(4)]
    for x in th:
        x.start()
    for x in th:
        x.join(timeout=120)
    assert not errors, errors
    assert sorted(done) == [0, 1, 2, 3]
