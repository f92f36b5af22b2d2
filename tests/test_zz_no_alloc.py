"""spec_verify_sample_noalloc against spec_verify_sample (needs an MI355X).

The allocation-free entry point runs the same kernels on the library's fixed
device scratch, so its outputs must equal spec_verify_sample's bit for bit.
Two calls in a row, the second on a smaller input, check that the scratch left
by one call does not leak into the next.
"""
import numpy as np
import pytest
import torch

import rejection_sampling_verify_sample_amd as rsv
from workloads import make_sample_inputs
from workloads.torch_io import sample_tensors

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"


def _both(s):
    t = sample_tensors(s, DEV)
    B, K, _ = s.shape
    ref = rsv.verify_sample(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"],
                            want_probs=True)
    ot = torch.full((B, K + 1), -7, dtype=torch.int32, device=DEV)
    on = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    op = torch.full((B, K, 2), -7.0, dtype=torch.float32, device=DEV)
    rsv.verify_sample_noalloc(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"],
                              out_tokens=ot, out_num_accepted=on, out_probs=op)
    torch.cuda.synchronize()
    return ref, (ot, on, op)


def test_noalloc_matches_verify_sample_on_consecutive_calls():
    for cfg, kw in ((3, {}), (1, {}), (2, dict(B=5, V=9001)), (4, dict(B=16, V=40003))):
        s = make_sample_inputs(cfg, 1, **kw)
        print(f"[no-alloc] case {s.name}", flush=True)
        ref, (ot, on, op) = _both(s)
        assert torch.equal(ot, ref.tokens) and torch.equal(on, ref.num_accepted)
        assert np.array_equal(op.cpu().numpy(), ref.probs.cpu().numpy(), equal_nan=True)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    assert rsv.sample_workspace_size(4096, 8, 128256) > rsv.lib().spec_verify_sample_noalloc_max_bytes()
    st = rsv.lib().spec_verify_sample_noalloc(None, None, 1, None, None, 4096, 8, 128256, 1.0, None, None, None,
                                              None)
    assert st == -5  # SPEC_ERR_WORKSPACE, before any pointer is looked at
