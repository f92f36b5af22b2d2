"""Move generated inputs into torch tensors (bf16 bit patterns become torch.bfloat16)."""
from __future__ import annotations

import numpy as np
import torch

from .configs import BF16, GreedyInputs, SampleInputs


def logits_tensor(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    if dtype == BF16:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def sample_tensors(s: SampleInputs, device) -> dict:
    return dict(target=logits_tensor(s.target, s.dtype, device), draft=logits_tensor(s.draft, s.dtype, device),
                draft_tokens=torch.from_numpy(np.ascontiguousarray(s.draft_tokens, dtype=np.int32)).to(device),
                uniforms=torch.from_numpy(np.ascontiguousarray(s.uniforms, dtype=np.float32)).to(device),
                temperature=s.temperature)


def greedy_tensors(g: GreedyInputs, device) -> dict:
    return dict(logits=logits_tensor(g.logits, g.dtype, device),
                cand=torch.from_numpy(np.ascontiguousarray(g.cand, dtype=np.int32)).to(device))
