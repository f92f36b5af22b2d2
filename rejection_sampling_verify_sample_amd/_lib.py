"""ctypes binding of libspecverify.so: argument marshalling only.

Every step of the verify computation runs in the HIP library. This module
checks tensor devices, dtypes, shapes and contiguity, allocates outputs and a
per-stream workspace through PyTorch, and passes raw pointers plus the current
HIP stream. If the library has not been built it raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading
from dataclasses import dataclass

import torch

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libspecverify.so")

SPEC_F32 = 0
SPEC_BF16 = 1
SPEC_MAX_K = 64

_c_void_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_u64 = ctypes.c_uint64
_size_t = ctypes.c_size_t

_SIGNATURES = {
    "spec_abi_version": (_i32, []),
    "spec_status_string": (ctypes.c_char_p, [_i32]),
    "spec_verify_sample_workspace_size": (_size_t, [_i32, _i32, _i32]),
    "spec_verify_sample": (_i32, [_c_void_p, _c_void_p, _i32, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                  ctypes.c_float, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size_t,
                                  _c_void_p]),
    "spec_verify_sample_phases": (_i32, [_c_void_p, _c_void_p, _i32, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                         ctypes.c_float, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size_t,
                                         _c_void_p, _i32]),
    "spec_verify_sample_staged": (_i32, [_c_void_p, _c_void_p, _i32, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                         ctypes.c_float, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size_t,
                                         _c_void_p, _c_void_p, _i32]),
    "spec_verify_sample_filtered_workspace_size": (_size_t, [_i32, _i32, _i32]),
    "spec_verify_sample_filtered": (_i32, [_c_void_p, _c_void_p, _i32, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                           ctypes.c_float, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size_t,
                                           _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "spec_verify_sample_filtered_phases": (_i32, [_c_void_p, _c_void_p, _i32, _c_void_p, _c_void_p, _i32, _i32,
                                                  _i32, ctypes.c_float, _c_void_p, _c_void_p, _c_void_p,
                                                  _c_void_p, _size_t, _c_void_p, _c_void_p, _c_void_p,
                                                  _c_void_p, _i32]),
    "spec_row_stats_workspace_size": (_size_t, [_i32, _i32]),
    "spec_row_stats": (_i32, [_c_void_p, _i32, _i32, _i32, ctypes.c_float, _c_void_p, _c_void_p, _c_void_p, _size_t,
                              _c_void_p]),
    "spec_verify_sample_noalloc_max_bytes": (_size_t, []),
    "spec_verify_sample_noalloc": (_i32, [_c_void_p, _c_void_p, _i32, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                          ctypes.c_float, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "spec_verify_greedy_workspace_size": (_size_t, [_i32, _i32, _i32, _i32]),
    "spec_verify_greedy": (_i32, [_c_void_p, _i32, _c_void_p, _i32, _i32, _i32, _i32, _c_void_p, _c_void_p,
                                  _c_void_p, _c_void_p, _size_t, _c_void_p]),
    "spec_fill_uniforms": (_i32, [_u64, _u64, _i32, _i32, _c_void_p, _c_void_p]),
    "spec_verify_ngram_sample_workspace_size": (_size_t, [_i32, _i32, _i32, _i32]),
    "spec_verify_ngram_sample": (_i32, [_c_void_p, _i32, _c_void_p, _c_void_p, _i32, _i32, _i32, _i32,
                                        ctypes.c_float, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size_t,
                                        _c_void_p]),
    "spec_ngram_pool_bytes": (_size_t, [_i32, _i32, _i32, _i32]),
    "spec_ngram_pool_init": (_i32, [_c_void_p, _size_t, _i32, _i32, _i32, _i32, _c_void_p]),
    "spec_ngram_pool_insert": (_i32, [_c_void_p, _size_t, _i32, _i32, _i32, _i32, _c_void_p, _i32, _c_void_p,
                                      _c_void_p]),
    "spec_ngram_pool_lookup": (_i32, [_c_void_p, _size_t, _i32, _i32, _i32, _i32, _c_void_p, _c_void_p, _c_void_p,
                                      _c_void_p]),
    "spec_ngram_cache_bytes": (_size_t, [_i32, _i32, _i32, _i32, _i32]),
    "spec_ngram_cache_init": (_i32, [_c_void_p, _size_t, _i32, _i32, _i32, _i32, _i32, _c_void_p]),
    "spec_ngram_cache_insert": (_i32, [_c_void_p, _size_t, _i32, _i32, _i32, _i32, _i32, _i32, _c_void_p, _i32,
                                       _c_void_p, _c_void_p]),
    "spec_ngram_cache_lookup": (_i32, [_c_void_p, _size_t, _i32, _i32, _i32, _i32, _i32, _i32, _c_void_p, _c_void_p,
                                       _c_void_p, _c_void_p]),
}

_lib = None
_lib_lock = threading.Lock()


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    with _lib_lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built; run `python -m rejection_sampling_verify_sample_amd.build`"
                                   " (hipcc, gfx950). There is no fallback path.")
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGNATURES.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().spec_status_string(int(status)).decode()


def abi_version() -> int:
    return int(lib().spec_abi_version())


def sample_workspace_size(B: int, K: int, V: int) -> int:
    return int(lib().spec_verify_sample_workspace_size(B, K, V))


def sample_filtered_workspace_size(B: int, K: int, V: int) -> int:
    return int(lib().spec_verify_sample_filtered_workspace_size(B, K, V))


def greedy_workspace_size(B: int, G: int, N: int, V: int) -> int:
    return int(lib().spec_verify_greedy_workspace_size(B, G, N, V))


# ------------------------------------------------------------------ tensors and streams

def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    if t.dtype == torch.float32:
        return SPEC_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _check(t: torch.Tensor, name: str, device: torch.device, dtype=None, shape=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_handle(stream, device: torch.device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


_workspaces: dict[tuple[int, int], torch.Tensor] = {}
_ws_lock = threading.Lock()


def workspace_for(device: torch.device, stream_handle: int, nbytes: int) -> torch.Tensor:
    """A workspace reused by every call on one (device, stream); it needs no initialisation."""
    key = (device.index, stream_handle)
    with _ws_lock:
        ws = _workspaces.get(key)
        if ws is None or ws.numel() < nbytes:
            ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
            _workspaces[key] = ws
        return ws


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# ------------------------------------------------------------------ entry points

@dataclass
class SampleOutputs:
    tokens: torch.Tensor        # [B, K+1] int32
    num_accepted: torch.Tensor  # [B] int32
    probs: torch.Tensor | None  # [B, K, 2] float32
    kept: torch.Tensor | None = None  # [B, 2K+1] int32 (filtered verify only)


PHASE_ROW_STATS, PHASE_ACCEPT, PHASE_MASS, PHASE_DRAW, PHASE_ALL = 1, 2, 4, 8, 15


def verify_sample(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor, uniforms: torch.Tensor,
                  temperature: float, *, out_tokens: torch.Tensor | None = None,
                  out_num_accepted: torch.Tensor | None = None, out_probs: torch.Tensor | None = None,
                  want_probs: bool = False, workspace: torch.Tensor | None = None, stream=None,
                  phases: int = PHASE_ALL) -> SampleOutputs:
    """spec_verify_sample on torch tensors (layouts as in include/spec_verify.h). Asynchronous on `stream`.

    `phases` (a mask of PHASE_*) runs only some of the four launches, through
    spec_verify_sample_phases; later phases read what earlier ones of the same
    arguments left in the workspace.
    """
    return _verify_sample(target, draft, draft_tokens, uniforms, temperature, out_tokens, out_num_accepted,
                          out_probs, want_probs, workspace, stream, phases, None)


def row_stats(logits: torch.Tensor, temperature: float, *, workspace: torch.Tensor | None = None,
              stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """spec_row_stats: (row maximum m [rows] float32, denominator S [rows] float64) of logits [rows, V].

    Row r's law is p_v = 2^(x_v * c - fl32(m * c)) / S with c = fl32(log2(e) / T).
    """
    if logits.dim() != 2:
        raise ValueError("logits must be [rows, V]")
    rows, V = logits.shape
    dev = logits.device
    _check(logits, "logits", dev)
    code = _dtype_code(logits)
    out_max = torch.empty((rows,), dtype=torch.float32, device=dev)
    out_sum = torch.empty((rows,), dtype=torch.float64, device=dev)
    sh = _stream_handle(stream, dev)
    nbytes = int(lib().spec_row_stats_workspace_size(rows, V))
    if nbytes == 0 and rows > 0:
        raise SpecVerifyError(-2, "spec_row_stats_workspace_size")
    if workspace is None:
        workspace = workspace_for(dev, sh, nbytes)
    _check(workspace, "workspace", dev, torch.uint8)
    st = lib().spec_row_stats(_ptr(logits), code, rows, V, float(temperature), _ptr(out_max), _ptr(out_sum),
                              _ptr(workspace), workspace.numel(), ctypes.c_void_p(sh))
    if st != 0:
        raise SpecVerifyError(st, "spec_row_stats")
    return out_max, out_sum


def verify_sample_noalloc(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
                          uniforms: torch.Tensor, temperature: float, *, out_tokens: torch.Tensor,
                          out_num_accepted: torch.Tensor, out_probs: torch.Tensor | None = None,
                          stream=None) -> SampleOutputs:
    """spec_verify_sample_noalloc: verify_sample with the library's fixed device scratch as workspace.

    The caller passes every output (nothing is allocated here either); sizes whose
    workspace exceeds spec_verify_sample_noalloc_max_bytes() are refused.
    """
    if target.dim() != 3:
        raise ValueError("target must be [B, K+1, V]")
    B, K1, V = target.shape
    K = K1 - 1
    dev = target.device
    _check(target, "target", dev)
    code = _dtype_code(target)
    _check(draft, "draft", dev, target.dtype, (B, K, V))
    _check(draft_tokens, "draft_tokens", dev, torch.int32, (B, K))
    _check(uniforms, "uniforms", dev, torch.float32, (B, K + 1, 2))
    _check(out_tokens, "out_tokens", dev, torch.int32, (B, K + 1))
    _check(out_num_accepted, "out_num_accepted", dev, torch.int32, (B,))
    if out_probs is not None:
        _check(out_probs, "out_probs", dev, torch.float32, (B, K, 2))
    sh = _stream_handle(stream, dev)
    st = lib().spec_verify_sample_noalloc(_ptr(target), _ptr(draft), code, _ptr(draft_tokens), _ptr(uniforms), B,
                                          K, V, float(temperature), _ptr(out_tokens), _ptr(out_num_accepted),
                                          _ptr(out_probs), ctypes.c_void_p(sh))
    if st != 0:
        raise SpecVerifyError(st, "spec_verify_sample_noalloc")
    return SampleOutputs(out_tokens, out_num_accepted, out_probs)


def verify_sample_staged(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
                         uniforms: torch.Tensor, temperature: float, stages, *,
                         out_tokens: torch.Tensor | None = None, out_num_accepted: torch.Tensor | None = None,
                         out_probs: torch.Tensor | None = None, want_probs: bool = False,
                         workspace: torch.Tensor | None = None, stream=None) -> SampleOutputs:
    """spec_verify_sample_staged: the verify with early exit over pass-1 stages.

    `stages` lists the stage ends (strictly increasing draft positions, the last
    one K; empty when K = 0). Outputs equal verify_sample's, except that with
    more than one stage out_probs is NaN past the first rejection.
    """
    ends = [int(e) for e in stages]
    return _verify_sample(target, draft, draft_tokens, uniforms, temperature, out_tokens, out_num_accepted,
                          out_probs, want_probs, workspace, stream, PHASE_ALL, None, ends)


def verify_sample_filtered(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
                           uniforms: torch.Tensor, temperature: float, top_k: torch.Tensor | None,
                           top_p: torch.Tensor | None, *, out_tokens: torch.Tensor | None = None,
                           out_num_accepted: torch.Tensor | None = None, out_probs: torch.Tensor | None = None,
                           want_probs: bool = False, out_kept: torch.Tensor | None = None, want_kept: bool = False,
                           workspace: torch.Tensor | None = None, stream=None,
                           phases: int = PHASE_ALL) -> SampleOutputs:
    """spec_verify_sample_filtered: the verify on top-k / top-p filtered laws.

    top_k [B] int32 and top_p [B] float32 (device tensors, either may be None)
    hold the filter of each batch row; out_kept [B, 2K+1] the kept counts.
    """
    return _verify_sample(target, draft, draft_tokens, uniforms, temperature, out_tokens, out_num_accepted,
                          out_probs, want_probs, workspace, stream, phases, (top_k, top_p, out_kept, want_kept))


def _verify_sample(target, draft, draft_tokens, uniforms, temperature, out_tokens, out_num_accepted, out_probs,
                   want_probs, workspace, stream, phases, filt, stages=None) -> SampleOutputs:
    if target.dim() != 3:
        raise ValueError("target must be [B, K+1, V]")
    B, K1, V = target.shape
    K = K1 - 1
    dev = target.device
    _check(target, "target", dev)
    code = _dtype_code(target)
    _check(draft, "draft", dev, target.dtype, (B, K, V))
    _check(draft_tokens, "draft_tokens", dev, torch.int32, (B, K))
    _check(uniforms, "uniforms", dev, torch.float32, (B, K + 1, 2))
    if out_tokens is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    _check(out_tokens, "out_tokens", dev, torch.int32, (B, K + 1))
    if out_num_accepted is None:
        out_num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(out_num_accepted, "out_num_accepted", dev, torch.int32, (B,))
    if out_probs is None and want_probs:
        out_probs = torch.empty((B, K, 2), dtype=torch.float32, device=dev)
    if out_probs is not None:
        _check(out_probs, "out_probs", dev, torch.float32, (B, K, 2))
    out_kept = None
    if filt is not None:
        top_k, top_p, out_kept, want_kept = filt
        if top_k is not None:
            _check(top_k, "top_k", dev, torch.int32, (B,))
        if top_p is not None:
            _check(top_p, "top_p", dev, torch.float32, (B,))
        if out_kept is None and want_kept:
            out_kept = torch.empty((B, 2 * K + 1), dtype=torch.int32, device=dev)
        if out_kept is not None:
            _check(out_kept, "out_kept", dev, torch.int32, (B, 2 * K + 1))
    sh = _stream_handle(stream, dev)
    nbytes = sample_workspace_size(B, K, V) if filt is None else sample_filtered_workspace_size(B, K, V)
    if nbytes == 0 and B > 0:
        raise SpecVerifyError(-9 if filt is not None and V > (1 << 24) else -2, "workspace size query")
    if workspace is None:
        workspace = workspace_for(dev, sh, nbytes)
    _check(workspace, "workspace", dev, torch.uint8)
    args = (_ptr(target), _ptr(draft), code, _ptr(draft_tokens), _ptr(uniforms), B, K, V, float(temperature),
            _ptr(out_tokens), _ptr(out_num_accepted), _ptr(out_probs), _ptr(workspace), workspace.numel(),
            ctypes.c_void_p(sh))
    if filt is not None:
        fargs = (_ptr(filt[0]), _ptr(filt[1]), _ptr(out_kept))
        if phases == PHASE_ALL:
            st, where = lib().spec_verify_sample_filtered(*args, *fargs), "spec_verify_sample_filtered"
        else:
            st, where = (lib().spec_verify_sample_filtered_phases(*args, *fargs, int(phases)),
                         "spec_verify_sample_filtered_phases")
    elif stages is not None:
        arr = (ctypes.c_int32 * max(1, len(stages)))(*stages)
        st, where = lib().spec_verify_sample_staged(*args, arr, len(stages)), "spec_verify_sample_staged"
    elif phases == PHASE_ALL:
        st, where = lib().spec_verify_sample(*args), "spec_verify_sample"
    else:
        st, where = lib().spec_verify_sample_phases(*args, int(phases)), "spec_verify_sample_phases"
    if st != 0:
        raise SpecVerifyError(st, where)
    return SampleOutputs(out_tokens, out_num_accepted, out_probs, out_kept)


@dataclass
class GreedyOutputs:
    tokens: torch.Tensor      # [B, N] int32
    accept_len: torch.Tensor  # [B] int32
    best: torch.Tensor        # [B] int32


def verify_greedy(logits: torch.Tensor, cand: torch.Tensor, *, out_tokens: torch.Tensor | None = None,
                  out_accept_len: torch.Tensor | None = None, out_best: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, stream=None) -> GreedyOutputs:
    """spec_verify_greedy on torch tensors (layouts as in include/spec_verify.h). Asynchronous on `stream`."""
    if logits.dim() != 4:
        raise ValueError("logits must be [B, G, N, V]")
    B, G, N, V = logits.shape
    dev = logits.device
    _check(logits, "logits", dev)
    code = _dtype_code(logits)
    _check(cand, "cand", dev, torch.int32, (B, G, N - 1))
    if out_tokens is None:
        out_tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    if out_accept_len is None:
        out_accept_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if out_best is None:
        out_best = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(out_tokens, "out_tokens", dev, torch.int32, (B, N))
    _check(out_accept_len, "out_accept_len", dev, torch.int32, (B,))
    _check(out_best, "out_best", dev, torch.int32, (B,))
    sh = _stream_handle(stream, dev)
    nbytes = greedy_workspace_size(B, G, N, V)
    if nbytes == 0 and B > 0:
        raise SpecVerifyError(-2, "spec_verify_greedy_workspace_size")
    if workspace is None:
        workspace = workspace_for(dev, sh, nbytes)
    _check(workspace, "workspace", dev, torch.uint8)
    st = lib().spec_verify_greedy(_ptr(logits), code, _ptr(cand), B, G, N, V, _ptr(out_tokens),
                                  _ptr(out_accept_len), _ptr(out_best), _ptr(workspace), workspace.numel(),
                                  ctypes.c_void_p(sh))
    if st != 0:
        raise SpecVerifyError(st, "spec_verify_greedy")
    return GreedyOutputs(out_tokens, out_accept_len, out_best)


@dataclass
class NgramSampleOutputs:
    tokens: torch.Tensor      # [B, N] int32
    accept_len: torch.Tensor  # [B] int32
    rows: torch.Tensor        # [B] int32


def ngram_sample_workspace_size(B: int, G: int, N: int, V: int) -> int:
    return int(lib().spec_verify_ngram_sample_workspace_size(B, G, N, V))


def verify_ngram_sample(logits: torch.Tensor, cand: torch.Tensor, uniforms: torch.Tensor, temperature: float, *,
                        out_tokens: torch.Tensor | None = None, out_accept_len: torch.Tensor | None = None,
                        out_rows: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                        stream=None) -> NgramSampleOutputs:
    """spec_verify_ngram_sample: sampling verify of G greedy-drafted candidate n-grams.

    logits [B, G, N, V] (bf16 or fp32), cand [B, G, N-1] int32, uniforms [B, N, G+1] float32.
    """
    if logits.dim() != 4:
        raise ValueError("logits must be [B, G, N, V]")
    B, G, N, V = logits.shape
    dev = logits.device
    _check(logits, "logits", dev)
    code = _dtype_code(logits)
    _check(cand, "cand", dev, torch.int32, (B, G, N - 1))
    _check(uniforms, "uniforms", dev, torch.float32, (B, N, G + 1))
    if out_tokens is None:
        out_tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    if out_accept_len is None:
        out_accept_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if out_rows is None:
        out_rows = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(out_tokens, "out_tokens", dev, torch.int32, (B, N))
    _check(out_accept_len, "out_accept_len", dev, torch.int32, (B,))
    _check(out_rows, "out_rows", dev, torch.int32, (B,))
    sh = _stream_handle(stream, dev)
    nbytes = ngram_sample_workspace_size(B, G, N, V)
    if nbytes == 0 and B > 0:
        raise SpecVerifyError(-2, "spec_verify_ngram_sample_workspace_size")
    if workspace is None:
        workspace = workspace_for(dev, sh, nbytes)
    _check(workspace, "workspace", dev, torch.uint8)
    st = lib().spec_verify_ngram_sample(_ptr(logits), code, _ptr(cand), _ptr(uniforms), B, G, N, V,
                                        float(temperature), _ptr(out_tokens), _ptr(out_accept_len), _ptr(out_rows),
                                        _ptr(workspace), workspace.numel(), ctypes.c_void_p(sh))
    if st != 0:
        raise SpecVerifyError(st, "spec_verify_ngram_sample")
    return NgramSampleOutputs(out_tokens, out_accept_len, out_rows)


def fill_uniforms(seed: int, rnd: int, B: int, K: int, *, out: torch.Tensor | None = None,
                  device: torch.device | str | None = None, stream=None) -> torch.Tensor:
    """spec_fill_uniforms: the verify uniforms [B, K+1, 2] of one round, on the device."""
    if out is None:
        dev = torch.device(device if device is not None else "cuda")
        out = torch.empty((B, K + 1, 2), dtype=torch.float32, device=dev)
    _check(out, "out", out.device, torch.float32, (B, K + 1, 2))
    sh = _stream_handle(stream, out.device)
    st = lib().spec_fill_uniforms(int(seed) & (2 ** 64 - 1), int(rnd) & (2 ** 64 - 1), B, K, _ptr(out),
                                  ctypes.c_void_p(sh))
    if st != 0:
        raise SpecVerifyError(st, "spec_fill_uniforms")
    return out


# ------------------------------------------------------------------ n-gram pool

def ngram_pool_bytes(B: int, V: int, G: int, N: int) -> int:
    return int(lib().spec_ngram_pool_bytes(B, V, G, N))


class NgramPool:
    """The n-gram pools of B sequences (spec_ngram_pool_*), held in a device buffer PyTorch allocates.

    `buffer` is the pool memory, [B, V, G, N-1] int32 viewed from its bytes; it is
    emptied at construction. insert() and lookup() run on `stream` (default: the
    current stream).
    """

    def __init__(self, B: int, V: int, G: int, N: int, device="cuda", stream=None):
        self.B, self.V, self.G, self.N = int(B), int(V), int(G), int(N)
        self.device = torch.device(device)
        nbytes = ngram_pool_bytes(B, V, G, N)
        if nbytes == 0 and B > 0:
            raise SpecVerifyError(-2, "spec_ngram_pool_bytes")
        self.buffer = torch.empty(max(nbytes // 4, 1), dtype=torch.int32, device=self.device)
        self.nbytes = nbytes
        st = lib().spec_ngram_pool_init(_ptr(self.buffer), nbytes, B, V, G, N,
                                        ctypes.c_void_p(_stream_handle(stream, self.device)))
        if st != 0:
            raise SpecVerifyError(st, "spec_ngram_pool_init")

    def table(self) -> torch.Tensor:
        """The pool memory as [B, V, G, N-1] int32 (a view, for inspection)."""
        return self.buffer[: self.B * self.V * self.G * (self.N - 1)].view(self.B, self.V, self.G, self.N - 1)

    def insert(self, ngrams: torch.Tensor, *, out_skipped: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """Insert ngrams [B, W, N] int32 (window order); returns the skipped counts [B]."""
        if ngrams.dim() != 3:
            raise ValueError("ngrams must be [B, W, N]")
        W = ngrams.shape[1]
        _check(ngrams, "ngrams", self.device, torch.int32, (self.B, W, self.N))
        if out_skipped is None:
            out_skipped = torch.empty((self.B,), dtype=torch.int32, device=self.device)
        _check(out_skipped, "out_skipped", self.device, torch.int32, (self.B,))
        st = lib().spec_ngram_pool_insert(_ptr(self.buffer), self.nbytes, self.B, self.V, self.G, self.N,
                                          _ptr(ngrams), W, _ptr(out_skipped),
                                          ctypes.c_void_p(_stream_handle(stream, self.device)))
        if st != 0:
            raise SpecVerifyError(st, "spec_ngram_pool_insert")
        return out_skipped

    def lookup(self, last_tokens: torch.Tensor, *, out_cand: torch.Tensor | None = None,
               out_count: torch.Tensor | None = None, stream=None) -> tuple[torch.Tensor, torch.Tensor]:
        """Candidates [B, G, N-1] (newest first, -1 past the count) and counts [B] for each last token [B]."""
        _check(last_tokens, "last_tokens", self.device, torch.int32, (self.B,))
        if out_cand is None:
            out_cand = torch.empty((self.B, self.G, self.N - 1), dtype=torch.int32, device=self.device)
        if out_count is None:
            out_count = torch.empty((self.B,), dtype=torch.int32, device=self.device)
        _check(out_cand, "out_cand", self.device, torch.int32, (self.B, self.G, self.N - 1))
        _check(out_count, "out_count", self.device, torch.int32, (self.B,))
        st = lib().spec_ngram_pool_lookup(_ptr(self.buffer), self.nbytes, self.B, self.V, self.G, self.N,
                                          _ptr(last_tokens), _ptr(out_cand), _ptr(out_count),
                                          ctypes.c_void_p(_stream_handle(stream, self.device)))
        if st != 0:
            raise SpecVerifyError(st, "spec_ngram_pool_lookup")
        return out_cand, out_count


# ------------------------------------------------------------------ hashed n-gram pool

def ngram_cache_bytes(B: int, sets: int, ways: int, G: int, N: int) -> int:
    return int(lib().spec_ngram_cache_bytes(B, sets, ways, G, N))


class NgramCache:
    """The hashed n-gram pools of B sequences (spec_ngram_cache_*): per sequence `sets` sets
    (a power of two) of `ways` keys, the least recently inserted key of a full set evicted.

    Same insert() / lookup() as NgramPool. `buffer` is the table memory (int32), emptied at
    construction; sequence b starts at int32 b * seq_elems: the clock, three zero words,
    then set s at 4 + s * set_elems: keys[ways], stamps[ways] (uint32 bits), slots[ways][G][N-1].
    """

    def __init__(self, B: int, V: int, G: int, N: int, sets: int, ways: int, device="cuda", stream=None):
        self.B, self.V, self.G, self.N, self.sets, self.ways = int(B), int(V), int(G), int(N), int(sets), int(ways)
        self.device = torch.device(device)
        nbytes = ngram_cache_bytes(B, sets, ways, G, N)
        if nbytes == 0 and B > 0:
            raise SpecVerifyError(-2, "spec_ngram_cache_bytes")
        self.set_elems = 2 * self.ways + self.ways * self.G * (self.N - 1)
        self.seq_elems = (4 + self.sets * self.set_elems + 3) // 4 * 4
        self.buffer = torch.empty(max(nbytes // 4, 1), dtype=torch.int32, device=self.device)
        self.nbytes = nbytes
        st = lib().spec_ngram_cache_init(_ptr(self.buffer), nbytes, B, sets, ways, G, N,
                                         ctypes.c_void_p(_stream_handle(stream, self.device)))
        if st != 0:
            raise SpecVerifyError(st, "spec_ngram_cache_init")

    def _sizes(self):
        return self.B, self.V, self.sets, self.ways, self.G, self.N

    def insert(self, ngrams: torch.Tensor, *, out_skipped: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """Insert ngrams [B, W, N] int32 (window order); returns the skipped counts [B]."""
        if ngrams.dim() != 3:
            raise ValueError("ngrams must be [B, W, N]")
        W = ngrams.shape[1]
        _check(ngrams, "ngrams", self.device, torch.int32, (self.B, W, self.N))
        if out_skipped is None:
            out_skipped = torch.empty((self.B,), dtype=torch.int32, device=self.device)
        _check(out_skipped, "out_skipped", self.device, torch.int32, (self.B,))
        st = lib().spec_ngram_cache_insert(_ptr(self.buffer), self.nbytes, *self._sizes(), _ptr(ngrams), W,
                                           _ptr(out_skipped), ctypes.c_void_p(_stream_handle(stream, self.device)))
        if st != 0:
            raise SpecVerifyError(st, "spec_ngram_cache_insert")
        return out_skipped

    def lookup(self, last_tokens: torch.Tensor, *, out_cand: torch.Tensor | None = None,
               out_count: torch.Tensor | None = None, stream=None) -> tuple[torch.Tensor, torch.Tensor]:
        """Candidates [B, G, N-1] (newest first, -1 past the count) and counts [B] for each last token [B]."""
        _check(last_tokens, "last_tokens", self.device, torch.int32, (self.B,))
        if out_cand is None:
            out_cand = torch.empty((self.B, self.G, self.N - 1), dtype=torch.int32, device=self.device)
        if out_count is None:
            out_count = torch.empty((self.B,), dtype=torch.int32, device=self.device)
        _check(out_cand, "out_cand", self.device, torch.int32, (self.B, self.G, self.N - 1))
        _check(out_count, "out_count", self.device, torch.int32, (self.B,))
        st = lib().spec_ngram_cache_lookup(_ptr(self.buffer), self.nbytes, *self._sizes(), _ptr(last_tokens),
                                           _ptr(out_cand), _ptr(out_count),
                                           ctypes.c_void_p(_stream_handle(stream, self.device)))
        if st != 0:
            raise SpecVerifyError(st, "spec_ngram_cache_lookup")
        return out_cand, out_count

    def entries(self) -> tuple[list[int], dict[tuple[int, int], tuple[int, int, int, list[tuple[int, ...]]]]]:
        """Copy the table to the host and read it: (clock per sequence,
        {(b, key): (set, way, stamp, held continuations)}), for inspection."""
        t = self.buffer[: self.B * self.seq_elems].view(self.B, self.seq_elems).cpu()
        clocks = [int(v) & 0xFFFFFFFF for v in t[:, 0].tolist()]
        sets = t[:, 4: 4 + self.sets * self.set_elems].view(self.B, self.sets, self.set_elems)
        keys = sets[:, :, : self.ways]
        stamps = sets[:, :, self.ways: 2 * self.ways]
        slots = sets[:, :, 2 * self.ways:].reshape(self.B, self.sets, self.ways, self.G, self.N - 1)
        out = {}
        for b, s, w in torch.nonzero(keys >= 0).tolist():
            held = [tuple(r) for r in slots[b, s, w].tolist() if r[0] >= 0]
            out[(b, int(keys[b, s, w]))] = (s, w, int(stamps[b, s, w]) & 0xFFFFFFFF, held)
        return clocks, out
