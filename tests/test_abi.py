"""The C ABI library: loads, exports what include/*.h declares, rejects bad arguments on the host (no GPU).

Argument errors are detected before any HIP call, so these calls run on a
machine without a GPU. Pointers here are never dereferenced: every call is
built to fail validation (or to be a B = 0 no-op).
"""
import ctypes
import glob
import os
import re

import pytest

import rejection_sampling_verify_sample_amd as rsv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, ERR_NULL, ERR_SHAPE, ERR_TEMP, ERR_DTYPE, ERR_WS, ERR_HIP, ERR_ALIGN, ERR_PHASE = 0, -1, -2, -3, -4, -5, -6, -7, -8
ERR_FILTER_V = -9
ERR_STAGES = -10
ERR_POOL = -11
P = 0x10000  # aligned, never dereferenced


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h, encoding="utf-8").read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names.update(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(spec_\w+)\s*\(", src, flags=re.M))
    return sorted(names)


def test_library_is_built_and_loads():
    assert os.path.exists(rsv.LIB_PATH)
    assert rsv.abi_version() == 1


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) == 26, names
    L = ctypes.CDLL(rsv.LIB_PATH)
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/ but not exported"


def sample(**kw):
    a = dict(target=P, draft=P, dtype=1, tokens=P, uniforms=P, B=4, K=3, V=100, T=1.0, out_tokens=P, out_n=P,
             out_probs=None, ws=P, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return rsv.lib().spec_verify_sample(a["target"], a["draft"], a["dtype"], a["tokens"], a["uniforms"], a["B"],
                                        a["K"], a["V"], a["T"], a["out_tokens"], a["out_n"], a["out_probs"],
                                        a["ws"], a["ws_bytes"], a["stream"])


def greedy(**kw):
    a = dict(logits=P, dtype=1, cand=P, B=2, G=3, N=4, V=100, out_tokens=P, out_len=P, out_best=P, ws=P,
             ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return rsv.lib().spec_verify_greedy(a["logits"], a["dtype"], a["cand"], a["B"], a["G"], a["N"], a["V"],
                                        a["out_tokens"], a["out_len"], a["out_best"], a["ws"], a["ws_bytes"],
                                        a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(B=-1), ERR_SHAPE), (dict(K=-1), ERR_SHAPE), (dict(K=65), ERR_SHAPE), (dict(V=0), ERR_SHAPE),
    (dict(V=(1 << 30) + 1), ERR_SHAPE), (dict(B=1 << 22, K=8), ERR_SHAPE),
    (dict(dtype=2), ERR_DTYPE), (dict(dtype=-1), ERR_DTYPE),
    (dict(T=0.0), ERR_TEMP), (dict(T=-1.0), ERR_TEMP), (dict(T=float("nan")), ERR_TEMP),
    (dict(T=float("inf")), ERR_TEMP), (dict(T=1e-45), ERR_TEMP),
    (dict(target=None), ERR_NULL), (dict(draft=None), ERR_NULL), (dict(tokens=None), ERR_NULL),
    (dict(uniforms=None), ERR_NULL), (dict(out_tokens=None), ERR_NULL), (dict(out_n=None), ERR_NULL),
    (dict(ws=None), ERR_NULL),
    (dict(target=P + 1), ERR_ALIGN), (dict(dtype=0, draft=P + 2), ERR_ALIGN), (dict(tokens=P + 2), ERR_ALIGN),
    (dict(out_probs=P + 1), ERR_ALIGN), (dict(ws=P + 4), ERR_ALIGN),
    (dict(ws_bytes=16), ERR_WS),
    (dict(B=0), OK), (dict(B=0, target=None, ws=None), OK),
])
def test_sample_argument_checks(kw, expect):
    assert sample(**kw) == expect


def test_phase_entry_point_checks_arguments():
    fn = rsv.lib().spec_verify_sample_phases
    args = [P, P, 1, P, P, 4, 3, 100, 1.0, P, P, None, P, 1 << 30, None]
    for bad in (0, 16, -1):
        assert fn(*args, bad) == ERR_PHASE
    a = list(args)
    a[8] = 0.0
    assert fn(*a, 1) == ERR_TEMP
    a = list(args)
    a[13] = 16
    assert fn(*a, 4) == ERR_WS
    a = list(args)
    a[6] = 99
    assert fn(*a, 2) == ERR_SHAPE


def filtered(**kw):
    a = dict(target=P, draft=P, dtype=1, tokens=P, uniforms=P, B=4, K=3, V=100, T=1.0, out_tokens=P, out_n=P,
             out_probs=None, ws=P, ws_bytes=1 << 30, stream=None, top_k=P, top_p=P, out_kept=P)
    a.update(kw)
    return rsv.lib().spec_verify_sample_filtered(a["target"], a["draft"], a["dtype"], a["tokens"], a["uniforms"],
                                                 a["B"], a["K"], a["V"], a["T"], a["out_tokens"], a["out_n"],
                                                 a["out_probs"], a["ws"], a["ws_bytes"], a["stream"], a["top_k"],
                                                 a["top_p"], a["out_kept"])


@pytest.mark.parametrize("kw,expect", [
    (dict(V=(1 << 24) + 1), ERR_FILTER_V), (dict(V=(1 << 30) + 1), ERR_SHAPE), (dict(K=65), ERR_SHAPE),
    (dict(T=0.0), ERR_TEMP), (dict(dtype=2), ERR_DTYPE), (dict(target=None), ERR_NULL),
    (dict(top_k=P + 2), ERR_ALIGN), (dict(top_p=P + 1), ERR_ALIGN), (dict(out_kept=P + 2), ERR_ALIGN),
    (dict(ws_bytes=16), ERR_WS), (dict(B=0), OK),
    # the filters and the kept counts are optional: with every check passed, only the workspace fails
    (dict(top_k=None, top_p=None, out_kept=None, ws_bytes=16), ERR_WS),
])
def test_filtered_argument_checks(kw, expect):
    assert filtered(**kw) == expect


def test_filtered_phases_checks_arguments():
    fn = rsv.lib().spec_verify_sample_filtered_phases
    args = [P, P, 1, P, P, 4, 3, 100, 1.0, P, P, None, P, 1 << 30, None, P, P, None]
    for bad in (0, 16):
        assert fn(*args, bad) == ERR_PHASE
    a = list(args)
    a[7] = (1 << 24) + 1
    assert fn(*a, 1) == ERR_FILTER_V


def staged(ends, **kw):
    a = dict(target=P, draft=P, dtype=1, tokens=P, uniforms=P, B=4, K=8, V=100, T=1.0, out_tokens=P, out_n=P,
             out_probs=None, ws=P, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    n = kw.pop("num_stages", None)
    arr = None if ends is None else (ctypes.c_int32 * max(1, len(ends)))(*ends)
    num = len(ends) if n is None and ends is not None else (n if n is not None else 0)
    return rsv.lib().spec_verify_sample_staged(a["target"], a["draft"], a["dtype"], a["tokens"], a["uniforms"],
                                               a["B"], a["K"], a["V"], a["T"], a["out_tokens"], a["out_n"],
                                               a["out_probs"], a["ws"], a["ws_bytes"], a["stream"], arr, num)


@pytest.mark.parametrize("ends,kw,expect", [
    # valid schedules get through to the workspace check
    ([8], dict(ws_bytes=16), ERR_WS), ([2, 4, 8], dict(ws_bytes=16), ERR_WS), ([1, 2, 3, 4, 5, 6, 7, 8],
                                                                                dict(ws_bytes=16), ERR_WS),
    ([], dict(K=0, ws_bytes=16), ERR_WS), (None, dict(K=0, ws_bytes=16), ERR_WS),
    # invalid schedules
    ([], {}, ERR_STAGES), (None, {}, ERR_STAGES), ([4], {}, ERR_STAGES), ([4, 9], {}, ERR_STAGES),
    ([0, 8], {}, ERR_STAGES), ([4, 4, 8], {}, ERR_STAGES), ([6, 4, 8], {}, ERR_STAGES), ([8, 8], {}, ERR_STAGES),
    ([1, 2, 3, 4, 5, 6, 7, 8, 8], {}, ERR_STAGES), ([2], dict(K=0), ERR_STAGES),
    # shape errors come first; B = 0 is a no-op once the schedule is valid
    ([8], dict(K=65), ERR_SHAPE), ([8], dict(B=0), OK), ([8], dict(T=0.0), ERR_TEMP),
])
def test_staged_argument_checks(ends, kw, expect):
    assert staged(ends, **kw) == expect


def test_staged_negative_stage_count():
    assert staged([8], num_stages=-1) == ERR_STAGES


def test_ngram_pool_bytes():
    assert rsv.ngram_pool_bytes(32, 32000, 7, 5) == 32 * 32000 * 7 * 4 * 4
    assert rsv.ngram_pool_bytes(0, 32000, 7, 5) == 0
    for bad in ((-1, 10, 2, 3), (1, 0, 2, 3), (1, 10, 0, 3), (1, 10, 65, 3), (1, 10, 2, 1), (1, 10, 2, 18),
                (1, (1 << 30) + 1, 2, 3)):
        assert rsv.ngram_pool_bytes(*bad) == 0, bad
    # sizes past what int64 byte offsets can address are rejected, not wrapped
    assert rsv.ngram_pool_bytes(1 << 30, 1 << 30, 64, 17) == 0


def pool_call(fn, **kw):
    a = dict(pool=P, nbytes=1 << 40, B=2, V=10, G=3, N=4, W=5, ngrams=P, skipped=None, last=P, cand=P, count=P,
             stream=None)
    a.update(kw)
    L = rsv.lib()
    if fn == "init":
        return L.spec_ngram_pool_init(a["pool"], a["nbytes"], a["B"], a["V"], a["G"], a["N"], a["stream"])
    if fn == "insert":
        return L.spec_ngram_pool_insert(a["pool"], a["nbytes"], a["B"], a["V"], a["G"], a["N"], a["ngrams"], a["W"],
                                        a["skipped"], a["stream"])
    return L.spec_ngram_pool_lookup(a["pool"], a["nbytes"], a["B"], a["V"], a["G"], a["N"], a["last"], a["cand"],
                                    a["count"], a["stream"])


@pytest.mark.parametrize("fn,kw,expect", [
    ("init", dict(G=0), ERR_SHAPE), ("init", dict(N=1), ERR_SHAPE), ("init", dict(N=18), ERR_SHAPE),
    ("init", dict(pool=None), ERR_NULL), ("init", dict(pool=P + 4), ERR_ALIGN), ("init", dict(nbytes=16), ERR_POOL),
    ("init", dict(B=0, pool=None), OK),
    ("insert", dict(W=-1), ERR_SHAPE), ("insert", dict(W=65), ERR_SHAPE), ("insert", dict(V=0), ERR_SHAPE),
    ("insert", dict(ngrams=None), ERR_NULL), ("insert", dict(ngrams=P + 2), ERR_ALIGN),
    ("insert", dict(skipped=P + 1), ERR_ALIGN), ("insert", dict(nbytes=100), ERR_POOL),
    ("insert", dict(B=0), OK), ("insert", dict(W=0, ngrams=None, nbytes=16), ERR_POOL),
    ("lookup", dict(G=65), ERR_SHAPE), ("lookup", dict(last=None), ERR_NULL), ("lookup", dict(cand=None), ERR_NULL),
    ("lookup", dict(count=None), ERR_NULL), ("lookup", dict(cand=P + 2), ERR_ALIGN), ("lookup", dict(nbytes=8), ERR_POOL),
    ("lookup", dict(B=0, last=None), OK),
])
def test_ngram_pool_argument_checks(fn, kw, expect):
    assert pool_call(fn, **kw) == expect


def test_ngram_cache_bytes():
    # per sequence: 4 + sets * (2 * ways + ways * G * (N - 1)) int32, rounded up to a multiple of 4
    assert rsv.ngram_cache_bytes(32, 512, 8, 7, 5) == 32 * (4 + 512 * (16 + 8 * 7 * 4)) * 4
    assert rsv.ngram_cache_bytes(3, 1, 1, 1, 2) == 3 * 8 * 4
    assert rsv.ngram_cache_bytes(2, 2, 3, 2, 3) == 2 * 40 * 4   # 4 + 2 * (6 + 12) = 40
    assert rsv.ngram_cache_bytes(1, 1, 3, 1, 2) == 16 * 4       # 4 + (6 + 3) = 13 -> 16
    assert rsv.ngram_cache_bytes(0, 512, 8, 7, 5) == 0
    for bad in ((-1, 1, 1, 1, 2), (1, 0, 1, 1, 2), (1, 3, 1, 1, 2), (1, 12, 1, 1, 2), (1, (1 << 24) * 2, 1, 1, 2),
                (1, 1, 0, 1, 2), (1, 1, 65, 1, 2), (1, 1, 1, 0, 2), (1, 1, 1, 65, 2), (1, 1, 1, 1, 1),
                (1, 1, 1, 1, 18)):
        assert rsv.ngram_cache_bytes(*bad) == 0, bad
    assert rsv.ngram_cache_bytes(1, 1 << 24, 1, 1, 2) == (4 + (1 << 24) * 3) * 4
    # sizes past what int64 byte offsets can address are rejected, not wrapped
    assert rsv.ngram_cache_bytes(1 << 30, 1 << 24, 64, 64, 17) == 0


def cache_call(fn, **kw):
    a = dict(cache=P, nbytes=1 << 40, B=2, V=10, sets=4, ways=2, G=3, N=4, W=5, ngrams=P, skipped=None, last=P,
             cand=P, count=P, stream=None)
    a.update(kw)
    L = rsv.lib()
    geo = (a["sets"], a["ways"], a["G"], a["N"])
    if fn == "init":
        return L.spec_ngram_cache_init(a["cache"], a["nbytes"], a["B"], *geo, a["stream"])
    if fn == "insert":
        return L.spec_ngram_cache_insert(a["cache"], a["nbytes"], a["B"], a["V"], *geo, a["ngrams"], a["W"],
                                         a["skipped"], a["stream"])
    return L.spec_ngram_cache_lookup(a["cache"], a["nbytes"], a["B"], a["V"], *geo, a["last"], a["cand"],
                                     a["count"], a["stream"])


@pytest.mark.parametrize("fn,kw,expect", [
    ("init", dict(sets=3), ERR_SHAPE), ("init", dict(sets=0), ERR_SHAPE), ("init", dict(ways=65), ERR_SHAPE),
    ("init", dict(G=0), ERR_SHAPE), ("init", dict(N=18), ERR_SHAPE),
    ("init", dict(cache=None), ERR_NULL), ("init", dict(cache=P + 4), ERR_ALIGN), ("init", dict(nbytes=16), ERR_POOL),
    ("init", dict(B=0, cache=None), OK),
    ("insert", dict(W=-1), ERR_SHAPE), ("insert", dict(W=65), ERR_SHAPE), ("insert", dict(V=0), ERR_SHAPE),
    ("insert", dict(V=(1 << 30) + 1), ERR_SHAPE), ("insert", dict(ways=0), ERR_SHAPE),
    ("insert", dict(ngrams=None), ERR_NULL), ("insert", dict(ngrams=P + 2), ERR_ALIGN),
    ("insert", dict(skipped=P + 1), ERR_ALIGN), ("insert", dict(nbytes=100), ERR_POOL),
    ("insert", dict(B=0), OK), ("insert", dict(W=0, ngrams=None, nbytes=16), ERR_POOL),
    ("lookup", dict(G=65), ERR_SHAPE), ("lookup", dict(V=0), ERR_SHAPE), ("lookup", dict(sets=6), ERR_SHAPE),
    ("lookup", dict(last=None), ERR_NULL), ("lookup", dict(cand=None), ERR_NULL),
    ("lookup", dict(count=None), ERR_NULL), ("lookup", dict(cand=P + 2), ERR_ALIGN),
    ("lookup", dict(nbytes=8), ERR_POOL), ("lookup", dict(B=0, last=None), OK),
])
def test_ngram_cache_argument_checks(fn, kw, expect):
    assert cache_call(fn, **kw) == expect


def ngram_sample(**kw):
    a = dict(logits=P, dtype=1, cand=P, uniforms=P, B=2, G=3, N=4, V=100, T=1.0, out_tokens=P, out_len=P,
             out_rows=P, ws=P, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return rsv.lib().spec_verify_ngram_sample(a["logits"], a["dtype"], a["cand"], a["uniforms"], a["B"], a["G"],
                                              a["N"], a["V"], a["T"], a["out_tokens"], a["out_len"], a["out_rows"],
                                              a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(B=-1), ERR_SHAPE), (dict(G=0), ERR_SHAPE), (dict(G=65), ERR_SHAPE), (dict(N=1), ERR_SHAPE),
    (dict(N=66), ERR_SHAPE), (dict(V=0), ERR_SHAPE), (dict(V=(1 << 20) + 1), ERR_SHAPE),
    (dict(B=1 << 20, G=64, N=2), ERR_SHAPE), (dict(G=64, N=17), ERR_SHAPE), (dict(G=16, N=65), ERR_SHAPE),
    (dict(dtype=2), ERR_DTYPE), (dict(T=0.0), ERR_TEMP), (dict(T=float("inf")), ERR_TEMP),
    (dict(logits=None), ERR_NULL), (dict(cand=None), ERR_NULL), (dict(uniforms=None), ERR_NULL),
    (dict(out_rows=None), ERR_NULL), (dict(ws=None), ERR_NULL),
    (dict(logits=P + 1), ERR_ALIGN), (dict(cand=P + 2), ERR_ALIGN), (dict(ws=P + 4), ERR_ALIGN),
    (dict(ws_bytes=16), ERR_WS), (dict(B=0), OK), (dict(B=0, logits=None), OK),
])
def test_ngram_sample_argument_checks(kw, expect):
    assert ngram_sample(**kw) == expect


def test_ngram_sample_workspace_size():
    assert rsv.ngram_sample_workspace_size(32, 7, 5, 32000) > 0
    assert rsv.ngram_sample_workspace_size(32, 65, 5, 32000) == 0
    assert rsv.ngram_sample_workspace_size(32, 7, 66, 32000) == 0
    assert rsv.ngram_sample_workspace_size(32, 64, 16, 32000) > 0
    assert rsv.ngram_sample_workspace_size(32, 64, 17, 32000) == 0


def test_sample_k0_needs_no_draft():
    # K = 0 draws from the bonus row only: draft pointers may be null; still fails on the workspace size
    assert sample(K=0, draft=None, tokens=None, ws_bytes=0) == ERR_WS


@pytest.mark.parametrize("kw,expect", [
    (dict(B=-1), ERR_SHAPE), (dict(G=0), ERR_SHAPE), (dict(N=1), ERR_SHAPE), (dict(N=66), ERR_SHAPE),
    (dict(G=3000, N=3), ERR_SHAPE), (dict(V=0), ERR_SHAPE),
    (dict(dtype=3), ERR_DTYPE), (dict(logits=None), ERR_NULL), (dict(cand=None), ERR_NULL),
    (dict(out_best=None), ERR_NULL), (dict(logits=P + 1), ERR_ALIGN), (dict(cand=P + 1), ERR_ALIGN),
    (dict(ws_bytes=8), ERR_WS), (dict(B=0), OK),
])
def test_greedy_argument_checks(kw, expect):
    assert greedy(**kw) == expect


def test_fill_uniforms_argument_checks():
    L = rsv.lib()
    assert L.spec_fill_uniforms(0, 0, -1, 4, P, None) == ERR_SHAPE
    assert L.spec_fill_uniforms(0, 0, 4, 65, P, None) == ERR_SHAPE
    assert L.spec_fill_uniforms(0, 0, 4, 4, None, None) == ERR_NULL
    assert L.spec_fill_uniforms(0, 0, 4, 4, P + 2, None) == ERR_ALIGN
    assert L.spec_fill_uniforms(0, 0, 0, 4, None, None) == OK


def test_workspace_sizes():
    assert rsv.sample_workspace_size(64, 8, 128256) > 0
    assert rsv.sample_workspace_size(0, 8, 100) > 0
    assert rsv.sample_workspace_size(-1, 8, 100) == 0
    assert rsv.sample_workspace_size(4, 65, 100) == 0
    assert rsv.sample_filtered_workspace_size(64, 8, 128256) > 0
    assert rsv.sample_filtered_workspace_size(4, 2, (1 << 24) + 1) == 0
    assert rsv.greedy_workspace_size(32, 7, 5, 32000) > 0
    assert rsv.greedy_workspace_size(32, 7, 1, 32000) == 0
    # the size depends on the shape only (never on a tuning override)
    os.environ["SPECVERIFY_S1"] = "3"
    try:
        assert rsv.sample_workspace_size(64, 8, 128256) == rsv.sample_workspace_size(64, 8, 128256)
    finally:
        del os.environ["SPECVERIFY_S1"]


def test_status_strings():
    for s in (OK, ERR_NULL, ERR_SHAPE, ERR_TEMP, ERR_DTYPE, ERR_WS, ERR_HIP, ERR_ALIGN, ERR_PHASE, ERR_FILTER_V,
              ERR_STAGES, ERR_POOL, 99):
        assert isinstance(rsv.status_string(s), str) and rsv.status_string(s)


def test_binding_checks_tensors_before_the_library():
    import torch
    t = torch.zeros(2, 3, 8)
    with pytest.raises((TypeError, ValueError)):
        rsv.verify_sample(t, torch.zeros(2, 2, 8, dtype=torch.float64), torch.zeros(2, 2, dtype=torch.int32),
                          torch.zeros(2, 3, 2), 1.0)
    with pytest.raises((TypeError, ValueError)):
        rsv.verify_greedy(torch.zeros(1, 2, 3, 8), torch.zeros(1, 2, 3, dtype=torch.int32))


def noalloc(**kw):
    a = dict(target=P, draft=P, dtype=1, tokens=P, uniforms=P, B=4, K=3, V=100, T=1.0, out_tokens=P, out_n=P,
             out_probs=None, stream=None)
    a.update(kw)
    return rsv.lib().spec_verify_sample_noalloc(a["target"], a["draft"], a["dtype"], a["tokens"], a["uniforms"],
                                                a["B"], a["K"], a["V"], a["T"], a["out_tokens"], a["out_n"],
                                                a["out_probs"], a["stream"])


def test_noalloc_limit_is_the_header_value():
    hdr = open(os.path.join(ROOT, "include", "spec_verify.h")).read()
    m = re.search(r"#define SPEC_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m, "the header states the scratch size"
    assert rsv.lib().spec_verify_sample_noalloc_max_bytes() == int(m.group(1)) << int(m.group(2))


def test_noalloc_scratch_holds_the_sampling_workloads():
    # B=1 K=4 V=32000, B=8 K=5 V=32000, B=64 K=8 V=128256, B=256 K=4 V=152064
    for B, K, V in ((1, 4, 32000), (8, 5, 32000), (64, 8, 128256), (256, 4, 152064)):
        assert rsv.sample_workspace_size(B, K, V) <= rsv.lib().spec_verify_sample_noalloc_max_bytes()


@pytest.mark.parametrize("kw,expect", [
    (dict(B=-1), ERR_SHAPE), (dict(K=65), ERR_SHAPE), (dict(V=0), ERR_SHAPE),
    (dict(dtype=2), ERR_DTYPE), (dict(T=0.0), ERR_TEMP), (dict(T=float("nan")), ERR_TEMP),
    (dict(target=None), ERR_NULL), (dict(draft=None), ERR_NULL), (dict(uniforms=None), ERR_NULL),
    (dict(out_tokens=None), ERR_NULL), (dict(out_n=None), ERR_NULL),
    (dict(target=P + 1), ERR_ALIGN), (dict(out_probs=P + 2), ERR_ALIGN),
    # sizes whose workspace exceeds the fixed scratch are refused before any HIP call
    (dict(B=4096, K=8, V=128256), ERR_WS), (dict(B=1024, K=4, V=152064), ERR_WS),
    (dict(B=0), OK), (dict(B=0, target=None), OK),
])
def test_noalloc_argument_checks(kw, expect):
    assert noalloc(**kw) == expect


def test_noalloc_scratch_covers_the_four_sampling_workloads():
    for B, K, V in ((1, 4, 32000), (8, 5, 32000), (64, 8, 128256), (256, 4, 152064)):
        assert 0 < rsv.sample_workspace_size(B, K, V) <= rsv.lib().spec_verify_sample_noalloc_max_bytes()


def rowstats(**kw):
    a = dict(logits=P, dtype=1, rows=5, V=100, T=1.0, out_max=P, out_sum=P, ws=P, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return rsv.lib().spec_row_stats(a["logits"], a["dtype"], a["rows"], a["V"], a["T"], a["out_max"], a["out_sum"],
                                    a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(rows=-1), ERR_SHAPE), (dict(V=0), ERR_SHAPE), (dict(rows=(1 << 24) + 1), ERR_SHAPE),
    (dict(dtype=3), ERR_DTYPE), (dict(T=0.0), ERR_TEMP), (dict(T=float("inf")), ERR_TEMP),
    (dict(logits=None), ERR_NULL), (dict(out_max=None), ERR_NULL), (dict(out_sum=None), ERR_NULL),
    (dict(ws=None), ERR_NULL), (dict(logits=P + 1), ERR_ALIGN), (dict(out_sum=P + 4), ERR_ALIGN),
    (dict(ws_bytes=8), ERR_WS), (dict(rows=0), OK), (dict(rows=0, logits=None), OK),
])
def test_row_stats_argument_checks(kw, expect):
    assert rowstats(**kw) == expect
