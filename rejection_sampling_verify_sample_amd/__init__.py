"""MI355X-native speculative-decoding verify: HIP kernels behind a C ABI (libspecverify.so).

Entry points (torch tensors in, torch tensors out; every computation runs in HIP):
  verify_sample  -- rejection-sampling verify of K draft tokens per row
  verify_sample_filtered -- the same on top-k / top-p filtered laws (same filter on both sides)
  verify_sample_staged -- verify_sample with early exit: pass 1 in stages over the draft positions
  verify_sample_noalloc -- verify_sample on the library's fixed device scratch (allocates nothing)
  verify_greedy  -- greedy longest-prefix verify of G candidate n-grams
  verify_ngram_sample -- sampling verify of G greedy-drafted (one-hot) candidate n-grams
  fill_uniforms  -- Philox4x32-10 verify uniforms on the device
  row_stats      -- softmax statistics (max, denominator) of logit rows, as the verify computes them
  NgramPool      -- the n-gram pool that supplies verify_greedy's candidates (insert / lookup)
  NgramCache     -- the same pool in a bounded hash table (sets x ways keys per sequence, LRU eviction)
"""
from ._lib import (LIB_PATH, PHASE_ACCEPT, PHASE_ALL, PHASE_DRAW, PHASE_MASS, PHASE_ROW_STATS, SPEC_BF16, SPEC_F32,
                   SPEC_MAX_K, GreedyOutputs, NgramCache, NgramPool, NgramSampleOutputs, SampleOutputs,
                   SpecVerifyError, abi_version, fill_uniforms, greedy_workspace_size, lib, ngram_cache_bytes,
                   ngram_pool_bytes, ngram_sample_workspace_size, row_stats, sample_filtered_workspace_size,
                   sample_workspace_size, status_string, verify_greedy, verify_ngram_sample, verify_sample,
                   verify_sample_filtered, verify_sample_noalloc, verify_sample_staged, workspace_for)

__all__ = [
    "LIB_PATH", "PHASE_ACCEPT", "PHASE_ALL", "PHASE_DRAW", "PHASE_MASS", "PHASE_ROW_STATS", "SPEC_BF16", "SPEC_F32",
    "SPEC_MAX_K", "GreedyOutputs", "NgramCache", "NgramPool", "NgramSampleOutputs", "SampleOutputs",
    "SpecVerifyError", "abi_version", "fill_uniforms", "greedy_workspace_size", "lib", "ngram_cache_bytes",
    "ngram_pool_bytes", "ngram_sample_workspace_size", "row_stats", "sample_filtered_workspace_size",
    "sample_workspace_size", "status_string", "verify_greedy", "verify_ngram_sample", "verify_sample",
    "verify_sample_filtered", "verify_sample_noalloc", "verify_sample_staged", "workspace_for",
]
