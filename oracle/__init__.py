"""CPU oracle of the verify step (float64 NumPy) and of the n-gram pool (oracle.ngram, plain Python).

TEST INFRASTRUCTURE: only the tests, the package's smoke check and the bench's
CPU-baseline leg may import it. The HIP library and its binding never do.
"""
from .verify import (FilteredResult, GreedyResult, KeepResult, NgramSampleResult, SampleResult,
                     acceptance_probability, filter_keep, filtered_softmax64, first_argmax, inverse_cdf_draw,
                     oracle_greedy, oracle_ngram_sample, oracle_sample, oracle_sample_filtered, row_is_valid,
                     softmax64, temperature64, token_probs, top_p64)

__all__ = [
    "FilteredResult", "GreedyResult", "KeepResult", "NgramSampleResult", "SampleResult", "acceptance_probability", "filter_keep",
    "filtered_softmax64", "first_argmax", "inverse_cdf_draw", "oracle_greedy", "oracle_ngram_sample", "oracle_sample",
    "oracle_sample_filtered", "row_is_valid", "softmax64", "temperature64", "token_probs", "top_p64",
]
