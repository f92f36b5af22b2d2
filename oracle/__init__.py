"""CPU oracle of the verify step (float64 NumPy).

TEST INFRASTRUCTURE: only the tests, the package's smoke check and the bench's
CPU-baseline leg may import it. The HIP library and its binding never do.
"""
from .verify import (GreedyResult, SampleResult, acceptance_probability, first_argmax, inverse_cdf_draw,
                     oracle_greedy, oracle_sample, row_is_valid, softmax64, temperature64, token_probs)

__all__ = [
    "GreedyResult", "SampleResult", "acceptance_probability", "first_argmax", "inverse_cdf_draw",
    "oracle_greedy", "oracle_sample", "row_is_valid", "softmax64", "temperature64", "token_probs",
]
