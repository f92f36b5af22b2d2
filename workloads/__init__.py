"""Seeded synthetic inputs for the verify step (shared by the oracle tests, the GPU tests and the bench).

Holds input construction only: no step of the verify method.
"""
from .bf16 import bf16_bits_to_f32, bf16_round, f32_to_bf16_bits
from .configs import (BF16, F32, GREEDY_CONFIGS, SAMPLE_CONFIGS, WORKLOAD_NAMES, GreedyInputs, NgramSampleInputs,
                      SampleInputs, make_filter_params, make_greedy_inputs, make_ngram_sample_inputs,
                      make_sample_inputs)
from .philox import ngram_uniforms, philox4x32_10, verify_uniforms, words_to_unit

__all__ = [
    "BF16", "F32", "GREEDY_CONFIGS", "SAMPLE_CONFIGS", "WORKLOAD_NAMES", "GreedyInputs", "NgramSampleInputs",
    "SampleInputs", "make_filter_params", "make_greedy_inputs", "make_ngram_sample_inputs", "make_sample_inputs",
    "ngram_uniforms", "philox4x32_10", "verify_uniforms", "words_to_unit",
    "bf16_bits_to_f32", "bf16_round", "f32_to_bf16_bits",
]
