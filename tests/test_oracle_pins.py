"""The CPU oracle against the facts that pin it (no GPU)."""
import os

import oracle
import pins


def test_golden_sample_rounds():
    pins.check_golden_sample(oracle)


def test_token_probabilities():
    pins.check_token_probs(oracle)


def test_golden_greedy_rounds():
    pins.check_golden_greedy(oracle)


def test_softmax_closed_forms():
    pins.check_softmax_closed_forms(oracle)


def test_acceptance_special_cases():
    pins.check_acceptance_special_cases(oracle)


def test_inverse_cdf_convention():
    pins.check_inverse_cdf(oracle)


def test_output_law_is_p_exactly_on_a_grid():
    pins.check_exact_law_on_grid(oracle)


def test_output_law_chisquare():
    pins.check_chisquare_law(oracle)


def _chi_job(args):
    import oracle as orc
    return pins.chisquare_counts(orc, *args)


def test_output_law_chisquare_one_million_trials():
    """The chi-square of the output law at 10^6 verify rows per vocabulary (V = 2, 5, 16), chunks in worker processes."""
    import concurrent.futures
    import multiprocessing
    workers = max(1, min(8, os.cpu_count() or 1))
    with concurrent.futures.ProcessPoolExecutor(workers, mp_context=multiprocessing.get_context("spawn")) as ex:
        pins.check_chisquare_law(oracle, trials=1_000_000, map_fn=lambda jobs: ex.map(_chi_job, jobs))


def test_acceptance_rate_is_one_minus_tv():
    pins.check_acceptance_is_one_minus_tv(oracle)


def test_tokens_per_round_closed_form():
    pins.check_tokens_per_round(oracle)


def test_greedy_lookahead_eq5():
    pins.check_greedy_eq5(oracle)


def test_greedy_argmax_brute_force():
    pins.check_greedy_argmax_brute_force(oracle)


def test_fault_reading():
    pins.check_faults(oracle)


def test_golden_filtered_rounds():
    pins.check_golden_filtered(oracle)


def test_filter_top_k_by_rank():
    pins.check_filter_top_k_by_rank(oracle)


def test_filter_top_p_nucleus_in_rationals():
    pins.check_filter_top_p_nucleus(oracle)


def test_filter_special_cases():
    pins.check_filter_special_cases(oracle)


def test_filters_off_match_plain_verify():
    pins.check_filters_off_match_plain(oracle)


def test_filtered_output_law_exact_on_a_grid():
    pins.check_filtered_exact_law(oracle)


def test_golden_ngram_sample_rounds():
    pins.check_golden_ngram_sample(oracle)


def test_ngram_sample_one_candidate_is_speculative_decoding():
    pins.check_ngram_sample_g1_matches_sample(oracle)


def test_ngram_sample_output_law_exact():
    pins.check_ngram_sample_exact_law(oracle)
