"""The CPU oracle against the facts that pin it (no GPU)."""
import oracle
import pins


def test_golden_sample_rounds():
    pins.check_golden_sample(oracle)


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
