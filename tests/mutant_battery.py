"""Runs the oracle pin battery against one build of the oracle library.

Usage: python tests/mutant_battery.py <path-to-libvif_oracle.so>

Prints one line per pin that fails and exits 1 if any failed, 0 if all
passed.  Used by test_oracle_mutations.py on deliberately broken copies of
the oracle (built in a temporary directory, never in place).
"""
import os
import sys
import traceback

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
import test_oracle_pins as P  # noqa: E402
import test_oracle_options as Q  # noqa: E402
import test_fssim_oracle as S  # noqa: E402


def battery(orc):
    cases = []
    for s in range(4):
        cases.append(("taps%d" % s, lambda s=s: P.test_taps_closed_form(orc, s)))
        cases.append(("impulse%d" % s,
                      lambda s=s: P.test_filter_interior_impulse(orc, s, 3.0)))
        cases.append(("mirror%d" % s,
                      lambda s=s: P.test_filter_whole_sample_mirror(orc, s)))
        cases.append(("brute%d" % s, lambda s=s: P.test_filter_vs_fp64_bruteforce(
            orc, (23, 17), s)))
    for s in (1, 2, 3):
        cases.append(("decim%d" % s,
                      lambda s=s: P.test_decimate_vs_fp64_bruteforce(orc, s)))
    for bpc in (8, 10, 12, 16):
        cases.append(("norm%d" % bpc,
                      lambda b=bpc: P.test_normalise_exact_for_every_code(orc, b)))
    cases += [
        ("mirror_rb", lambda: P.test_filter_right_bottom_mirror(orc)),
        ("order", lambda: P.test_filter_order_is_vertical_then_horizontal(orc)),
        ("decim_phase", lambda: P.test_decimate_even_phase_impulse(orc)),
        ("bitdepth", lambda: P.test_cross_bit_depth_invariance(orc)),
        ("flat_sums", lambda: P.test_flat_frame_sums_are_pixel_counts(
            orc, (40, 40))),
        ("sums_closed", lambda: P.test_ordered_sums_closed_form(orc)),
        ("sums_2_24",
         lambda: P.test_ordered_sums_rounding_accumulates_past_2_24(orc)),
        ("flat_one", lambda: P.test_flat_frame_scores_exactly_one(orc, 8, 128)),
        ("self", lambda: P.test_reference_against_itself(orc, 1)),
        ("stat_low", lambda: P.test_statistic_low_variance_branch(orc)),
        ("stat_thr", lambda: P.test_statistic_threshold_is_inclusive_high(orc)),
        ("stat_s2", lambda: P.test_statistic_zero_distorted_variance(orc)),
        ("stat_neg", lambda: P.test_statistic_negative_gain(orc)),
        ("stat_fp64", lambda: P.test_statistic_vs_fp64_formula(orc)),
        ("num_ratio", lambda: P.test_num_ratio_vs_extended_precision(orc)),
        ("den_ratio", lambda: P.test_den_ratio_closed_form(orc)),
        ("checker", lambda: P.test_checkerboard_translation_symmetry(orc)),
        ("reflect", lambda: P.test_intensity_reflection_symmetry_random(orc)),
        ("log2_pow", lambda: P.test_log2_powers_of_two_exact(orc)),
        ("log2_all", lambda: P.test_log2_exhaustive_first_binade(orc)),
        ("log2_e5", lambda: P.test_log2_other_binades(orc, 5)),
        ("pipe1", lambda: P.test_pipeline_vs_fp64_definition(orc, (32, 32), 1)),
        ("pipe3", lambda: P.test_pipeline_vs_fp64_definition(orc, (41, 73), 3)),
        ("opt_default", lambda: Q.test_default_options_equal_default_entry(orc)),
        ("opt_huge_nsq",
         lambda: Q.test_huge_nsq_puts_every_pixel_in_the_low_branch(orc)),
        ("opt_zero_nsq", lambda: Q.test_zero_nsq_follows_ieee_arithmetic(orc)),
        ("opt_gain0",
         lambda: Q.test_zero_gain_limit_zeroes_every_high_branch_numerator(
             orc)),
        ("opt_gain_mono",
         lambda: Q.test_gain_limit_is_monotone_and_idle_above_the_largest_gain(
             orc)),
        ("opt_gain_self",
         lambda: Q.test_gain_limit_one_leaves_identical_frames_alone(orc)),
        ("opt_skip", lambda: Q.test_skip_scale0(orc)),
        ("opt_floors",
         lambda: Q.test_scale_floors_act_on_reported_scores_only(orc)),
    ]
    for nsq in (2.0, 4.7):
        cases.append(("opt_thr%g" % nsq,
                      lambda v=nsq: Q.test_nsq_threshold_is_an_fp64_comparison(
                          orc, v)))
    for nsq in (1.5, 4.7):
        cases.append(("opt_num%g" % nsq,
                      lambda v=nsq:
                      Q.test_num_ratio_with_nsq_vs_extended_precision(orc, v)))
        cases.append(("opt_den%g" % nsq,
                      lambda v=nsq:
                      Q.test_den_ratio_with_nsq_vs_extended_precision(orc, v)))
    for nsq, lim in ((2.0, 0.3), (4.7, 1.0), (0.5, 0.05)):
        cases.append(("opt_stat%g_%g" % (nsq, lim),
                      lambda v=nsq, l=lim:
                      Q.test_statistic_with_options_vs_fp64_formula(orc, v, l)))
    cases.append(("opt_pipe", lambda:
                  Q.test_pipeline_with_options_vs_fp64_definition(orc, 4.7,
                                                                  0.8)))
    # float SSIM
    cases += [
        ("fs_scale", lambda: S.test_scale_examples_from_the_page(orc)),
        ("fs_round", lambda: S.test_scale_rounds_half_away_from_zero(orc, 384,
                                                                     1000, 2)),
        ("fs_size", lambda: S.test_decimated_size(orc, 1921, 4, 481)),
        ("fs_sym", lambda: S.test_symmetric_border_matches_numpy(orc, 7)),
        ("fs_dec3", lambda: S.test_decimation_is_the_exact_sum_rounded_once(
            orc, 3, 8)),
        ("fs_dec4", lambda: S.test_decimation_is_the_exact_sum_rounded_once(
            orc, 4, 10)),
        ("fs_pow2", lambda: S.test_power_of_two_factor_is_the_plain_mean(orc,
                                                                         4)),
        ("fs_win", lambda: S.test_decimation_window_position_and_offsets(orc)),
        ("fs_taps", lambda: S.test_gaussian_taps(orc)),
        ("fs_filt", lambda: S.test_filter_interior_impulse_and_border(orc)),
        ("fs_self", lambda: S.test_frame_against_itself_scores_exactly_one(
            orc)),
        ("fs_flat", lambda: S.test_flat_frames_closed_form(orc, 10, 240)),
        ("fs_fp64", lambda: S.test_score_vs_fp64_definition(orc, (120, 160), 8,
                                                            1)),
        ("fs_auto",
         lambda: S.test_score_decimates_both_planes_with_the_auto_factor(orc)),
    ]
    for opt in ({"kernelscale": 2.0}, {"sigma_nsq": -1.0},
                {"enhn_gain_limit": -0.5}):
        cases.append(("opt_bad_%s" % list(opt)[0],
                      lambda o=opt: Q.test_bad_options_rejected(orc, o)))
    return cases


def main(path):
    orc = oracle.Oracle(path)
    failed = []
    for name, fn in battery(orc):
        try:
            fn()
        except Exception:  # an assertion or any error counts as caught
            failed.append(name)
            tb = traceback.format_exc().strip().splitlines()[-1]
            print("FAIL %s: %s" % (name, tb[:160]))
    sys.stdout.flush()
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
