"""The pins are sharp: plausible mistakes planted in a copy of the oracle
are each caught by at least one pin.

Each mutant is the oracle's C source with one textual change, compiled into
a temporary directory and run through tests/mutant_battery.py in its own
process (so a mutant that crashes cannot take the test run down; a crash
also counts as caught).  The real oracle must pass the same battery.
CPU only.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "vif_oracle.c")

# (name, text in vif_oracle.c, replacement).  Not listed: removing the
# clamp of sigma1_sq at zero, an equivalent mutant (a negative sigma1_sq
# takes the low-variance branch either way, so no output can change), and
# evaluating the denominator ratio in fp32 as 1.0f + sigma1_sq * 0.5f, which
# is provably the same value (see test_den_ratio_closed_form); and comparing
# the gain with fl32(limit) in fp32 in place of the fp64 comparison, which
# selects the same value for every limit (no fp32 value lies strictly
# between a limit and its nearest fp32, so the two comparisons can differ
# only where g is that fp32 value, and then both results are it); and
# letting a NaN gain pass the limit: a NaN gain comes only from 0/0, which
# makes sv_sq NaN as well unless the sigma2_sq rule resets both, so the
# numerator quotient is NaN whatever the gain is.
MUTANTS = [
    ("sigma_n_over_6", "(double)n / 5.0", "(double)n / 6.0"),
    ("taps_unnormalised", "taps[k] = (float)(g[k] / sum);",
     "taps[k] = (float)(g[k]);"),
    ("mirror_half_sample_low", "        m = -m;\n", "        m = -m - 1;\n"),
    ("mirror_half_sample_high", "m = 2 * (n - 1) - m;", "m = 2 * n - 1 - m;"),
    ("vertical_tap_offset", "const int yy = mirror(y + k - r, h);",
     "const int yy = mirror(y + k - r + (k == 0), h);"),
    ("horizontal_reads_src", "taps[k] * v[(size_t)y * w + xx]",
     "taps[k] * src[(size_t)y * w + xx]"),
    ("decimate_odd_phase", "full[(size_t)(2 * y) * w + 2 * x]",
     "full[(size_t)(2 * y + 1) * w + 2 * x + 1]"),
    ("decimate_prev_scale_taps",
     "            if (vifo_decimate(X, ws, hs, taps, nt, Xn) != 0 ||\n"
     "                vifo_decimate(Y, ws, hs, taps, nt, Yn) != 0)\n",
     "            float pt[VIFO_MAX_TAPS];\n"
     "            const int np = vifo_taps(s - 1, pt);\n"
     "            if (vifo_decimate(X, ws, hs, pt, np, Xn) != 0 ||\n"
     "                vifo_decimate(Y, ws, hs, pt, np, Yn) != 0)\n"),
    ("xy_is_xx", "XY[i] = X[i] * Y[i];", "XY[i] = X[i] * X[i];"),
    ("ref_dist_swapped", "vifo_normalise(ref, w, h, bpc, X);\n"
     "    vifo_normalise(dist, w, h, bpc, Y);",
     "vifo_normalise(dist, w, h, bpc, X);\n"
     "    vifo_normalise(ref, w, h, bpc, Y);"),
    ("norm10_wrong", "scale = 0.25f;", "scale = 0.125f;"),
    ("sigma12_sign", "const float sigma12 = xy - mu1_mu2;",
     "const float sigma12 = mu1_mu2 - xy;"),
    ("sigma2_no_mean", "float sigma2_sq = yy - mu2_sq;",
     "float sigma2_sq = yy;"),
    ("threshold_1", "if ((double)sigma1_sq < nsq) {",
     "if ((double)sigma1_sq < 1.0) {"),
    ("threshold_le", "if ((double)sigma1_sq < nsq) {",
     "if ((double)sigma1_sq <= nsq) {"),
    ("low_branch_num_0", "        *num_t = 1.0f;\n", "        *num_t = 0.0f;\n"),
    ("no_nsq_in_num", "(double)sv_sq + nsq;", "(double)sv_sq + 1.0;"),
    ("nsq_fp32_num", "const double num_q = (double)num_arg / num_den;",
     "const double num_q = (double)(num_arg / (float)num_den);"),
    ("num_single_rounding_fp32", "return (float)(1.0 + num_q);",
     "return 1.0f + (float)num_q;"),
    ("den_ratio_inverted", "const double den_q = (double)sigma1_sq / nsq;",
     "const double den_q = nsq / (double)sigma1_sq;"),
    ("no_negative_gain_rule", "if (g < 0.0f) {", "if (g < -1e30f) {"),
    ("sv_floor_1", "if (sv_sq < eps)\n        sv_sq = eps;",
     "if (sv_sq < 1.0f)\n        sv_sq = 1.0f;"),
    ("gain_not_squared", "const float g_sq = g * g;", "const float g_sq = g;"),
    ("log2_bias", "- 127;", "- 126;"),
    ("log2_coef_sign", "0xbe6194f1u", "0x3e6194f1u"),
    ("log2_drop_last_coef", "0xbb96254au", "0x00000000u"),
    ("log2_t_not_minus_one", "const float t = m - 1.0f;",
     "const float t = m - 0.5f;"),
    ("row_sum_swapped", "n_s = n_s + n_y;", "n_s = n_s + d_y;"),
    # the ordered sums (O9)
    ("row_acc_fp64", "float n_y = 0.0f, d_y = 0.0f;",
     "double n_y = 0.0, d_y = 0.0;"),
    ("scale_acc_fp64", "float n_s = 0.0f, d_s = 0.0f;\n    for (int y = 0;",
     "double n_s = 0.0, d_s = 0.0;\n    for (int y = 0;"),
    ("rows_bottom_up", "    for (int y = 0; y < h; y++) {\n        float n_y",
     "    for (int y = h - 1; y >= 0; y--) {\n        float n_y"),
    ("row_right_to_left",
     "        for (int x = 0; x < w; x++) {\n"
     "            const size_t i = (size_t)y * w + x;\n            n_y",
     "        for (int x = w - 1; x >= 0; x--) {\n"
     "            const size_t i = (size_t)y * w + x;\n            n_y"),
    ("one_accumulator_per_plane",
     "        n_s = n_s + n_y;\n        d_s = d_s + d_y;\n    }\n    *n_out",
     "        for (int x = 0; x < w; x++) {\n"
     "            n_s = n_s + num_t[(size_t)y * w + x];\n"
     "            d_s = d_s + den_t[(size_t)y * w + x];\n"
     "        }\n    }\n    *n_out"),
    ("totals_skip_scale1", "num = (double)N[0] + (double)N[1];",
     "num = (double)N[0] + (double)N[0];"),
    ("score_inverted", "out[s] = (double)N[s] / (double)D[s];",
     "out[s] = (double)D[s] / (double)N[s];"),
    # the option surface
    ("nsq_threshold_fp32", "if ((double)sigma1_sq < nsq) {",
     "if (sigma1_sq < (float)nsq) {"),
    ("num_nsq_fixed", "(double)sv_sq + nsq;", "(double)sv_sq + kNsq;"),
    ("den_nsq_fixed", "(double)sigma1_sq / nsq;", "(double)sigma1_sq / kNsq;"),
    ("gain_limit_ignored", "if (!((double)g < gain_limit))", "if (0)"),
    ("gain_limit_as_floor", "if (!((double)g < gain_limit))",
     "if ((double)g < gain_limit)"),
    ("gain_limit_before_sv",
     "    float g = sigma12 / sigma1_sq;\n",
     "    float g = sigma12 / sigma1_sq;\n"
     "    if (!((double)g < gain_limit))\n"
     "        g = (float)gain_limit;\n"),
    ("gain_limit_squared_twice", "const float g_sq = g * g;",
     "const float g_sq = (g < (float)gain_limit ? g * g : g);"),
    ("skip_wrong_scale", "if (s == 0 && opt->skip_scale0) {",
     "if (s == 1 && opt->skip_scale0) {"),
    ("skip_keeps_score0", "        out[0] = 0.0;\n", "        out[0] = out[0];\n"),
    ("skip_rows_kept", "rowsums[2 * (row_base + y)] = 0.0f;",
     "rowsums[2 * (row_base + y)] = 1.0f;"),
    ("floor_wrong_scale", "if (out[s] < opt->scale_min_val[s - 1])",
     "if (out[s] < opt->scale_min_val[s % 3])"),
    ("floor_as_cap", "if (out[s] < opt->scale_min_val[s - 1])",
     "if (out[s] > opt->scale_min_val[s - 1])"),
    ("kernelscale_unchecked", "if (o->kernelscale != 1.0)\n        return 0;",
     "if (o->kernelscale != o->kernelscale)\n        return 0;"),
]


# Mutants of the float SSIM oracle (fssim_oracle.c).
FSSIM_MUTANTS = [
    ("fs_scale_floor", "const int s = (int)round((double)m / 256.0);",
     "const int s = (int)floor((double)m / 256.0);"),
    ("fs_scale_by_max", "const int m = w < h ? w : h;",
     "const int m = w > h ? w : h;"),
    ("fs_size_no_odd", "return n / f + (n & 1);", "return n / f;"),
    ("fs_mirror_whole_sample", "        m = p - 1 - m;\n",
     "        m = p - 2 - m;\n"),
    ("fs_tap_wrong", "const float tap = 1.0f / (float)(f * f);",
     "const float tap = 1.0f / (float)(f * f + 1);"),
    ("fs_window_centred_odd", "const int hi = f / 2 - (f % 2 == 0 ? 1 : 0);",
     "const int hi = f / 2;"),
    ("fs_window_origin", "const int yy = fssimo_symmetric(y * f + dy, h);",
     "const int yy = fssimo_symmetric(y * f + dy + 1, h);"),
    ("fs_sum_fp32", "            double sum = 0.0;\n            for (int dy",
     "            float sum = 0.0f;\n            for (int dy"),
    ("fs_sigma_2", "const double sigma = 1.5;", "const double sigma = 2.0;"),
    ("fs_filter_no_vertical",
     "acc = acc + t[k] * src[(size_t)yy * w + x];",
     "acc = acc + t[k] * src[(size_t)y * w + x];"),
    ("fs_c2_wrong", "(float)((0.03 * 255.0) * (0.03 * 255.0));",
     "(float)((0.01 * 255.0) * (0.01 * 255.0));"),
    ("fs_sigma12_sign", "const float s12 = xy - m12;",
     "const float s12 = m12 - xy;"),
    ("fs_num_no_c1", "const float num = (2.0f * m12 + c1)",
     "const float num = (2.0f * m12)"),
    ("fs_mean_fp64", "out[0] = (double)(float)(total / (double)n);",
     "out[0] = total / (double)n;"),
    ("fs_ref_twice", "normalise(dist, w, h, bpc, Y0);",
     "normalise(ref, w, h, bpc, Y0);"),
    ("fs_no_decimation", "    if (f > 1) {\n        if (fssimo_decimate",
     "    if (f > 1000) {\n        if (fssimo_decimate"),
]


def _run(path):
    return subprocess.run([sys.executable, os.path.join(HERE,
                                                        "mutant_battery.py"),
                           path], capture_output=True, text=True, timeout=600)


FSSIM_SRC = os.path.join(ROOT, "oracle", "fssim_oracle.c")


def _build_mutant(tmp, name, old, new, fssim=False):
    import oracle
    src = open(FSSIM_SRC if fssim else SRC).read()
    assert src.count(old) >= 1, "mutation %s does not apply" % name
    mutated = src.replace(old, new, 1)
    cpath = os.path.join(tmp, name + ".c")
    with open(cpath, "w") as f:
        f.write(mutated)
    out = os.path.join(tmp, name + ".so")
    if fssim:
        return oracle.build(out=out, fssim_src=cpath)
    return oracle.build(src=cpath, out=out)


def test_real_oracle_passes_battery():
    import oracle
    oracle._load()
    r = _run(oracle._LIB)
    assert r.returncode == 0, r.stdout + r.stderr


def test_every_mutant_is_caught(tmp_path):
    tmp = str(tmp_path)
    libs = [(name, _build_mutant(tmp, name, old, new))
            for (name, old, new) in MUTANTS]
    libs += [(name, _build_mutant(tmp, name, old, new, fssim=True))
             for (name, old, new) in FSSIM_MUTANTS]
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda nl: (nl[0], _run(nl[1])), libs))
    survivors = [name for name, r in results if r.returncode == 0]
    assert not survivors, "mutants not caught by any pin: %s" % survivors
