"""Pins of the CPU oracle to what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: closed
forms, exact special cases, invariants, or a brute-force fp64 evaluation of
the definition in real arithmetic.  They are chosen so that a plausible
mistake (a dropped term, a wrong sign or index, a transposed operand, the
wrong mirror or decimation phase, wrong coefficients) fails at least one.
CPU only.
"""
import json
import math
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
FACTS = json.load(open(os.path.join(HERE, "golden", "page_facts.json")))

F32 = np.float32


def ulp32(x):
    x = abs(float(F32(x)))
    return float(np.spacing(F32(x)))


# ---------------------------------------------------------------- P1 / P1b

@pytest.mark.parametrize("bpc", [8, 10, 12, 16])
def test_normalise_exact_for_every_code(orc, bpc):
    """Research-2130, Sources: the normalised sample is v / divisor, exactly."""
    div = FACTS["normalisation_divisor"]["value"][str(bpc)]
    codes = np.arange(1 << bpc, dtype=np.uint8 if bpc == 8 else np.uint16)
    plane = codes.reshape(1, -1)
    x = orc.normalise(plane, bpc).astype(np.float64).ravel()
    assert np.array_equal(x * div, codes.astype(np.float64))


def test_normalise_rejects_bad_bpc(orc):
    with pytest.raises(ValueError):
        orc.normalise(np.zeros((2, 2), np.uint16), 9)


def test_cross_bit_depth_invariance(orc):
    """A 10/12/16-bit frame whose codes are 4/16/256 times an 8-bit frame's
    normalises to the same plane, so every output is bit-identical."""
    g = np.random.Generator(np.random.PCG64(11))
    ref8 = g.integers(0, 256, size=(40, 48)).astype(np.uint8)
    dist8 = np.clip(ref8.astype(np.int64) + g.integers(-20, 21, size=ref8.shape),
                    0, 255).astype(np.uint8)
    base, bsums = orc.score(ref8, dist8, 8)
    for bpc, mul in ((10, 4), (12, 16), (16, 256)):
        r = (ref8.astype(np.uint32) * mul).astype(np.uint16)
        d = (dist8.astype(np.uint32) * mul).astype(np.uint16)
        out, sums = orc.score(r, d, bpc)
        assert out.tobytes() == base.tobytes(), bpc
        assert sums.tobytes() == bsums.tobytes(), bpc


# --------------------------------------------------------------------- P2

def _indep_taps(n):
    """Independent fp64 Gaussian: 1/(2 sigma^2) = 25 / (2 n^2), fsum."""
    r = (n - 1) // 2
    g = [math.exp(-12.5 * (k - r) ** 2 / (n * n)) for k in range(n)]
    s = math.fsum(g)
    return [v / s for v in g]


@pytest.mark.parametrize("scale", [0, 1, 2, 3])
def test_taps_closed_form(orc, scale):
    t = orc.taps(scale)
    n = FACTS["filter_widths"]["value"][scale]
    assert len(t) == n
    r = (n - 1) // 2
    # symmetric, bitwise
    assert t.tobytes() == t[::-1].tobytes()
    # unimodal, peak at the centre
    assert all(t[k] < t[k + 1] for k in range(r))
    # sums to one within n roundings
    assert abs(math.fsum(float(v) for v in t) - 1.0) <= n * 2.0 ** -24
    # each tap is the fp32 rounding of an independent fp64 evaluation
    ref = _indep_taps(n)
    for k in range(n):
        assert abs(float(t[k]) - ref[k]) <= 0.5 * ulp32(t[k]) * (1 + 1e-9), k


def test_taps_bad_scale(orc):
    with pytest.raises(ValueError):
        orc.taps(4)


# --------------------------------------------------------------------- P3

@pytest.mark.parametrize("scale", [0, 1, 2, 3])
@pytest.mark.parametrize("v", [1.0, 3.0, 255.0, 0.74609375])
def test_filter_interior_impulse(orc, scale, v):
    """An impulse of height v at (y0, x0) filters to
    fl32(t[x0-x+r] * fl32(t[y0-y+r] * v)): vertical pass first, then
    horizontal; everything else exactly zero."""
    t = orc.taps(scale)
    n = len(t)
    r = (n - 1) // 2
    h, w = 37, 41
    y0, x0 = 18, 21
    P = np.zeros((h, w), np.float32)
    P[y0, x0] = F32(v)
    Q = orc.filter2d(P, t)
    E = np.zeros((h, w), np.float32)
    for y in range(y0 - r, y0 + r + 1):
        vy = F32(t[y0 - y + r] * F32(v))
        for x in range(x0 - r, x0 + r + 1):
            E[y, x] = F32(t[x0 - x + r] * vy)
    assert Q.tobytes() == E.tobytes()


def test_filter_order_is_vertical_then_horizontal(orc):
    """With off-centre taps the two product orders round differently for
    some v; the oracle must match the vertical-first order everywhere and
    differ from the horizontal-first order somewhere."""
    t = orc.taps(0)
    r = 8
    h, w = 37, 41
    y0, x0 = 18, 21
    diffs = 0
    for v in np.linspace(1.0, 255.0, 97, dtype=np.float32):
        P = np.zeros((h, w), np.float32)
        P[y0, x0] = v
        Q = orc.filter2d(P, t)
        for dy in range(-r, r + 1):
            for dx in range(-r, r + 1):
                vert = F32(t[r + dx] * F32(t[r + dy] * v))
                horz = F32(t[r + dy] * F32(t[r + dx] * v))
                got = Q[y0 - dy, x0 - dx]
                assert got == vert
                diffs += int(vert != horz)
    assert diffs > 0


@pytest.mark.parametrize("scale", [0, 1, 2, 3])
def test_filter_whole_sample_mirror(orc, scale):
    """Impulse next to the left (top) edge: output column (row) 0 reads the
    sample at index 1 twice under whole-sample reflection (-1 -> 1), so it
    is exactly 2 fl32(t[r+1] * V); half-sample reflection would read it
    once."""
    t = orc.taps(scale)
    n = len(t)
    r = (n - 1) // 2
    h, w = 20, 24
    v = F32(200.0)
    P = np.zeros((h, w), np.float32)
    P[10, 1] = v
    Q = orc.filter2d(P, t)
    Vc = F32(t[r] * v)  # vertical pass at row 10, column 1
    assert Q[10, 0] == F32(2.0) * F32(t[r + 1] * Vc)
    P = np.zeros((h, w), np.float32)
    P[1, 10] = v
    Q = orc.filter2d(P, t)
    Vt = F32(2.0) * F32(t[r + 1] * v)  # vertical pass at row 0, column 10
    assert Q[0, 10] == F32(t[r] * Vt)


def test_filter_right_bottom_mirror(orc):
    """Impulse at column w-2: output column w-1 reads it twice."""
    t = orc.taps(1)
    r = 4
    h, w = 18, 19
    v = F32(77.0)
    P = np.zeros((h, w), np.float32)
    P[9, w - 2] = v
    Q = orc.filter2d(P, t)
    assert Q[9, w - 1] == F32(2.0) * F32(t[r + 1] * F32(t[r] * v))
    P = np.zeros((h, w), np.float32)
    P[h - 2, 9] = v
    Q = orc.filter2d(P, t)
    assert Q[h - 1, 9] == F32(t[r] * F32(F32(2.0) * F32(t[r + 1] * v)))


# --------------------------------------------------------------------- P4

def _conv_fp64(P, t):
    """Brute-force 2-D convolution in fp64 with whole-sample reflection
    (numpy's 'reflect' padding), taps taken as exact values."""
    P = np.asarray(P, np.float64)
    t = np.asarray(t, np.float64)
    n = len(t)
    r = (n - 1) // 2
    h, w = P.shape
    A = np.pad(P, r, mode="reflect")
    out = np.zeros((h, w), np.float64)
    for i in range(n):
        for j in range(n):
            out += t[i] * t[j] * A[i:i + h, j:j + w]
    return out


@pytest.mark.parametrize("shape", [(16, 16), (23, 17), (16, 40)])
@pytest.mark.parametrize("scale", [0, 1, 2, 3])
def test_filter_vs_fp64_bruteforce(orc, shape, scale):
    """fp32 separable filter within 1e-6 of the exact 2-D convolution,
    relative to sum |t_i t_j P| (rigorous bound (2N+1) 2^-24)."""
    g = np.random.Generator(np.random.PCG64(100 + scale))
    P = g.integers(0, 256, size=shape).astype(np.float32)
    t = orc.taps(scale)
    Q = orc.filter2d(P, t).astype(np.float64)
    E = _conv_fp64(P, t)
    S = _conv_fp64(np.abs(P), np.abs(t))
    rel = np.max(np.abs(Q - E) / S)
    assert rel <= 1e-6, rel


@pytest.mark.parametrize("scale", [1, 2, 3])
def test_decimate_vs_fp64_bruteforce(orc, scale):
    g = np.random.Generator(np.random.PCG64(200 + scale))
    P = (g.integers(0, 65536, size=(23, 17)) / 256.0).astype(np.float32)
    t = orc.taps(scale)
    D = orc.decimate(P, t).astype(np.float64)
    assert D.shape == (11, 8)
    E = _conv_fp64(P, t)[0::2, 0::2][:11, :8]
    S = _conv_fp64(np.abs(P), np.abs(t))[0::2, 0::2][:11, :8]
    assert np.max(np.abs(D - E) / S) <= 1e-6


def test_decimate_even_phase_impulse(orc):
    """An impulse at an even position (2a, 2b) lands centred on (a, b); one at
    an odd position does not reach any output with the centre tap."""
    t = orc.taps(1)
    r = 4
    v = F32(100.0)
    P = np.zeros((20, 22), np.float32)
    P[8, 10] = v
    D = orc.decimate(P, t)
    assert D.shape == (10, 11)
    assert D[4, 5] == F32(t[r] * F32(t[r] * v))
    assert D[4, 4] == F32(t[r + 2] * F32(t[r] * v))
    assert D[3, 5] == F32(t[r] * F32(t[r + 2] * v))
    P = np.zeros((20, 22), np.float32)
    P[9, 11] = v
    D = orc.decimate(P, t)
    assert D[4, 5] == F32(t[r - 1] * F32(t[r - 1] * v))
    assert np.max(D) < F32(t[r] * F32(t[r] * v))


# --------------------------------------------------------------------- P5

@pytest.mark.parametrize("w", list(range(16, 160)))
def test_pyramid_floor_sizes_match_small_frame_bound(w, orc):
    """Floor halving: the scale-3 width w//8 is below nine exactly when the
    frame is below 72 px (ADR-1444, Context)."""
    bound = FACTS["small_frame_fault_bound"]["value"]
    nine = FACTS["scale3_min_samples"]["value"]
    w3 = ((w // 2) // 2) // 2
    assert (w3 < nine) == (w < bound)


@pytest.mark.parametrize("wh", [(16, 16), (17, 23), (40, 40), (73, 41),
                                (576, 324)])
def test_flat_frame_sums_are_pixel_counts(orc, wh):
    """P10: a flat frame against itself puts every pixel in the low-variance
    branch, so each row sum is the row's width and each scale's sums are
    w_s * h_s, all exact integers below 2^24."""
    w, h = wh
    f = np.full((h, w), 117, np.uint8)
    out, sums, rows = orc.score(f, f, 8, want_rows=True)
    ws, hs, base = w, h, 0
    for s in range(4):
        assert sums[2 * s] == ws * hs and sums[2 * s + 1] == ws * hs
        assert np.all(rows[base:base + hs] == ws)
        base += hs
        ws, hs = ws // 2, hs // 2
    assert rows.shape[0] == base


# -------------------------------------------------------------- P10 / O9

# Two crafted 4x4 term planes whose ordered fp32 sums are closed forms.
# fp32 holds every integer up to 2^24 = 16777216; above it the spacing is 2
# (4 above 2^25), and round-to-nearest-even sends a tie to the neighbour
# whose last significand bit is 0, i.e. the multiple of 4 here.
#   num row 0  [2^24, 1, 1, 1]: each 2^24 + 1 is a tie, kept at 2^24.
#   num row 1  [1, 1, 1, 1]: 4, exactly.
#   num row 2  [1, 1, 1, 2^24]: 3 + 2^24 = 16777219 is a tie, 16777220.
#   num row 3  zeros.
#   N = 2^24 + 4, then + 16777220 = 2^25 + 8 (a multiple of 4, exact), + 0.
#   den rows   [2^24, 0, 0, 0], then three rows [1, 0, 0, 0]: row sums
#              2^24, 1, 1, 1; top to bottom each + 1 is a tie kept at
#              2^24, so D = 2^24.
# Mistakes this separates: rows added right to left (num row 0 gives
# 2^24 + 4), rows or the plane accumulated in fp64 (2^24 + 3 rounds to
# 2^24 + 4 when stored), rows summed bottom to top (D = 2^24 + 4), one
# accumulator for the whole plane (N = 2^25).
P24 = float(1 << 24)
SUM_NUM = np.array([[P24, 1, 1, 1], [1, 1, 1, 1], [1, 1, 1, P24],
                    [0, 0, 0, 0]], dtype=np.float32)
SUM_DEN = np.array([[P24, 0, 0, 0], [1, 0, 0, 0], [1, 0, 0, 0],
                    [1, 0, 0, 0]], dtype=np.float32)
SUM_ROWS = np.array([[16777216.0, 16777216.0], [4.0, 1.0],
                     [16777220.0, 1.0], [0.0, 1.0]], dtype=np.float32)
SUM_N = np.float32(33554440.0)
SUM_D = np.float32(16777216.0)


def test_ordered_sums_closed_form(orc):
    """O9 (ADR-1422 Context and Decision): one fp32 accumulator per row from
    zero, terms left to right, then the row sums top to bottom in fp32."""
    rows, n, d = orc.ordered_sums(SUM_NUM, SUM_DEN)
    assert np.array_equal(rows, SUM_ROWS)
    assert n == SUM_N and d == SUM_D
    # each plane alone: the num rows' sums with zero den terms, and so on
    rows2, n2, d2 = orc.ordered_sums(SUM_DEN, SUM_NUM)
    assert np.array_equal(rows2, SUM_ROWS[:, ::-1])
    assert n2 == SUM_D and d2 == SUM_N


def test_ordered_sums_rounding_accumulates_past_2_24(orc):
    """O9 over many rows: a 3 x 2^23 plane of ones has row sums 3.  The
    running fp32 total is exact up to 3 * 5592405 = 2^24 - 1; from there an
    odd partial sum lies halfway between two representable even integers,
    and RNE takes the multiple of 4, so every further row adds 4 (or 2 once)
    and the total is not 3 * 2^23, which fp32 holds exactly."""
    h = 1 << 23
    ones = np.ones((h, 3), dtype=np.float32)
    rows, n, d = orc.ordered_sums(ones, ones)
    assert np.all(rows == 3.0)
    # the running total in fp32, row by row: below 2^24 every partial sum
    # 3k is exact; at and above it, S + 3 is odd, so fl32 goes to the
    # neighbour that is a multiple of 4 (S is even there)
    s = 0
    for _ in range(h):
        t = s + 3
        if t > (1 << 24) and t % 2 == 1:
            t = t - 1 if (t - 1) % 4 == 0 else t + 1
        s = t
    assert float(n) == float(s) == float(d)
    assert s != 3 * h


def test_frame_sums_round_in_fp32_past_2_24(orc):
    """O9 through the whole feature: with a noise variance of 1e30 every
    pixel takes the low-variance branch, so every term is exactly 1 and
    each scale-0 row sums to w = 1023 exactly.  The frame has 1023 x 16500 >
    2^24 pixels: the top-to-bottom fp32 total is exact up to row 16400
    (16777200) and from there each odd partial sum is a tie that RNE sends
    to the multiple of 4.  N_0 and D_0 must be that total, not w * h."""
    w, h = 1023, 16500
    g = np.random.Generator(np.random.PCG64(11))
    r = g.integers(0, 256, size=(h, w), dtype=np.uint8)
    out, sums, rows = orc.score(r, r, 8, want_rows=True,
                                options={"sigma_nsq": 1e30})
    assert np.all(rows[:h] == w)
    s = 0
    for _ in range(h):
        t = s + w
        if t > (1 << 24) and t % 2 == 1:
            t = t - 1 if (t - 1) % 4 == 0 else t + 1
        s = t
    assert s != w * h
    assert float(sums[0]) == float(s) and float(sums[1]) == float(s)
    # scale 1 has 511 x 8250 < 2^24 pixels: its sums are exact
    assert float(sums[2]) == 511 * 8250 == float(sums[3])


# --------------------------------------------------------------------- P7

@pytest.mark.parametrize("bpc,val", [(8, 0), (8, 128), (8, 255), (10, 1023),
                                     (12, 2049), (16, 65535), (16, 49152)])
def test_flat_frame_scores_exactly_one(orc, bpc, val):
    dt = np.uint8 if bpc == 8 else np.uint16
    f = np.full((36, 52), val, dt)
    out, sums = orc.score(f, f, bpc)
    assert np.all(out[:7] == 1.0) or (out[4] == out[5] and
                                       np.all(out[:4] == 1.0))
    assert out[6] == 1.0
    assert out[7] == 0.0


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_reference_against_itself(orc, seed):
    """X = Y: g = 1 and sv clamps to eps, so each term pair differs only by
    the eps in the denominator: |num - den| <= 1e-6 den."""
    g = np.random.Generator(np.random.PCG64(seed))
    r = g.integers(0, 256, size=(48, 64)).astype(np.uint8)
    out, sums = orc.score(r, r, 8)
    assert abs(out[4] - out[5]) <= 1e-6 * out[5]
    for s in range(4):
        assert abs(out[s] - 1.0) <= 1e-6


def test_statistic_low_variance_branch(orc):
    # sigma1_sq = 101 - 100 = 1 < 2
    assert orc.statistic(10.0, 3.0, 101.0, 50.0, 31.0) == (1.0, 1.0)
    # negative sigma1_sq clamps to 0 -> low branch
    assert orc.statistic(10.0, 3.0, 99.0, 50.0, 31.0) == (1.0, 1.0)
    # just below 2 (fp32 value under 2.0)
    s = np.nextafter(F32(2.0), F32(0.0))
    assert orc.statistic(0.0, 0.0, s, 5.0, 0.0) == (1.0, 1.0)


def test_statistic_threshold_is_inclusive_high(orc):
    """sigma1_sq == 2 exactly takes the high branch: den = log2(1 + 1) = 1."""
    n, d = orc.statistic(0.0, 0.0, 2.0, 0.0, 0.0)
    assert d == F32(1.0)
    assert n == F32(0.0)  # sigma2_sq = 0 -> g = 0 -> 1 + 0


def test_statistic_zero_distorted_variance(orc):
    """sigma2_sq = 0 with sigma1_sq >= 2: g = 0, so the numerator is
    log2(1) = 0 exactly; the denominator is log2(1 + sigma1_sq / 2)."""
    n, d = orc.statistic(10.0, 5.0, 150.0, 25.0, 60.0)  # s1 = 50, s2 = 0
    assert n == F32(0.0)
    assert abs(float(d) - math.log2(1.0 + 50.0 / 2.0)) <= 2e-7 * 5


def test_statistic_negative_gain(orc):
    """sigma12 < 0 gives g < 0 -> g = 0 -> numerator term 0."""
    n, d = orc.statistic(10.0, 10.0, 200.0, 200.0, 50.0)  # s12 = -50
    assert n == F32(0.0)
    assert abs(float(d) - math.log2(1.0 + 100.0 / 2.0)) <= 1e-6


def test_statistic_vs_fp64_formula(orc):
    """Over random high-branch inputs the terms equal log2 of the fp64
    one-plus-ratio values built from the fp32 sigmas, to within the
    polynomial bound plus the fp32 rounding of the argument."""
    g = np.random.Generator(np.random.PCG64(7))
    worst = 0.0
    for _ in range(3000):
        mu1 = F32(g.uniform(0, 255))
        mu2 = F32(g.uniform(0, 255))
        s1 = g.uniform(2.0, 5000.0)
        s2 = g.uniform(0.0, 5000.0)
        rho = g.uniform(-1.0, 1.0)
        s12 = rho * math.sqrt(s1 * s2)
        xx = F32(F32(mu1 * mu1) + F32(s1))
        yy = F32(F32(mu2 * mu2) + F32(s2))
        xy = F32(F32(mu1 * mu2) + F32(s12))
        n, d = orc.statistic(mu1, mu2, xx, yy, xy)
        # the fp32 sigmas exactly as the definition forms them
        S1 = max(F32(xx - F32(mu1 * mu1)), F32(0))
        S2 = max(F32(yy - F32(mu2 * mu2)), F32(0))
        S12 = F32(xy - F32(mu1 * mu2))
        if float(S1) < 2.0:
            assert (n, d) == (1.0, 1.0)
            continue
        gg = float(S12) / float(S1)
        sv = float(S2) - gg * float(S12)
        if float(S2) < 1e-10:
            gg, sv = 0.0, 0.0
        if gg < 0:
            gg, sv = 0.0, float(S2)
        sv = max(sv, 1e-10)
        en = math.log2(1.0 + gg * gg * float(S1) / (sv + 2.0))
        ed = math.log2(1.0 + float(S1) / 2.0)
        # the num term goes through fp32 g, g*s12, g*g, (g*g)*s1: a few
        # relative ulps of the argument; log2 of 1+q turns a relative error
        # e of q into <= e*q/((1+q) ln 2)
        assert abs(float(d) - ed) <= 1.7e-7 + 0.5 * ulp32(d) + 1e-7 * ed
        tol_n = 1.7e-7 + 0.5 * ulp32(n) + 1e-5 * max(en, 1e-3) + 1e-6
        worst = max(worst, abs(float(n) - en) - tol_n)
        assert abs(float(n) - en) <= tol_n
    assert worst <= 0


def _rne32_extended(a, sv, nsq=2.0):
    """fp32 rounding of 1 + a/(sv + nsq) from x87 extended precision (64-bit
    significand), plus a flag for values within 2^-50 (relative) of an fp32
    rounding midpoint, where one fp64 rounding before the fp32 one may
    legitimately land on the other side."""
    ld = np.longdouble
    e = ld(1) + a.astype(ld) / (sv.astype(ld) + ld(nsq))
    f = e.astype(np.float32)
    up = np.nextafter(f, np.float32(np.inf))
    dn = np.nextafter(f, np.float32(0))
    m_up = (f.astype(ld) + up.astype(ld)) / 2
    m_dn = (f.astype(ld) + dn.astype(ld)) / 2
    tol = e * ld(2.0) ** -50
    near = (np.abs(e - m_up) < tol) | (np.abs(e - m_dn) < tol)
    return f, near


def test_num_ratio_vs_extended_precision(orc):
    """fl32(1 + a/(sv + nsq)) through fp64 equals the single fp32 rounding of
    the (extended-precision) real value except within 2^-50 of a midpoint.
    Catches an fp32 nsq, an fp32 quotient or a different rounding sequence
    (ADR-1422, Context: the expression is evaluated in fp64 and rounded to
    fp32 once)."""
    g = np.random.Generator(np.random.PCG64(21))
    n = 1 << 21
    a = np.exp(g.uniform(np.log(1e-6), np.log(5e8), n)).astype(np.float32)
    sv = np.exp(g.uniform(np.log(1e-10), np.log(1e5), n)).astype(np.float32)
    sv[:1000] = np.float32(1e-10)
    a[1000:2000] = 0
    num, _ = orc.ratios(a, sv)
    ref, near = _rne32_extended(a, sv)
    bad = (num != ref) & ~near
    assert not bad.any(), (a[bad][:5], sv[bad][:5], num[bad][:5], ref[bad][:5])
    assert near.sum() < n // 10000
    assert np.all(num[1000:2000] == 1.0)


def test_den_ratio_closed_form(orc):
    """With nsq = 2 the denominator value is one fp32 rounding of
    1 + sigma1_sq / 2: sigma1_sq / 2 is exact and 1 + sigma1_sq / 2 fits 53
    bits, so fl32(fl64(1 + fl64(s / 2))) = fl32(1 + s * 0.5) in fp32."""
    g = np.random.Generator(np.random.PCG64(22))
    s1 = np.exp(g.uniform(np.log(2.0), np.log(2.0 ** 40), 1 << 21))
    s1 = s1.astype(np.float32)
    _, den = orc.ratios(s1, np.ones_like(s1))
    closed = (np.float32(1) + (s1 * np.float32(0.5)).astype(np.float32))
    assert np.array_equal(den, closed.astype(np.float32))
    ref, near = _rne32_extended(s1, np.zeros_like(s1))
    assert np.array_equal(den[~near], ref[~near])


# --------------------------------------------------------------------- P8

def _checker(h, w, shift, lo=64, hi=940, sq=10):
    y = np.arange(h)[:, None]
    x = np.arange(w)[None, :] - shift
    return np.where(((x // sq) + (y // sq)) % 2 == 0, lo, hi)


def test_checkerboard_translation_symmetry(orc):
    """Shifting a 64/940 checkerboard by one square maps every sample v to
    1004 - v; local variances and covariances are unchanged, so the scores
    agree to fp32 noise.  Shifting by a whole period (20 px) leaves the
    frames, hence every output bit, unchanged.  The fp32 taps sum to
    1 + delta with |delta| <= 17 * 2^-24, which breaks the invariance by
    about c^2 delta in each variance (c = 251 here): 1e-5 relative bounds
    that, while a missing mean subtraction moves scores by O(1)."""
    h, w = 120, 200
    g = np.random.Generator(np.random.PCG64(5))
    noise = g.normal(0, 2.0, size=(h, w))
    ref = _checker(h, w, 0)
    dist = np.clip(np.rint(_checker(h, w, 1) + noise), 0, 1023)
    a, _ = orc.score(ref.astype(np.uint16), dist.astype(np.uint16), 10)
    ref10 = _checker(h, w, 10)
    dist10 = 1004 - dist
    assert np.array_equal(ref10, 1004 - ref)
    b, _ = orc.score(ref10.astype(np.uint16), dist10.astype(np.uint16), 10)
    assert np.all(np.abs(a[:4] - b[:4]) <= 1e-5 * np.abs(a[:4]))
    c, _ = orc.score(_checker(h, w, 20).astype(np.uint16),
                     dist.astype(np.uint16), 10)
    assert c.tobytes() == a.tobytes()


def test_intensity_reflection_symmetry_random(orc):
    """The same invariance on textured frames: v -> 255 - v in both.  At
    scale 3 (8x10 samples) the variances are small after three low-passes,
    so the c^2 delta breakage is relatively larger: 2e-4 there, 1e-5 at
    scales 0-2; a missing mean subtraction moves scores by O(1)."""
    g = np.random.Generator(np.random.PCG64(6))
    r = g.integers(0, 256, size=(64, 80))
    d = np.clip(r + g.integers(-30, 31, size=r.shape), 0, 255)
    a, _ = orc.score(r.astype(np.uint8), d.astype(np.uint8), 8)
    b, _ = orc.score((255 - r).astype(np.uint8), (255 - d).astype(np.uint8), 8)
    tol = np.array([1e-5, 1e-5, 1e-5, 2e-4])
    assert np.all(np.abs(a[:4] - b[:4]) <= tol * np.abs(a[:4]))


# --------------------------------------------------------------------- P9

LOG2_BOUND = 1.7e-7  # max |L(x) - log2(x)| over x in [1, 2), measured


def test_log2_powers_of_two_exact(orc):
    for k in range(0, 32):
        assert orc.log2(F32(2.0 ** k)) == F32(k)


def test_log2_exhaustive_first_binade(orc):
    """All 2^23 fp32 values in [1, 2): within the frozen bound of log2."""
    m = np.arange(1 << 23, dtype=np.uint32)
    x = (m | np.uint32(0x3F800000)).view(np.float32)
    L = orc.log2_array(x).astype(np.float64)
    err = np.abs(L - np.log2(x.astype(np.float64)))
    assert err.max() <= LOG2_BOUND, err.max()
    # monotone up to one ulp of wobble
    assert np.all(np.diff(L) >= -1.2e-7)


@pytest.mark.parametrize("e", [1, 2, 5, 9, 16, 23, 31])
def test_log2_other_binades(orc, e):
    """L(2^e (1 + t)) = fl32(e + L(1 + t)): error <= bound + half an ulp."""
    g = np.random.Generator(np.random.PCG64(e))
    m = g.integers(0, 1 << 23, size=200000, dtype=np.uint32)
    x = ((np.uint32(127 + e) << np.uint32(23)) | m).view(np.float32)
    L = orc.log2_array(x).astype(np.float64)
    exact = np.log2(x.astype(np.float64))
    half_ulp = 0.5 * np.spacing(L.astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(L - exact) <= LOG2_BOUND + half_ulp)
    base = orc.log2_array(((np.uint32(127) << np.uint32(23)) | m)
                          .view(np.float32))
    assert np.array_equal(L.astype(np.float32),
                          (F32(e) + base).astype(np.float32))


def test_log2_coefficients_are_the_fit(orc):
    """The oracle's frozen coefficients are what oracle/fit_log2.py produces:
    Horner with the fitted fp32 coefficients reproduces the oracle bitwise."""
    from oracle import fit_log2
    c = fit_log2.fit_coefficients()
    assert len(c) == 10
    m = np.arange(0, 1 << 23, 7, dtype=np.uint32)
    x = (m | np.uint32(0x3F800000)).view(np.float32)
    t = (x - F32(1)).astype(np.float32)
    p = np.full_like(t, c[-1])
    for k in range(len(c) - 2, -1, -1):
        p = ((p * t).astype(np.float32) + c[k]).astype(np.float32)
    q = (p * t).astype(np.float32)
    assert np.array_equal(q, orc.log2_array(x))


# ------------------------------------------------------ whole pipeline fp64

def _vif_fp64(ref, dist, bpc, nsq=2.0, gain_limit=np.inf):
    """The whole definition in real (fp64) arithmetic with exact log2 and
    numpy reflection padding: no fp32 rounding anywhere except the taps.
    The gain limit bounds g where it enters the numerator."""
    div = 2.0 ** (bpc - 8)
    X = ref.astype(np.float64) / div
    Y = dist.astype(np.float64) / div
    N, D = [], []
    for s in range(4):
        n = (17, 9, 5, 3)[s]
        t = np.asarray(_indep_taps(n), np.float64)
        if s > 0:
            h, w = X.shape
            X = _conv_fp64(X, t)[0::2, 0::2][:h // 2, :w // 2]
            Y = _conv_fp64(Y, t)[0::2, 0::2][:h // 2, :w // 2]
        mu1, mu2 = _conv_fp64(X, t), _conv_fp64(Y, t)
        s1 = np.maximum(_conv_fp64(X * X, t) - mu1 * mu1, 0)
        s2 = np.maximum(_conv_fp64(Y * Y, t) - mu2 * mu2, 0)
        s12 = _conv_fp64(X * Y, t) - mu1 * mu2
        hi = s1 >= nsq
        near = np.abs(s1 - nsq) < 1e-3
        assert not near.any()
        with np.errstate(divide="ignore", invalid="ignore"):
            g = np.where(hi, s12 / np.where(hi, s1, 1), 0)
        sv = s2 - g * s12
        lo2 = s2 < 1e-10
        g = np.where(lo2, 0, g)
        sv = np.where(lo2, 0, sv)
        neg = g < 0
        sv = np.where(neg, s2, sv)
        g = np.where(neg, 0, g)
        sv = np.maximum(sv, 1e-10)
        g = np.minimum(g, gain_limit)
        num = np.where(hi, np.log2(1 + g * g * s1 / (sv + nsq)), 1.0)
        den = np.where(hi, np.log2(1 + s1 / nsq), 1.0)
        N.append(num.sum())
        D.append(den.sum())
    out = [N[s] / D[s] for s in range(4)]
    return np.array(out + [sum(N), sum(D), sum(N) / sum(D)])


@pytest.mark.parametrize("shape,seed", [((32, 32), 1), ((40, 56), 2),
                                        ((41, 73), 3), ((16, 16), 4),
                                        ((64, 64), 5), ((48, 80), 6)])
def test_pipeline_vs_fp64_definition(orc, shape, seed):
    """Scores agree with an fp64 evaluation of the definition: catches a
    dropped term, a wrong scale's taps, a wrong decimation, a swapped
    ref/dist or a wrong sign anywhere on the path.  The fp32 cancellation in
    sigma^2 = xx - mu^2 costs about ulp(mu^2) / sigma^2 relative, which
    grows at the coarse scales where the planes are small and smooth, so the
    bound widens with the scale (measured worst 1.5e-4 at scale 3)."""
    g = np.random.Generator(np.random.PCG64(seed))
    r = g.integers(0, 256, size=shape).astype(np.uint8)
    d = np.clip(r.astype(np.int64) + g.integers(-40, 41, size=shape),
                0, 255).astype(np.uint8)
    got, _ = orc.score(r, d, 8)
    exp = _vif_fp64(r, d, 8)
    rel = np.abs(got[:7] - exp) / np.abs(exp)
    tol = np.array([2e-6, 1e-4, 3e-4, 5e-4, 2e-5, 2e-6, 2e-5])
    assert np.all(rel <= tol), (rel, got[:7], exp)
    # and a swapped pair really differs (ref and dist are not symmetric)
    sw, _ = orc.score(d, r, 8)
    assert abs(sw[0] - got[0]) > 1e-3


# ----------------------------------------------------------------- P11, misc

@pytest.mark.parametrize("wh", [(16, 16), (40, 40), (56, 56), (64, 64),
                                (71, 71), (73, 41), (16, 200), (200, 16)])
def test_small_frames_run(orc, wh):
    w, h = wh
    g = np.random.Generator(np.random.PCG64(w * 1000 + h))
    r = g.integers(0, 256, size=(h, w)).astype(np.uint8)
    d = g.integers(0, 256, size=(h, w)).astype(np.uint8)
    out, sums = orc.score(r, d, 8)
    assert np.all(np.isfinite(out))
    assert np.all(sums[1::2] > 0)


@pytest.mark.parametrize("wh", [(15, 16), (16, 15), (8, 100)])
def test_too_small_rejected(orc, wh):
    w, h = wh
    f = np.zeros((h, w), np.uint8)
    with pytest.raises(ValueError):
        orc.score(f, f, 8)


def test_bad_bpc_rejected(orc):
    f = np.zeros((16, 16), np.uint16)
    with pytest.raises(ValueError):
        orc.score(f, f, 9)
