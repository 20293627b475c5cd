"""Pins of the oracle's option surface: vif_sigma_nsq, vif_enhn_gain_limit,
vif_skip_scale0, vif_scale1..3_min_val and vif_kernelscale.

The pages name these options (ADR-1422 Decision and Consequences; ADR-1444
Decision and Consequences) without printing their arithmetic; the oracle's
readings are in vif_oracle.h.  Each test checks the oracle against
something other than itself: closed forms (every pixel in one branch, a
zero gain), exact special cases of IEEE arithmetic (a zero noise variance),
extended-precision roundings, an fp64 evaluation of the definition, and
invariants (a gain limit that no gain reaches, the scales a skip leaves
untouched).  CPU only.
"""
import math

import numpy as np
import pytest

import test_oracle_pins as P

F32 = np.float32


def _frame(seed, shape=(48, 64), spread=40):
    g = np.random.Generator(np.random.PCG64(seed))
    r = g.integers(0, 256, size=shape).astype(np.uint8)
    d = np.clip(r.astype(np.int64) + g.integers(-spread, spread + 1,
                                                size=shape),
                0, 255).astype(np.uint8)
    return r, d


def _pixels(w, h):
    n = []
    for _ in range(4):
        n.append(w * h)
        w, h = w // 2, h // 2
    return n


# ------------------------------------------------------- sigma_nsq (nsq)

def test_default_options_equal_default_entry(orc):
    r, d = _frame(1)
    a, sa, ra = orc.score(r, d, 8, want_rows=True)
    b, sb, rb = orc.score(r, d, 8, want_rows=True, options={})
    assert a.tobytes() == b.tobytes()
    assert sa.tobytes() == sb.tobytes() and ra.tobytes() == rb.tobytes()


def test_huge_nsq_puts_every_pixel_in_the_low_branch(orc):
    """Every sigma1_sq is below nsq = 1e30, so both terms are 1 on every
    pixel: the sums are the pixel counts and every score is exactly 1."""
    r, d = _frame(2, (41, 57))
    out, sums = orc.score(r, d, 8, options={"sigma_nsq": 1e30})
    counts = _pixels(57, 41)
    assert list(sums[0::2]) == counts and list(sums[1::2]) == counts
    assert np.all(out[:4] == 1.0) and out[6] == 1.0
    assert out[4] == out[5] == float(sum(counts))


@pytest.mark.parametrize("nsq", [2.0, 1.5, 4.7, 0.3])
def test_nsq_threshold_is_an_fp64_comparison(orc, nsq):
    """With mu1 = 0 the fp32 sigma1_sq is xx itself, so the branch can be
    probed at the fp32 neighbours of nsq.  The comparison is in fp64
    (ADR-1422, Decision: sigma1_sq < vif_sigma_nsq is a comparison of the
    reference's doubles): the nearest fp32 below nsq, and fl32(nsq) when it
    lies below nsq, take the low branch; the first fp32 at or above nsq
    takes the high one."""
    lo = F32(nsq)
    if float(lo) >= nsq:
        lo = np.nextafter(lo, F32(0))
    hi = np.nextafter(lo, F32(np.inf))
    assert float(lo) < nsq <= float(hi)
    # sigma12 = 0: the high branch has gain 0 and a numerator term of
    # exactly log2(1) = 0, the low branch exactly 1
    n, d = orc.statistic(0.0, 0.0, lo, 7.0, 0.0, nsq=nsq)
    assert (n, d) == (1.0, 1.0)
    n, d = orc.statistic(0.0, 0.0, hi, 7.0, 0.0, nsq=nsq)
    assert n == 0.0 and d >= 1.0
    if float(F32(nsq)) < nsq:           # 1.5 and 2.0 are exact; 4.7 is not
        n, d = orc.statistic(0.0, 0.0, F32(nsq), 7.0, 0.0, nsq=nsq)
        assert (n, d) == (1.0, 1.0)


@pytest.mark.parametrize("nsq", [1.5, 4.7, 0.5, 1e-3])
def test_num_ratio_with_nsq_vs_extended_precision(orc, nsq):
    """fl32(1 + a/(sv + nsq)) through fp64 equals the fp32 rounding of the
    extended-precision value away from rounding midpoints, for any nsq
    (ADR-1422, Context: nsq stays a double; Decision: fp64 sum, quotient,
    sum with one, one conversion)."""
    g = np.random.Generator(np.random.PCG64(31))
    n = 1 << 19
    a = np.exp(g.uniform(np.log(1e-6), np.log(5e8), n)).astype(np.float32)
    sv = np.exp(g.uniform(np.log(1e-10), np.log(1e5), n)).astype(np.float32)
    num, _ = orc.ratios(a, sv, nsq=nsq)
    ref, near = P._rne32_extended(a, sv, nsq)
    bad = (num != ref) & ~near
    assert not bad.any(), (a[bad][:4], sv[bad][:4])
    assert near.sum() < n // 10000


@pytest.mark.parametrize("nsq", [1.5, 4.7, 0.5, 3.0])
def test_den_ratio_with_nsq_vs_extended_precision(orc, nsq):
    """fl32(1 + s/nsq) through fp64 against the extended-precision value;
    for the default-entry value nsq = 2 see test_den_ratio_closed_form."""
    g = np.random.Generator(np.random.PCG64(32))
    s1 = np.exp(g.uniform(np.log(nsq), np.log(2.0 ** 30), 1 << 19))
    s1 = s1.astype(np.float32)
    _, den = orc.ratios(s1, np.ones_like(s1), nsq=nsq)
    ref, near = P._rne32_extended(s1, np.zeros_like(s1), nsq)
    assert np.array_equal(den[~near], ref[~near])


def test_zero_nsq_follows_ieee_arithmetic(orc):
    """Reading for nsq = 0: no special rule, IEEE 754 throughout.  A
    positive sigma1_sq divides by zero in the denominator expression:
    1 + s/0 = +inf, whose fp32 exponent field 255 makes log2f_approx return
    exactly 128 (t = 0).  With sigma1_sq = 0 the denominator is 1 + 0/0 =
    NaN: exponent field 255 again, and the default quiet NaN's fraction 1/2
    gives 128 plus the polynomial at t = 1/2, about 128 + log2(1.5).  The
    numerator then depends on sigma12: 0 gives the gain 0/0 = NaN and
    sv_sq = sigma2_sq - NaN = NaN (no floor catches a NaN), so its term is
    the same NaN value; +3 gives g = +inf, sv_sq = -inf, floored to eps,
    and the bounded gain times sigma1_sq = 0, so log2(1) = 0; -3 gives
    g = -inf, which the negative-gain rule zeroes: again 0."""
    n, d = orc.statistic(0.0, 0.0, 9.0, 5.0, 1.0, nsq=0.0)
    assert d == 128.0 and 0 < n < 128
    nan_term = orc.log2(np.frombuffer(np.uint32(0x7FC00000).tobytes(),
                                      np.float32)[0])
    # within half an fp32 step at 128 (2^-17) plus the polynomial error
    assert abs(float(nan_term) - (128 + math.log2(1.5))) < 2.0 ** -17 + 1e-6
    for s12, want_n in ((0.0, nan_term), (3.0, 0.0), (-3.0, 0.0)):
        n, d = orc.statistic(0.0, 0.0, 0.0, 5.0, s12, nsq=0.0)
        assert n == want_n, s12
        assert d == nan_term, s12


# ------------------------------------------------------ enhn_gain_limit

def _fp64_terms(s1, s2, s12, nsq, limit):
    """The statistic's definition in fp64 from given fp32 sigmas, with the
    gain bounded where it enters the numerator, after sv_sq is settled."""
    s1, s2, s12 = float(s1), float(s2), float(s12)
    if s1 < nsq:
        return 1.0, 1.0
    gg = s12 / s1
    sv = s2 - gg * s12
    if s2 < 1e-10:
        gg, sv = 0.0, 0.0
    if gg < 0:
        gg, sv = 0.0, s2
    sv = max(sv, 1e-10)
    gg = min(gg, limit)
    return (math.log2(1.0 + gg * gg * s1 / (sv + nsq)),
            math.log2(1.0 + s1 / nsq))


@pytest.mark.parametrize("nsq,limit", [(2.0, 0.3), (2.0, 1.0), (1.5, 2.5),
                                       (4.7, math.inf), (0.5, 0.05),
                                       (4.7, 1.0)])
def test_statistic_with_options_vs_fp64_formula(orc, nsq, limit):
    """Random high-branch inputs against the fp64 definition: pins where the
    limit acts (on the gain in the numerator, with sv_sq from the gain
    before the bound) and that nsq enters the branch and both ratios.
    Tolerances as in test_statistic_vs_fp64_formula."""
    g = np.random.Generator(np.random.PCG64(int(nsq * 100 + limit * 7
                                                if limit < 1e9 else 99)))
    for _ in range(2000):
        mu1 = F32(g.uniform(0, 255))
        mu2 = F32(g.uniform(0, 255))
        s1 = g.uniform(nsq, 5000.0)
        s2 = g.uniform(0.0, 5000.0)
        rho = g.uniform(-0.3, 1.0)
        s12 = rho * math.sqrt(s1 * s2)
        xx = F32(F32(mu1 * mu1) + F32(s1))
        yy = F32(F32(mu2 * mu2) + F32(s2))
        xy = F32(F32(mu1 * mu2) + F32(s12))
        n, d = orc.statistic(mu1, mu2, xx, yy, xy, nsq=nsq, gain_limit=limit)
        S1 = max(F32(xx - F32(mu1 * mu1)), F32(0))
        S2 = max(F32(yy - F32(mu2 * mu2)), F32(0))
        S12 = F32(xy - F32(mu1 * mu2))
        if abs(float(S1) - nsq) < 1e-4:
            continue
        en, ed = _fp64_terms(S1, S2, S12, nsq, limit)
        if float(S1) < nsq:
            assert (n, d) == (1.0, 1.0)
            continue
        assert abs(float(d) - ed) <= 1.7e-7 + 0.5 * P.ulp32(d) + 1e-7 * ed
        tol_n = 1.7e-7 + 0.5 * P.ulp32(n) + 1e-5 * max(en, 1e-3) + 1e-6
        assert abs(float(n) - en) <= tol_n, (mu1, mu2, xx, yy, xy, n, en)


def test_zero_gain_limit_zeroes_every_high_branch_numerator(orc):
    """Limit 0: the gain is 0 on every high-branch pixel, so the numerator
    term is log2(1) = 0 exactly; low-branch pixels keep 1; the denominator
    terms do not depend on the gain."""
    g = np.random.Generator(np.random.PCG64(41))
    n = 20000
    mu1 = g.uniform(0, 255, n).astype(np.float32)
    mu2 = g.uniform(0, 255, n).astype(np.float32)
    s1 = g.uniform(0, 50, n)
    s2 = g.uniform(0, 50, n)
    s12 = g.uniform(-1, 1, n) * np.sqrt(s1 * s2)
    xx = (mu1 * mu1 + s1.astype(np.float32)).astype(np.float32)
    yy = (mu2 * mu2 + s2.astype(np.float32)).astype(np.float32)
    xy = (mu1 * mu2 + s12.astype(np.float32)).astype(np.float32)
    n0, d0 = orc.statistic_array(mu1, mu2, xx, yy, xy, nsq=2.0,
                                 gain_limit=0.0)
    n1, d1 = orc.statistic_array(mu1, mu2, xx, yy, xy)
    low = d1 == 1.0
    assert low.any() and (~low).any()
    assert np.all(n0[low] == 1.0) and np.all(n0[~low] == 0.0)
    assert np.array_equal(d0, d1)


def test_gain_limit_is_monotone_and_idle_above_the_largest_gain(orc):
    """A larger limit never lowers a numerator term (the bounded gain, its
    square and the ratio are monotone under rounding).  On 8-bit content
    no gain reaches 100 (|g| <= sigma2/sigma1 <= 127.5/sqrt(2) < 91), so
    limits 100, 1e6 and +inf give the same bits."""
    g = np.random.Generator(np.random.PCG64(42))
    n = 20000
    mu1 = g.uniform(0, 255, n).astype(np.float32)
    mu2 = g.uniform(0, 255, n).astype(np.float32)
    s1 = np.exp(g.uniform(np.log(2.5), np.log(3000), n))
    s2 = np.exp(g.uniform(np.log(1e-3), np.log(3000), n))
    s12 = g.uniform(-0.2, 1, n) * np.sqrt(s1 * s2)
    xx = (mu1 * mu1 + s1.astype(np.float32)).astype(np.float32)
    yy = (mu2 * mu2 + s2.astype(np.float32)).astype(np.float32)
    xy = (mu1 * mu2 + s12.astype(np.float32)).astype(np.float32)
    prev = None
    for lim in (0.0, 0.1, 0.5, 1.0, 2.0, 8.0, math.inf):
        num, _ = orc.statistic_array(mu1, mu2, xx, yy, xy, nsq=2.0,
                                     gain_limit=lim)
        if prev is not None:
            assert np.all(num >= prev), lim
        prev = num
    r, d = _frame(3, (40, 52), spread=120)
    base = orc.score(r, d, 8, want_rows=True)
    for lim in (1e6, math.inf):
        other = orc.score(r, d, 8, want_rows=True,
                          options={"enhn_gain_limit": lim})
        for x, y in zip(base, other):
            assert x.tobytes() == y.tobytes(), lim


def test_gain_limit_one_leaves_identical_frames_alone(orc):
    """For a frame against itself sigma12 = sigma1_sq on every pixel, so the
    gain is exactly 1 and any limit >= 1 changes nothing; a limit below 1
    lowers every high-branch numerator term and leaves the denominators."""
    r, _ = _frame(4, (48, 48))
    base, sb = orc.score(r, r, 8)
    one, s1 = orc.score(r, r, 8, options={"enhn_gain_limit": 1.0})
    assert base.tobytes() == one.tobytes() and sb.tobytes() == s1.tobytes()
    half, sh = orc.score(r, r, 8, options={"enhn_gain_limit": 0.5})
    assert np.all(sh[0::2] < sb[0::2])
    assert np.array_equal(sh[1::2], sb[1::2])


@pytest.mark.parametrize("nsq,limit", [(4.7, 0.8), (1.5, 1e9), (2.0, 0.25)])
def test_pipeline_with_options_vs_fp64_definition(orc, nsq, limit):
    """Whole frames against the fp64 definition with nsq and the gain
    limit, tolerances as in test_pipeline_vs_fp64_definition."""
    r, d = _frame(int(nsq * 10), (40, 56))
    got, _ = orc.score(r, d, 8, options={"sigma_nsq": nsq,
                                         "enhn_gain_limit": limit})
    exp = P._vif_fp64(r, d, 8, nsq=nsq, gain_limit=limit)
    rel = np.abs(got[:7] - exp) / np.abs(exp)
    tol = np.array([2e-6, 1e-4, 3e-4, 5e-4, 2e-5, 2e-6, 2e-5])
    assert np.all(rel <= tol), (rel, got[:7], exp)


# --------------------------------------------------------- skip_scale0

def test_skip_scale0(orc):
    """Skipping scale 0 leaves scales 1..3 as they are (their planes come
    from the same pyramid), zeroes scale 0's sums and rows, reports 0 for
    vif_scale0, and totals the remaining scales in fp64 in scale order."""
    r, d = _frame(5, (45, 70))
    out, sums, rows = orc.score(r, d, 8, want_rows=True)
    sk, ss, rs = orc.score(r, d, 8, want_rows=True,
                           options={"skip_scale0": 1})
    assert sk[0] == 0.0 and np.all(ss[:2] == 0)
    assert ss[2:].tobytes() == sums[2:].tobytes()
    assert sk[1:4].tobytes() == out[1:4].tobytes()
    assert np.all(rs[:45] == 0) and rs[45:].tobytes() == rows[45:].tobytes()
    num = (0.0 + float(ss[2])) + float(ss[4])
    num = num + float(ss[6])
    den = (0.0 + float(ss[3])) + float(ss[5])
    den = den + float(ss[7])
    assert sk[4] == num and sk[5] == den and sk[6] == num / den


# ------------------------------------------------------------- floors

def test_scale_floors_act_on_reported_scores_only(orc):
    """A floor above a scale's score replaces it exactly; a floor below it
    changes nothing; sums, totals and the frame ratio never change, and
    each floor acts on its own scale (1, 2 or 3)."""
    r, d = _frame(6, (48, 64))
    out, sums = orc.score(r, d, 8)
    floors = (out[1] + 0.25, out[2] - 0.25, out[3] + 0.5)
    got, gs = orc.score(r, d, 8, options={"scale_min_val": floors})
    assert got[1] == floors[0] and got[2] == out[2] and got[3] == floors[2]
    assert got[0] == out[0]
    assert got[4:].tobytes() == out[4:].tobytes()
    assert gs.tobytes() == sums.tobytes()
    # a floor can lift a skipped or flat scale too, but not scale 0
    got, _ = orc.score(r, d, 8, options={"scale_min_val": (5.0, 5.0, 5.0),
                                         "skip_scale0": 1})
    assert got[0] == 0.0 and np.all(got[1:4] == 5.0)


# ----------------------------------------------------------- validation

@pytest.mark.parametrize("opt", [{"kernelscale": 2.0}, {"kernelscale": 0.5},
                                 {"sigma_nsq": -1.0},
                                 {"sigma_nsq": math.nan},
                                 {"sigma_nsq": math.inf},
                                 {"enhn_gain_limit": math.nan},
                                 {"enhn_gain_limit": -0.5},
                                 {"scale_min_val": (0.0, math.nan, 0.0)},
                                 {"skip_scale0": 2}])
def test_bad_options_rejected(orc, opt):
    r, d = _frame(7, (16, 16))
    with pytest.raises(ValueError):
        orc.score(r, d, 8, options=opt)


def test_unknown_option_name_rejected():
    import oracle
    with pytest.raises(ValueError):
        oracle.make_options({"vif_sigma": 1.0})
