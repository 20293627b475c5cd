"""Pins of the float SSIM oracle (decimation and SSIM stage) to what the
pages and the mathematics fix.

The decimation is the page's definition ("Research-2130: float_ssim
decimation on the SYCL device", Question, Sources and Findings): its
factor, sizes, window, border and the exactness of its double sum are
checked against independent evaluations (exact rational arithmetic, numpy's
symmetric padding, closed forms).  The SSIM stage is a reading of the
published SSIM; it is pinned by closed forms (a frame against itself scores
exactly 1, flat frames), an fp64 evaluation of the definition and
invariants.  CPU only.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
FACTS = json.load(open(os.path.join(HERE, "golden", "page_facts.json")))
F32 = np.float32


# --------------------------------------------------------------- factor

def test_scale_examples_from_the_page(orc):
    for wh, s in FACTS["fssim_scale_examples"]["value"].items():
        w, h = (int(v) for v in wh.split("x"))
        assert orc.fssim_scale(w, h) == s


@pytest.mark.parametrize("w,h,s", [(576, 324, 1), (100, 100, 1), (16, 16, 1),
                                   (383, 1000, 1), (384, 1000, 2),
                                   (640, 640, 3), (1280, 720, 3),
                                   (2560, 1440, 6), (7680, 4320, 17)])
def test_scale_rounds_half_away_from_zero(orc, w, h, s):
    """max(1, round(min(w, h) / 256)) with C's round: 384/256 = 1.5 -> 2,
    383/256 -> 1, 720/256 = 2.81 -> 3."""
    m = min(w, h)
    q = Fraction(m, 256)
    want = max(1, int(q + Fraction(1, 2)))  # q > 0: half away from zero
    assert want == s
    assert orc.fssim_scale(w, h) == s


@pytest.mark.parametrize("n,f,size", [(1920, 4, 480), (1080, 4, 270),
                                      (3840, 8, 480), (2160, 8, 270),
                                      (1921, 4, 481), (1081, 8, 136),
                                      (7, 3, 3), (9, 2, 5)])
def test_decimated_size(orc, n, f, size):
    """Research-2130, Sources: n / factor + (n & 1)."""
    assert orc.fssim_decimated_size(n, f) == size == n // f + (n & 1)


@pytest.mark.parametrize("n", [1, 2, 3, 7, 16])
def test_symmetric_border_matches_numpy(orc, n):
    """The period-2n mirror is numpy's 'symmetric' padding, repeated."""
    base = np.arange(n)
    reps = 3
    padded = np.pad(base, reps * 2 * n, mode="symmetric")
    for i in range(-reps * 2 * n, n + reps * 2 * n):
        assert orc.fssim_symmetric(i, n) == padded[i + reps * 2 * n], (i, n)


# ------------------------------------------------------------ decimation

def _exact_decimate(plane, f):
    """Independent evaluation: every fp32 product as an exact rational, the
    exact sum, rounded once to fp32 (via an exact double, since the sum is
    a multiple of 2^-45 below 256)."""
    h, w = plane.shape
    tap = F32(1.0) / F32(f * f)
    lo, hi = -(f // 2), f // 2 - (1 if f % 2 == 0 else 0)
    ow, oh = w // f + (w & 1), h // f + (h & 1)
    pad = 2 * f + 2
    P = np.pad(plane, pad, mode="symmetric")
    out = np.empty((oh, ow), np.float32)
    for y in range(oh):
        for x in range(ow):
            win = P[y * f + lo + pad:y * f + hi + 1 + pad,
                    x * f + lo + pad:x * f + hi + 1 + pad]
            prods = (win.astype(np.float32) * tap).astype(np.float32)
            s = sum((Fraction(float(v)) for v in prods.ravel()), Fraction(0))
            d = float(s)
            assert Fraction(d) == s          # exact in fp64
            out[y, x] = F32(d)
    return out


@pytest.mark.parametrize("f,bpc", [(2, 8), (3, 8), (4, 10), (5, 16), (7, 12),
                                   (8, 8), (6, 16)])
def test_decimation_is_the_exact_sum_rounded_once(orc, f, bpc):
    g = np.random.Generator(np.random.PCG64(100 + f))
    h, w = 3 * f + 5, 4 * f + 3
    codes = g.integers(0, 1 << bpc, size=(h, w))
    plane = (codes.astype(np.float64) / 2.0 ** (bpc - 8)).astype(np.float32)
    got = orc.fssim_decimate(plane, f)
    want = _exact_decimate(plane, f)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_fp32_window_sums_would_differ(orc):
    """The page rejects fp32 sums for non-power-of-two taps: the oracle's
    double sum differs from an fp32 running sum on some windows."""
    g = np.random.Generator(np.random.PCG64(7))
    f = 5
    plane = g.integers(0, 256, size=(60, 60)).astype(np.float32)
    got = orc.fssim_decimate(plane, f)
    tap = F32(1.0) / F32(25)
    P = np.pad(plane, 20, mode="symmetric")
    diff = 0
    for y in range(got.shape[0]):
        for x in range(got.shape[1]):
            acc = F32(0)
            for dy in range(-2, 3):
                for dx in range(-2, 3):
                    acc = F32(acc + F32(P[y * f + dy + 20, x * f + dx + 20]
                                        * tap))
            diff += int(acc != got[y, x])
    assert diff > 0


@pytest.mark.parametrize("f", [2, 4, 8])
def test_power_of_two_factor_is_the_plain_mean(orc, f):
    """For f = 2^k the tap is exact, the products are exact and so is the
    mean of the window: the output is RN32(window mean)."""
    g = np.random.Generator(np.random.PCG64(f))
    plane = (g.integers(0, 1 << 16, size=(5 * f, 6 * f)) / 256.0).astype(
        np.float32)
    got = orc.fssim_decimate(plane, f)
    lo = -(f // 2)
    P = np.pad(plane.astype(np.float64), f, mode="symmetric")
    for y in range(got.shape[0]):
        for x in range(got.shape[1]):
            win = P[y * f + lo + f:y * f + lo + 2 * f, x * f + lo + f:
                    x * f + lo + 2 * f]
            assert got[y, x] == F32(win.mean())


def test_decimation_window_position_and_offsets(orc):
    """An impulse at (yi, xi) reaches exactly the outputs whose window
    (offsets -f/2 .. f/2 - 1 for even f, -(f-1)/2 .. (f-1)/2 for odd f,
    around (x*f, y*f)) covers it, with the value fl32(v * tap)."""
    for f in (3, 4):
        plane = np.zeros((8 * f, 8 * f), np.float32)
        yi, xi = 3 * f + 1, 4 * f - 1
        plane[yi, xi] = 200.0
        got = orc.fssim_decimate(plane, f)
        lo, hi = -(f // 2), f // 2 - (1 if f % 2 == 0 else 0)
        want = np.zeros_like(got)
        v = F32(F32(200.0) * (F32(1.0) / F32(f * f)))
        for y in range(got.shape[0]):
            for x in range(got.shape[1]):
                if y * f + lo <= yi <= y * f + hi and \
                        x * f + lo <= xi <= x * f + hi:
                    want[y, x] = v
        assert np.array_equal(got, want), f


def test_flat_plane_decimates_to_itself_for_exact_taps(orc):
    for f in (2, 4, 8):
        plane = np.full((40, 36), 77.25, np.float32)
        assert np.all(orc.fssim_decimate(plane, f) == F32(77.25))


# ----------------------------------------------------------- SSIM stage

def test_gaussian_taps(orc):
    t = orc.fssim_taps().astype(np.float64)
    assert np.array_equal(t, t[::-1])
    g = np.exp(-((np.arange(11) - 5.0) ** 2) / (2 * 1.5 ** 2))
    ind = g / g.sum()
    assert np.all(np.abs(t - ind) <= 0.5 * np.spacing(ind.astype(np.float32)))
    assert abs(t.sum() - 1.0) < 1e-6


def test_filter_interior_impulse_and_border(orc):
    """An interior impulse gives the separable outer product of the taps
    (each entry fl32(t_i * fl32(t_j * v))); an impulse at the corner folds
    back by the symmetric border."""
    t = orc.fssim_taps()
    p = np.zeros((31, 29), np.float32)
    p[15, 14] = 3.0
    got = orc.fssim_filter(p)
    want = np.zeros_like(got)
    for dy in range(-5, 6):
        for dx in range(-5, 6):
            want[15 + dy, 14 + dx] = F32(t[5 - dx] * F32(t[5 - dy] * F32(3)))
    assert np.array_equal(got, want)
    p = np.zeros((20, 20), np.float32)
    p[0, 0] = 1.0
    got = orc.fssim_filter(p).astype(np.float64)
    P = np.pad(p.astype(np.float64), 5, mode="symmetric")
    k2 = np.outer(t, t)
    ref = np.array([[np.sum(P[y:y + 11, x:x + 11] * k2) for x in range(20)]
                    for y in range(20)])
    assert np.max(np.abs(got - ref)) < 1e-6


def _ssim_fp64(X, Y):
    """SSIM stage of the definition in fp64 (separable filter, symmetric
    border, combined formula), with numpy."""
    t = np.exp(-((np.arange(11) - 5.0) ** 2) / (2 * 1.5 ** 2))
    t = t / t.sum()

    def filt(P):
        Q = np.pad(P, 5, mode="symmetric")
        h, w = P.shape
        V = sum(t[k] * Q[k:k + h, :] for k in range(11))
        return sum(t[k] * V[:, k:k + w] for k in range(11))
    mu1, mu2 = filt(X), filt(Y)
    s11 = filt(X * X) - mu1 * mu1
    s22 = filt(Y * Y) - mu2 * mu2
    s12 = filt(X * Y) - mu1 * mu2
    c1, c2 = (0.01 * 255) ** 2, (0.03 * 255) ** 2
    return ((2 * mu1 * mu2 + c1) * (2 * s12 + c2) /
            ((mu1 * mu1 + mu2 * mu2 + c1) * (s11 + s22 + c2)))


def test_frame_against_itself_scores_exactly_one(orc):
    g = np.random.Generator(np.random.PCG64(9))
    for shape, bpc in (((324, 576), 8), ((1080, 1920), 10), ((64, 48), 16)):
        top = (1 << bpc) - 1
        r = g.integers(0, top + 1, size=shape).astype(
            np.uint8 if bpc == 8 else np.uint16)
        out, smap, _, _ = orc.fssim_score(r, r, bpc, want=True)
        assert out[0] == 1.0 and np.all(smap == 1.0)


@pytest.mark.parametrize("a,b", [(100, 140), (10, 240), (0, 255)])
def test_flat_frames_closed_form(orc, a, b):
    """Two flat frames a and b: the variances vanish up to the fp32
    rounding of the filtered values (two passes of 11 products and 10 sums:
    at most 44 * 2^-24 relative each), so each pixel is
    (2ab + C1) / (a^2 + b^2 + C1) times 1 + (2 s12 - s11 - s22) / C2 with
    |s..| <= 2 * 44 * 2^-24 * (product of the means)."""
    r = np.full((64, 80), a, np.uint8)
    d = np.full((64, 80), b, np.uint8)
    out = orc.fssim_score(r, d, 8)
    c1, c2 = (0.01 * 255) ** 2, (0.03 * 255) ** 2
    want = (2 * a * b + c1) / (a * a + b * b + c1)
    eps = 44 * 2.0 ** -24
    bound = 2 * eps * (2 * a * b + a * a + b * b) / c2 + 1e-6
    assert abs(out[0] - want) <= bound * want
    # and the mean term alone moves the score far more than that
    assert abs(want - 1.0) > 10 * bound or a == b


@pytest.mark.parametrize("shape,bpc,seed", [((120, 160), 8, 1),
                                            ((1080, 1920), 8, 2),
                                            ((300, 520), 10, 3),
                                            ((770, 1030), 16, 4)])
def test_score_vs_fp64_definition(orc, shape, bpc, seed):
    """The whole feature against an fp64 evaluation of the definition from
    the oracle's own decimated planes (whose exactness is pinned above):
    within the pages' 5e-5 float_ssim tolerance, and in practice far
    inside it."""
    g = np.random.Generator(np.random.PCG64(seed))
    top = (1 << bpc) - 1
    r = g.integers(0, top + 1, size=shape)
    d = np.clip(r + g.integers(-top // 8, top // 8 + 1, size=shape), 0, top)
    dt = np.uint8 if bpc == 8 else np.uint16
    out, smap, planes, rows = orc.fssim_score(r.astype(dt), d.astype(dt), bpc,
                                              want=True)
    exp = _ssim_fp64(planes[0].astype(np.float64),
                     planes[1].astype(np.float64))
    assert abs(out[0] - exp.mean()) < 1e-5
    assert abs(out[0] - exp.mean()) < FACTS["fssim_parity_gate"]["value"]
    assert np.max(np.abs(smap - exp)) < 2e-4
    # the mean is the fp32 rounding of the ordered fp64 sums: each row left
    # to right, then the rows top to bottom
    assert np.array_equal(rows, np.array([sum(float(v) for v in row)
                                          for row in smap]))
    total = 0.0
    for v in rows:
        total += float(v)
    assert out[0] == float(F32(total / smap.size))


def test_score_decimates_both_planes_with_the_auto_factor(orc):
    g = np.random.Generator(np.random.PCG64(11))
    r = g.integers(0, 256, size=(1080, 1920)).astype(np.uint8)
    d = g.integers(0, 256, size=(1080, 1920)).astype(np.uint8)
    out, smap, planes, _ = orc.fssim_score(r, d, 8, want=True)
    assert out[1] == 4 and smap.shape == (270, 480)
    assert np.array_equal(planes[0], orc.fssim_decimate(r.astype(np.float32),
                                                         4))
    assert np.array_equal(planes[1], orc.fssim_decimate(d.astype(np.float32),
                                                         4))
    # swapping ref and dist leaves SSIM (symmetric in x, y) unchanged
    sw = orc.fssim_score(d, r, 8)
    assert sw[0] == out[0]


def test_score_rejects_bad_arguments(orc):
    f = np.zeros((16, 16), np.uint8)
    with pytest.raises(ValueError):
        orc.fssim_score(f, f, 9)
    with pytest.raises(ValueError):
        orc.fssim_score(f.astype(np.uint16), f.astype(np.uint16), 8)
