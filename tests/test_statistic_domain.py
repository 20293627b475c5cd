"""The domain of the statistic's written-out fp32 division (CPU).

For a power-of-two noise variance the kernels divide sigma12 by sigma1_sq
with the fp32 division's steps but without its scaling and fix-up steps
(div_in_range_f32), which gives the correctly rounded quotient only when
sigma1_sq lies in [2^-20, 2^17] and sigma12 is +0 or at least 2^-100 in
magnitude.  The division runs only above the noise variance (sigma1_sq >=
nsq >= 2^-20).  The rest follows from the samples and the taps: a sample
normalised from 8 to 16 bits is 0 or at least 2^-8 and below 256, every
filter and decimation adds non-negative products in fp32, so a non-zero
filtered value is at least the smallest single product, and sigma12 is the
fp32 difference of two such values (xy and mu1 * mu2), a multiple of the
smaller one's ulp.  Here: that chain of bounds with the oracle's taps, and
the oracle's own filters and pyramid on frames built to make the smallest
non-zero values, with and without a textured reference."""
import math

import numpy as np

import oracle

F32 = np.float32


def _smallest_nonzero_bounds():
    """(scale, smallest non-zero xx/yy/xy, smallest non-zero mu1*mu2) under
    the chain of single-product bounds, each product rounded down by one
    fp32 rounding."""
    down = 1.0 - 2.0 ** -23
    plane = 2.0 ** -8          # smallest non-zero normalised sample
    out = []
    for s in range(4):
        if s > 0:
            t = float(min(oracle.taps(s)))
            plane = t * t * plane * down ** 2
        t = float(min(oracle.taps(s)))
        mu = t * t * plane * down ** 2
        second = t * t * plane * plane * down ** 3
        out.append((s, second, mu * mu * down))
    return out


def test_chain_bound_keeps_sigma12_in_domain():
    for s, second, m12 in _smallest_nonzero_bounds():
        smallest = min(second, m12)
        assert smallest >= 2.0 ** -80, (s, math.log2(smallest))
        # a non-zero difference of two values >= 2^e is >= 2^(e - 23)
        e = math.floor(math.log2(smallest))
        assert 2.0 ** (e - 23) >= 2.0 ** -103 * 8, (s, e)


def test_taps_keep_filtered_values_below_2_17():
    top = (65535 / 256.0) ** 2          # the largest squared sample
    for s in range(4):
        t = np.asarray(oracle.taps(s), dtype=np.float64)
        assert t.min() > 0
        # fp32 sums of non-negative products with taps summing to ~1, two
        # passes per filter, a decimation per scale
        assert (t.sum() * (1 + 2.0 ** -20)) ** 8 * top < 2.0 ** 17


def _stat_inputs(ref16, dist16):
    """Per scale: the oracle's five filtered planes, from its own pyramid."""
    x = oracle.normalise(ref16, 16)
    y = oracle.normalise(dist16, 16)
    for s in range(4):
        t = np.asarray(oracle.taps(s), dtype=F32)
        if s > 0:
            x = oracle.decimate(x, t)
            y = oracle.decimate(y, t)
        yield s, (oracle.filter2d(x, t), oracle.filter2d(y, t),
                  oracle.filter2d(x * x, t), oracle.filter2d(y * y, t),
                  oracle.filter2d(x * y, t))


def _check_pair(ref16, dist16):
    seen = 0
    for s, (mu1, mu2, xx, yy, xy) in _stat_inputs(ref16, dist16):
        s1 = np.maximum(xx - mu1 * mu1, F32(0))
        s12 = xy - mu1 * mu2
        assert s1.dtype == F32 and s12.dtype == F32
        assert float(xx.max()) < 2.0 ** 17
        live = s1.astype(np.float64) >= 2.0 ** -20
        a = np.abs(s12[live]).astype(np.float64)
        nz = a[a > 0]
        if nz.size:
            assert nz.min() >= 2.0 ** -100, (s, math.log2(nz.min()))
        assert not np.any(np.signbit(s12) & (s12 == 0))   # never -0
        seen += int(live.sum())
    return seen


def test_smallest_values_on_sparse_frames():
    g = np.random.Generator(np.random.PCG64(41))
    h, w = 128, 128
    # a textured reference (so the division runs) with many zero samples,
    # against a distorted frame of isolated smallest samples
    ref = g.integers(0, 65536, size=(h, w)).astype(np.uint16)
    ref[g.random((h, w)) < 0.5] = 0
    dist = np.zeros((h, w), dtype=np.uint16)
    dist[g.random((h, w)) < 0.01] = 1
    assert _check_pair(ref, dist) > 0
    # and the other way round, and a pair of isolated smallest samples
    assert _check_pair(dist, ref) >= 0
    one = np.zeros((h, w), dtype=np.uint16)
    one[h // 2, w // 2] = 1
    other = np.zeros((h, w), dtype=np.uint16)
    other[h // 2 + 3, w // 2 - 5] = 1
    _check_pair(one, other)
