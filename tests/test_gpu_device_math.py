"""Device-math gates (GPU): the kernels' own device functions against the
host, bit for bit, before the pipeline is trusted.

ADR-1444 "float_vif_hip runs the arithmetic of the CUDA twin ...",
Decision, reports a host comparison of the device's fp64 add and divide
over tens of millions of operand pairs and several noise variances.  Here:
2^25 pairs with magnitudes from 2^-40 to 2^40, six variances, targeted
near-ties, each checked on the sum, the quotient and both fp32 roundings of
one plus the quotient; the fp32 division, and the statistic's written-out
fp32 division over its domain; the log2 polynomial exhaustively
(every mantissa of exponents 0..31); the ratios and the whole statistic
against the oracle.
"""
import json
import os

import numpy as np
import pytest

from libutil import ensure_built

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
FACTS = json.load(open(os.path.join(HERE, "golden", "page_facts.json")))


@pytest.fixture(scope="module")
def dev():
    import torch
    lib = ensure_built()
    assert torch.cuda.is_available()
    return lib


def _d(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _h(t):
    return t.cpu().numpy()


def _check(rc):
    assert rc == 0, rc


def _span_operands(g, n, lo=-40, hi=40):
    e = g.uniform(lo, hi, size=n)
    return np.exp2(e).astype(np.float32)


def _near_ties(g, n, nsq):
    """Pairs (a, b) whose 1 + a/(b + nsq) lies within ~2^-24 (relative) of a
    midpoint between two fp32 values: the double-rounding zone."""
    lo = np.exp2(g.uniform(0, 20, size=n)).astype(np.float32)
    up = np.nextafter(lo, np.float32(np.inf))
    mid = (lo.astype(np.float64) + up.astype(np.float64)) / 2
    b = _span_operands(g, n, -20, 20)
    a = ((mid - 1.0) * (b.astype(np.float64) + nsq)).astype(np.float32)
    return a, b


@pytest.mark.parametrize("nsq", FACTS["fp64_gate_nsq_values"]["value"])
def test_fp64_add_div_cvt_bitwise(dev, nsq):
    import torch
    from vif_image_fidelity_amd import _lib
    total = FACTS["fp64_gate_pairs"]["value"]
    lo, hi = FACTS["fp64_gate_exponent_span"]["value"]
    n = total // 6 + 1
    g = np.random.Generator(np.random.PCG64(int(nsq * 1000)))
    a = _span_operands(g, n, lo, hi)
    b = _span_operands(g, n, lo, hi)
    ta, tb = _near_ties(g, 1 << 18, nsq)
    a = np.concatenate([a, ta])
    b = np.concatenate([b, tb])
    m = a.size
    da, db = _d(a), _d(b)
    s = torch.empty(m, dtype=torch.float64, device="cuda:0")
    q = torch.empty_like(s)
    rn = torch.empty(m, dtype=torch.float32, device="cuda:0")
    rd = torch.empty_like(rn)
    _check(_lib.load().vif_selftest_fp64(da.data_ptr(), db.data_ptr(), nsq, m,
                                         s.data_ptr(), q.data_ptr(),
                                         rn.data_ptr(), rd.data_ptr(), None))
    hs = b.astype(np.float64) + nsq
    hq = a.astype(np.float64) / hs
    hrn = (1.0 + hq).astype(np.float32)
    hrd = (1.0 + a.astype(np.float64) / nsq).astype(np.float32)
    assert np.array_equal(_h(s).view(np.uint64), hs.view(np.uint64))
    assert np.array_equal(_h(q).view(np.uint64), hq.view(np.uint64))
    assert np.array_equal(_h(rn).view(np.uint32), hrn.view(np.uint32))
    assert np.array_equal(_h(rd).view(np.uint32), hrd.view(np.uint32))


def test_fp32_division_bitwise(dev):
    import torch
    from vif_image_fidelity_amd import _lib
    g = np.random.Generator(np.random.PCG64(31))
    n = 1 << 25
    a = (_span_operands(g, n, -60, 60) *
         np.where(g.random(n) < 0.5, -1, 1)).astype(np.float32)
    b = (_span_operands(g, n, -60, 60) *
         np.where(g.random(n) < 0.5, -1, 1)).astype(np.float32)
    q = torch.empty(n, dtype=torch.float32, device="cuda:0")
    da, db = _d(a), _d(b)  # keep the device copies alive across the call
    _check(_lib.load().vif_selftest_div32(da.data_ptr(), db.data_ptr(),
                                          n, q.data_ptr(), None))
    assert np.array_equal(_h(q).view(np.uint32), (a / b).view(np.uint32))


def test_fp32_division_in_range_bitwise(dev):
    """The statistic's written-out fp32 division for a power-of-two noise
    variance (div_in_range_f32) against the host's IEEE division over its
    whole domain: 2^25 pairs with |a| from 2^-100 to 2^17 (and zeros) and b
    from 2^-20 to 2^17, 2^20 quotients within an ulp of a midpoint between
    two fp32 values, and the domain's corners."""
    import torch
    from vif_image_fidelity_amd import _lib
    g = np.random.Generator(np.random.PCG64(37))
    n = 1 << 25
    a = (_span_operands(g, n, -100, 17) *
         np.where(g.random(n) < 0.5, -1, 1)).astype(np.float32)
    b = _span_operands(g, n, -20, 17)
    a[:4096] = 0.0
    # near-ties: a = fl32(b * m) with m the midpoint of two fp32 quotients
    m = 1 << 20
    bt = _span_operands(g, m, -20, 17)
    la = g.uniform(-99, 16, size=m)
    q0 = np.exp2(la - np.log2(bt.astype(np.float64))).astype(np.float32)
    mid = (q0.astype(np.float64) +
           np.nextafter(q0, np.float32(np.inf)).astype(np.float64)) / 2
    at = (mid * bt.astype(np.float64)).astype(np.float32)
    a[4096:4096 + m], b[4096:4096 + m] = at, bt
    corners_a = np.array([2.0 ** -100, -2.0 ** -100, 2.0 ** 17, -2.0 ** 17,
                          1.0, 3.0, -7.0, 2.0 ** -99 * 3], dtype=np.float32)
    corners_b = np.array([2.0 ** -20, 2.0 ** 17, 1.0, 3.0, 2.0 ** -20 * 3,
                          2.0 ** 17 * 0.75], dtype=np.float32)
    ca, cb = np.meshgrid(corners_a, corners_b)
    k = ca.size
    a[-k:], b[-k:] = ca.ravel(), cb.ravel()
    aa = np.abs(a.astype(np.float64))
    assert np.all((a == 0) | ((aa >= 2.0 ** -100) & (aa <= 2.0 ** 17)))
    assert np.all((b >= 2.0 ** -20) & (b <= 2.0 ** 17))
    q = torch.empty(n, dtype=torch.float32, device="cuda:0")
    da, db = _d(a), _d(b)
    _check(_lib.load().vif_selftest_div32_in_range(
        da.data_ptr(), db.data_ptr(), n, q.data_ptr(), None))
    assert np.array_equal(_h(q).view(np.uint32), (a / b).view(np.uint32))


def test_log2_exhaustive_bitwise(dev, orc):
    """Every fp32 mantissa of every exponent 0..31: device == oracle."""
    import torch
    from vif_image_fidelity_amd import _lib
    m = np.arange(1 << 23, dtype=np.uint32)
    y = torch.empty(1 << 23, dtype=torch.float32, device="cuda:0")
    for e in range(32):
        x = ((np.uint32(127 + e) << np.uint32(23)) | m).view(np.float32)
        dx = _d(x)
        _check(_lib.load().vif_selftest_log2(dx.data_ptr(), x.size,
                                             y.data_ptr(), None))
        ref = orc.log2_array(x)
        assert np.array_equal(_h(y).view(np.uint32), ref.view(np.uint32)), e


def _same_bits_or_both_nan(x, y):
    """Bitwise equality, except that NaNs compare by being NaN: the host's
    default NaN has the sign bit set, the device's does not, and nothing
    downstream reads a NaN's sign (the log2 polynomial masks it)."""
    nx, ny = np.isnan(x), np.isnan(y)
    return (np.array_equal(nx, ny)
            and np.array_equal(x[~nx].view(np.uint32),
                               y[~ny].view(np.uint32)))


@pytest.mark.parametrize("nsq", [2.0, 1.5, 4.7, 0.5, 4.0, 1e-3, 0.0])
def test_ratios_bitwise(dev, orc, nsq):
    """Both one-plus-ratio values for the default noise variance, for
    values that are not powers of two (the division path), for powers of two
    (the exact-reciprocal path) and for zero (IEEE division by zero)."""
    import torch
    from vif_image_fidelity_amd import _lib
    g = np.random.Generator(np.random.PCG64(32))
    n = 1 << 22 if nsq == 2.0 else 1 << 20
    a = np.exp(g.uniform(np.log(1e-6), np.log(5e8), n)).astype(np.float32)
    sv = np.exp(g.uniform(np.log(1e-10), np.log(1e5), n)).astype(np.float32)
    a[:64] = 0.0
    ta, tb = _near_ties(g, 1 << 18, max(nsq, 1e-3))
    a = np.concatenate([a, ta])
    sv = np.concatenate([sv, tb])
    num = torch.empty(a.size, dtype=torch.float32, device="cuda:0")
    den = torch.empty_like(num)
    da, dsv = _d(a), _d(sv)
    _check(_lib.load().vif_selftest_ratios(da.data_ptr(), dsv.data_ptr(),
                                           nsq, a.size, num.data_ptr(),
                                           den.data_ptr(), None))
    rn, rd = orc.ratios(a, sv, nsq=nsq)
    assert _same_bits_or_both_nan(_h(num), rn)
    assert _same_bits_or_both_nan(_h(den), rd)
    if nsq == 0.0:
        assert np.isnan(rd[a == 0]).all() and np.isinf(rd[a > 0]).all()


@pytest.mark.parametrize("nsq", [2.0 ** -20, 2.0 ** 20, 2.0 ** -21, 2.0 ** 21])
def test_ratios_bitwise_whole_range(dev, orc, nsq):
    """The numerator ratio over every finite fp32 a >= 0 the kernels can
    form (0 and 2^-149 .. 2^127, log-uniform) and sv from the floor 1e-10 to
    2^127, at the ends of the power-of-two form's nsq range (2^-20, 2^20:
    the fp64 division without scaling steps) and just outside it (2^-21,
    2^21: the general form), against the oracle's fp64 ratios."""
    import torch
    from vif_image_fidelity_amd import _lib
    g = np.random.Generator(np.random.PCG64(34))
    n = 1 << 20
    a = np.exp2(g.uniform(-149, 127.9, n)).astype(np.float32)
    sv = np.exp(g.uniform(np.log(1e-10), np.log(2.0 ** 127), n)).astype(
        np.float32)
    a[:64] = 0.0
    a[64:128] = np.float32(2.0 ** -149)
    a[128:192] = np.nextafter(np.float32(np.inf), np.float32(0))
    sv[192:256] = np.float32(1e-10)
    num = torch.empty(n, dtype=torch.float32, device="cuda:0")
    den = torch.empty_like(num)
    da, dsv = _d(a), _d(sv)   # held until the call has finished
    _check(_lib.load().vif_selftest_ratios(da.data_ptr(), dsv.data_ptr(),
                                           nsq, n, num.data_ptr(),
                                           den.data_ptr(), None))
    rn, rd = orc.ratios(a, sv, nsq=nsq)
    assert np.array_equal(_h(num).view(np.uint32), rn.view(np.uint32))
    assert np.array_equal(_h(den).view(np.uint32), rd.view(np.uint32))


def _statistic_inputs(g, n):
    """Five filtered values shaped like real data: means in [0, 256),
    variances from 0 to ~2e4 (many near the noise variance 2), covariance
    of either sign, with the cancellation of xx - mu^2 in fp32."""
    mu1 = g.uniform(0, 256, n).astype(np.float32)
    mu2 = g.uniform(0, 256, n).astype(np.float32)
    v1 = np.where(g.random(n) < 0.3, g.uniform(0, 4, n),
                  np.exp(g.uniform(-3, 10, n)))
    v2 = np.where(g.random(n) < 0.3, g.uniform(0, 4, n),
                  np.exp(g.uniform(-3, 10, n)))
    rho = g.uniform(-1, 1, n)
    c = rho * np.sqrt(v1 * v2)
    xx = (mu1.astype(np.float64) ** 2 + v1).astype(np.float32)
    yy = (mu2.astype(np.float64) ** 2 + v2).astype(np.float32)
    xy = (mu1.astype(np.float64) * mu2 + c).astype(np.float32)
    return mu1, mu2, xx, yy, xy


@pytest.mark.parametrize("nsq,limit", [(2.0, 100.0), (4.7, 1.0),
                                       (1.5, 0.3), (0.5, np.inf),
                                       (2.0, 0.0), (0.0, 100.0)])
def test_statistic_bitwise(dev, orc, nsq, limit):
    """The whole per-pixel statistic against the oracle's, for the default
    options and for noise variances and gain limits that take every path:
    the division and reciprocal paths of the denominator, a binding gain
    limit, a zero limit, and nsq = 0 (zero variances divide by zero)."""
    import torch
    from vif_image_fidelity_amd import _lib
    g = np.random.Generator(np.random.PCG64(33))
    n = 1 << 22 if (nsq, limit) == (2.0, 100.0) else 1 << 20
    ins = _statistic_inputs(g, n)
    dins = [_d(a) for a in ins]
    num = torch.empty(n, dtype=torch.float32, device="cuda:0")
    den = torch.empty_like(num)
    _check(_lib.load().vif_selftest_statistic(
        *[t.data_ptr() for t in dins], n, nsq, limit, num.data_ptr(),
        den.data_ptr(), None))
    rn, rd = orc.statistic_array(*ins, nsq=nsq, gain_limit=limit)
    assert np.array_equal(_h(num).view(np.uint32), rn.view(np.uint32))
    assert np.array_equal(_h(den).view(np.uint32), rd.view(np.uint32))
    # the sample really exercises both branches and every clamp
    hi = rd != 1.0
    if nsq > 0:
        assert 0.2 < hi.mean() < 0.95
        assert (rn[hi] == 0).any()
    else:
        assert (rd >= 128.0).any()      # sigma1_sq / 0 reached the log2
    if 0 < limit < 10:
        un, _ = orc.statistic_array(*ins, nsq=nsq, gain_limit=np.inf)
        assert (un > rn).any()          # the limit binds somewhere


def test_selftests_reject_bad_options(dev):
    from vif_image_fidelity_amd import _lib
    L = _lib.load()
    for nsq, lim in ((-1.0, 100.0), (np.nan, 100.0), (np.inf, 100.0),
                     (2.0, -1.0), (2.0, np.nan)):
        assert L.vif_selftest_statistic(None, None, None, None, None, 0, nsq,
                                        lim, None, None, None) == \
            _lib.VIF_EINVAL
    assert L.vif_selftest_ratios(None, None, -2.0, 0, None, None, None) == \
        _lib.VIF_EINVAL


def test_valu_rate_microbenchmark_runs(dev):
    """The issue-rate microbenchmark at 6 and 8 waves per SIMD: it runs,
    times itself and leaves finite results."""
    import ctypes
    import torch
    from vif_image_fidelity_amd import _lib
    blocks = 256
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32,
                     device="cuda:0")
    for w in (6, 8):
        ms = ctypes.c_double(0.0)
        _check(_lib.load().vif_selftest_valu_rate(w, 64, blocks,
                                                  out.data_ptr(),
                                                  ctypes.byref(ms), None))
        assert ms.value > 0.0
        assert torch.isfinite(out).all()


def test_carry_wait_gives_up_and_reports(dev):
    """Scale 0 hands each row's fp32 sum from tile to tile; a tile waits for
    its left neighbour's word with a bounded number of reads.  Forced from
    the host: only the second tile column of a two-column frame runs, so the
    words it waits for never arrive.  The kernel must still end, raise its
    error word and store NaN rather than a sum."""
    import ctypes
    import time
    from vif_image_fidelity_amd import _lib
    raised = ctypes.c_int(0)
    row = np.zeros(1, dtype=np.float32)
    t0 = time.time()
    rc = _lib.load().vif_selftest_carry_wait(
        ctypes.byref(raised), row.ctypes.data_as(ctypes.POINTER(
            ctypes.c_float)), None)
    took = time.time() - t0
    print("carry wait gave up after %.3f s" % took, flush=True)
    assert rc == _lib.VIF_OK
    assert raised.value == 1
    assert np.isnan(row[0])
    assert took < 30
