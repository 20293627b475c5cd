"""The normalisation of 10- to 16-bit samples carried by the vertical
pass's taps (CPU): for every sample value of every bit depth and every tap
of scale 0's filter and the decimation low-pass, the products the kernel
forms from the raw sample with the scaled taps equal, bit for bit, the
products of the normalised sample with the plain taps (fp32 arithmetic,
each product rounded once): t * (v * s) == (t * s) * v, and
t * fl((v * s)^2) == (t * s^2) * fl(v^2), the cross product likewise.
Exhaustive over the sample values; the taps are the library's own."""
import numpy as np
import pytest

from vif_image_fidelity_amd import _lib

F32 = np.float32


def _taps(scale):
    buf = np.zeros(_lib.MAX_TAPS, dtype=F32)
    n = _lib.vif_taps(scale, buf)
    return buf[:n]


@pytest.mark.parametrize("bpc,s", [(10, 2.0 ** -2), (12, 2.0 ** -4),
                                   (16, 2.0 ** -8)])
def test_scaled_taps_give_the_same_products(bpc, s):
    s = F32(s)
    v = np.arange(1 << bpc, dtype=F32)          # every raw sample value
    p = v * s                                   # the normalised sample
    assert np.array_equal(p.astype(np.float64), v.astype(np.float64) * float(s))
    sq = p * p                                  # fl((v s)^2)
    sq_raw = v * v                              # fl(v^2)
    for t in np.concatenate([_taps(0), _taps(1)]):
        t = F32(t)
        ts, ts2 = t * s, t * s * s
        # exact: powers of two times normal values
        assert float(ts) == float(t) * float(s)
        assert float(ts2) == float(t) * float(s) ** 2
        assert np.array_equal((t * p).view(np.uint32),
                              (ts * v).view(np.uint32))
        assert np.array_equal((t * sq).view(np.uint32),
                              (ts2 * sq_raw).view(np.uint32))


def test_scaled_cross_products_match():
    g = np.random.Generator(np.random.PCG64(43))
    s = F32(2.0 ** -8)
    a = g.integers(0, 1 << 16, size=1 << 20).astype(F32)
    b = g.integers(0, 1 << 16, size=1 << 20).astype(F32)
    for t in _taps(0):
        t = F32(t)
        assert np.array_equal((t * ((a * s) * (b * s))).view(np.uint32),
                              ((t * s * s) * (a * b)).view(np.uint32))
