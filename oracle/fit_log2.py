"""Fit of the log2 polynomial used by log2f_approx (test infrastructure).

The float VIF definition evaluates log2 of its two one-plus-ratio values with
a polynomial in fp32 rather than with a library log2 (ADR-1422 "float_vif_sycl
computes the CPU's arithmetic ...", Context: the device log2 of the old twin
differed from the CPU's polynomial; ADR-1444, Context: the four properties a
twin must copy include that polynomial).  The pages do not print its
coefficients, so this method defines its own:

  * x >= 1 is split as x = 2^e * (1 + t), t in [0, 1);
  * log2(1 + t) = t * P(t), P of degree K-1 = 9 (K = 10 coefficients);
  * P interpolates g(t) = log2(1 + t) / t at the K Chebyshev points of the
    first kind on [0, 1] (numpy's Chebyshev.interpolate), computed in fp64,
    converted to the monomial basis in t and rounded to fp32 once.

Running this script prints the ten coefficients c_1..c_10 as fp32 hex.  The
oracle holds them as literals; a CPU test re-runs this fit and checks the
literals are what it produces.  The fit is deterministic (fixed nodes, no
random numbers).
"""
import numpy as np
from numpy.polynomial import chebyshev as _cheb
from numpy.polynomial import polynomial as _poly

K = 10


def _g(t):
    t = np.asarray(t, dtype=np.float64)
    out = np.empty_like(t)
    nz = t != 0.0
    out[nz] = np.log1p(t[nz]) / np.log(2.0) / t[nz]
    out[~nz] = 1.0 / np.log(2.0)
    return out


def fit_coefficients(k=K):
    """Return c_1..c_k as numpy float32 (c_1 multiplies t, c_k multiplies t^k)."""
    ch = _cheb.Chebyshev.interpolate(_g, k - 1, domain=[0.0, 1.0])
    mono = ch.convert(kind=_poly.Polynomial, domain=[-1.0, 1.0],
                      window=[-1.0, 1.0]).coef
    return np.asarray(mono, dtype=np.float64).astype(np.float32)


def fp32_hex(v):
    return "0x%08x" % int(np.float32(v).view(np.uint32))


if __name__ == "__main__":
    c = fit_coefficients()
    for i, v in enumerate(c, start=1):
        print("c_%d = %s  /* %.9e */" % (i, fp32_hex(v), float(v)))
