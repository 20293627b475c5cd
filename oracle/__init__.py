"""ctypes binding of the plain CPU oracle of the float VIF feature.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the GPU library and
its Python binding never do.  The C source (vif_oracle.c) cites the passage
each step follows.

The shared library is built next to its source with gcc, on demand if it is
missing (``build()`` rebuilds it unconditionally).  ``Oracle(path)`` wraps
any build of the same source, which the mutation tests use to load
deliberately broken copies.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vif_oracle.c")
_FSSIM_SRC = os.path.join(_HERE, "fssim_oracle.c")
_LIB = os.path.join(_HERE, "libvif_oracle.so")

CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
          "-fno-builtin", "-msse2", "-mfpmath=sse", "-fPIC", "-shared",
          "-Wall", "-Wextra"]

NSCALES = 4
WIDTHS = (17, 9, 5, 3)

_default = None


class Options(ctypes.Structure):
    """vifo_options: readings of the option names the pages give."""
    _fields_ = [("sigma_nsq", ctypes.c_double),
                ("enhn_gain_limit", ctypes.c_double),
                ("kernelscale", ctypes.c_double),
                ("scale_min_val", ctypes.c_double * 3),
                ("skip_scale0", ctypes.c_int)]


DEFAULT_OPTIONS = {"sigma_nsq": 2.0, "enhn_gain_limit": 100.0,
                   "kernelscale": 1.0, "scale_min_val": (0.0, 0.0, 0.0),
                   "skip_scale0": 0}


def make_options(options=None):
    """An Options structure from a dict of overrides of the defaults."""
    d = dict(DEFAULT_OPTIONS)
    if options:
        unknown = set(options) - set(d)
        if unknown:
            raise ValueError("unknown options %s" % sorted(unknown))
        d.update(options)
    o = Options()
    o.sigma_nsq = float(d["sigma_nsq"])
    o.enhn_gain_limit = float(d["enhn_gain_limit"])
    o.kernelscale = float(d["kernelscale"])
    mv = tuple(d["scale_min_val"])
    if len(mv) != 3:
        raise ValueError("scale_min_val needs three floors")
    o.scale_min_val[:] = [float(v) for v in mv]
    o.skip_scale0 = int(d["skip_scale0"])
    return o


def build(src=_SRC, out=_LIB, fssim_src=_FSSIM_SRC):
    """Compile the oracle C sources (the VIF oracle, possibly a mutated
    copy, and the float SSIM oracle) into one shared library (default: in
    place)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc"] + CFLAGS + ["-I", _HERE, "-o", tmp, src, fssim_src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _fp(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


class Oracle:
    """numpy-facing wrapper of one build of the oracle library."""

    def __init__(self, path):
        lib = ctypes.CDLL(path)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        lib.vifo_taps.argtypes = [ctypes.c_int, f32p]
        lib.vifo_taps.restype = ctypes.c_int
        lib.vifo_log2.argtypes = [ctypes.c_float]
        lib.vifo_log2.restype = ctypes.c_float
        lib.vifo_log2_array.argtypes = [f32p, f32p, ctypes.c_long]
        lib.vifo_log2_array.restype = None
        lib.vifo_ratio_arrays.argtypes = [f32p, f32p, f32p, f32p,
                                          ctypes.c_long]
        lib.vifo_ratio_arrays.restype = None
        lib.vifo_ratio_arrays_nsq.argtypes = [f32p, f32p, ctypes.c_double,
                                              f32p, f32p, ctypes.c_long]
        lib.vifo_ratio_arrays_nsq.restype = None
        lib.vifo_statistic.argtypes = [ctypes.c_float] * 5 + [f32p, f32p]
        lib.vifo_statistic_array.argtypes = [f32p] * 7 + [ctypes.c_long]
        lib.vifo_statistic_array.restype = None
        lib.vifo_statistic.restype = None
        lib.vifo_statistic_ex.argtypes = ([ctypes.c_float] * 5
                                          + [ctypes.c_double] * 2
                                          + [f32p, f32p])
        lib.vifo_statistic_ex.restype = None
        lib.vifo_statistic_array_ex.argtypes = ([f32p] * 5
                                                + [ctypes.c_double] * 2
                                                + [f32p, f32p, ctypes.c_long])
        lib.vifo_statistic_array_ex.restype = None
        lib.vifo_normalise.argtypes = [ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, f32p]
        lib.vifo_normalise.restype = ctypes.c_int
        for name in ("vifo_filter", "vifo_decimate"):
            fn = getattr(lib, name)
            fn.argtypes = [f32p, ctypes.c_int, ctypes.c_int, f32p,
                           ctypes.c_int, f32p]
            fn.restype = ctypes.c_int
        lib.vifo_ordered_sums.argtypes = [f32p, f32p, ctypes.c_int,
                                          ctypes.c_int, f32p, f32p, f32p]
        lib.vifo_ordered_sums.restype = ctypes.c_int
        lib.vifo_total_rows.argtypes = [ctypes.c_int, ctypes.c_int]
        lib.vifo_total_rows.restype = ctypes.c_int
        lib.vifo_score.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   f64p, f32p, f32p]
        lib.vifo_score.restype = ctypes.c_int
        lib.vifo_score_ex.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.POINTER(Options), f64p, f32p,
                                      f32p]
        lib.vifo_score_ex.restype = ctypes.c_int
        lib.fssimo_scale.argtypes = [ctypes.c_int, ctypes.c_int]
        lib.fssimo_scale.restype = ctypes.c_int
        lib.fssimo_decimated_size.argtypes = [ctypes.c_int, ctypes.c_int]
        lib.fssimo_decimated_size.restype = ctypes.c_int
        lib.fssimo_symmetric.argtypes = [ctypes.c_int, ctypes.c_int]
        lib.fssimo_symmetric.restype = ctypes.c_int
        lib.fssimo_decimate.argtypes = [f32p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, f32p]
        lib.fssimo_decimate.restype = ctypes.c_int
        lib.fssimo_taps.argtypes = [f32p]
        lib.fssimo_taps.restype = None
        lib.fssimo_filter.argtypes = [f32p, ctypes.c_int, ctypes.c_int, f32p]
        lib.fssimo_filter.restype = ctypes.c_int
        lib.fssimo_pixel.argtypes = [ctypes.c_float] * 5
        lib.fssimo_pixel.restype = ctypes.c_float
        lib.fssimo_score.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     f64p, f32p, f32p, f64p]
        lib.fssimo_score.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def taps(self, scale):
        buf = np.zeros(17, dtype=np.float32)
        n = self.lib.vifo_taps(int(scale), _fp(buf))
        if n < 0:
            raise ValueError("bad scale %r" % (scale,))
        return buf[:n].copy()

    def log2(self, x):
        return np.float32(self.lib.vifo_log2(float(np.float32(x))))

    def log2_array(self, xs):
        """Element-wise oracle log2f_approx over a float32 array."""
        xs = np.ascontiguousarray(xs, dtype=np.float32)
        out = np.empty_like(xs)
        self.lib.vifo_log2_array(_fp(xs), _fp(out), xs.size)
        return out

    def ratios(self, a, sv, nsq=None):
        """(fl32(1 + a/(sv + nsq)), fl32(1 + a/nsq)) element-wise; nsq=None
        is the default 2.0 through the default entry point."""
        a = np.ascontiguousarray(a, dtype=np.float32)
        sv = np.ascontiguousarray(sv, dtype=np.float32)
        num = np.empty_like(a)
        den = np.empty_like(a)
        if nsq is None:
            self.lib.vifo_ratio_arrays(_fp(a), _fp(sv), _fp(num), _fp(den),
                                       a.size)
        else:
            self.lib.vifo_ratio_arrays_nsq(_fp(a), _fp(sv), float(nsq),
                                           _fp(num), _fp(den), a.size)
        return num, den

    def statistic(self, mu1, mu2, xx, yy, xy, nsq=None, gain_limit=None):
        n = ctypes.c_float()
        d = ctypes.c_float()
        args = [float(np.float32(v)) for v in (mu1, mu2, xx, yy, xy)]
        if nsq is None and gain_limit is None:
            self.lib.vifo_statistic(*args, ctypes.byref(n), ctypes.byref(d))
        else:
            self.lib.vifo_statistic_ex(
                *args, 2.0 if nsq is None else float(nsq),
                100.0 if gain_limit is None else float(gain_limit),
                ctypes.byref(n), ctypes.byref(d))
        return np.float32(n.value), np.float32(d.value)

    def statistic_array(self, mu1, mu2, xx, yy, xy, nsq=None,
                        gain_limit=None):
        """vifo_statistic element-wise over five float32 arrays."""
        ins = [np.ascontiguousarray(a, dtype=np.float32)
               for a in (mu1, mu2, xx, yy, xy)]
        num = np.empty_like(ins[0])
        den = np.empty_like(ins[0])
        if nsq is None and gain_limit is None:
            self.lib.vifo_statistic_array(*[_fp(a) for a in ins], _fp(num),
                                          _fp(den), ins[0].size)
        else:
            self.lib.vifo_statistic_array_ex(
                *[_fp(a) for a in ins], 2.0 if nsq is None else float(nsq),
                100.0 if gain_limit is None else float(gain_limit),
                _fp(num), _fp(den), ins[0].size)
        return num, den

    def normalise(self, plane, bpc):
        plane = np.ascontiguousarray(plane)
        h, w = plane.shape
        out = np.empty((h, w), dtype=np.float32)
        rc = self.lib.vifo_normalise(plane.ctypes.data, w, h, int(bpc),
                                     _fp(out))
        if rc != 0:
            raise ValueError("normalise rejected its arguments")
        return out

    def filter2d(self, plane, tap):
        plane = np.ascontiguousarray(plane, dtype=np.float32)
        tap = np.ascontiguousarray(tap, dtype=np.float32)
        h, w = plane.shape
        out = np.empty((h, w), dtype=np.float32)
        rc = self.lib.vifo_filter(_fp(plane), w, h, _fp(tap), len(tap),
                                  _fp(out))
        if rc != 0:
            raise ValueError("filter rejected its arguments")
        return out

    def decimate(self, plane, tap):
        plane = np.ascontiguousarray(plane, dtype=np.float32)
        tap = np.ascontiguousarray(tap, dtype=np.float32)
        h, w = plane.shape
        out = np.empty((h // 2, w // 2), dtype=np.float32)
        rc = self.lib.vifo_decimate(_fp(plane), w, h, _fp(tap), len(tap),
                                    _fp(out))
        if rc != 0:
            raise ValueError("decimate rejected its arguments")
        return out

    def ordered_sums(self, num_t, den_t):
        """The ordered fp32 sums of two (h, w) term planes: returns
        (rows (h, 2) float32 of n_y, d_y; N float32; D float32)."""
        num_t = np.ascontiguousarray(num_t, dtype=np.float32)
        den_t = np.ascontiguousarray(den_t, dtype=np.float32)
        if num_t.shape != den_t.shape or num_t.ndim != 2:
            raise ValueError("two equal 2-D term planes needed")
        h, w = num_t.shape
        rows = np.zeros((h, 2), dtype=np.float32)
        n = np.zeros(1, dtype=np.float32)
        d = np.zeros(1, dtype=np.float32)
        rc = self.lib.vifo_ordered_sums(_fp(num_t), _fp(den_t), w, h,
                                        _fp(rows), _fp(n), _fp(d))
        if rc != 0:
            raise ValueError("vifo_ordered_sums rejected its arguments")
        return rows, n[0], d[0]

    def total_rows(self, w, h):
        return int(self.lib.vifo_total_rows(int(w), int(h)))

    def score(self, ref, dist, bpc, want_rows=False, options=None):
        """Return (out[8] float64, sums[8] float32[, rowsums (rows, 2)]).
        options: None (the default entry point) or a dict of overrides of
        DEFAULT_OPTIONS (through vifo_score_ex)."""
        ref = np.ascontiguousarray(ref)
        dist = np.ascontiguousarray(dist)
        if ref.shape != dist.shape or ref.ndim != 2:
            raise ValueError("ref and dist must be equal 2-D planes")
        want = np.uint8 if bpc == 8 else np.uint16
        if ref.dtype != want or dist.dtype != want:
            raise ValueError("bpc %d needs %s samples"
                             % (bpc, np.dtype(want).name))
        h, w = ref.shape
        out = np.zeros(8, dtype=np.float64)
        sums = np.zeros(8, dtype=np.float32)
        rows = None
        rp = None
        if want_rows:
            rows = np.zeros((self.total_rows(w, h), 2), dtype=np.float32)
            rp = _fp(rows)
        op = out.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
        if options is None:
            rc = self.lib.vifo_score(ref.ctypes.data, dist.ctypes.data, w, h,
                                     int(bpc), op, _fp(sums), rp)
        else:
            o = make_options(options)
            rc = self.lib.vifo_score_ex(ref.ctypes.data, dist.ctypes.data, w,
                                        h, int(bpc), ctypes.byref(o), op,
                                        _fp(sums), rp)
        if rc != 0:
            raise ValueError("vifo_score rejected its arguments (rc=%d)" % rc)
        if want_rows:
            return out, sums, rows
        return out, sums


    # ----------------------------------------------------- float SSIM
    def fssim_scale(self, w, h):
        return int(self.lib.fssimo_scale(int(w), int(h)))

    def fssim_decimated_size(self, n, f):
        return int(self.lib.fssimo_decimated_size(int(n), int(f)))

    def fssim_symmetric(self, i, n):
        return int(self.lib.fssimo_symmetric(int(i), int(n)))

    def fssim_decimate(self, plane, f):
        plane = np.ascontiguousarray(plane, dtype=np.float32)
        h, w = plane.shape
        ow = self.fssim_decimated_size(w, f)
        oh = self.fssim_decimated_size(h, f)
        out = np.empty((oh, ow), dtype=np.float32)
        if self.lib.fssimo_decimate(_fp(plane), w, h, int(f), _fp(out)) != 0:
            raise ValueError("fssimo_decimate rejected its arguments")
        return out

    def fssim_taps(self):
        t = np.zeros(11, dtype=np.float32)
        self.lib.fssimo_taps(_fp(t))
        return t

    def fssim_filter(self, plane):
        plane = np.ascontiguousarray(plane, dtype=np.float32)
        h, w = plane.shape
        out = np.empty((h, w), dtype=np.float32)
        if self.lib.fssimo_filter(_fp(plane), w, h, _fp(out)) != 0:
            raise ValueError("fssimo_filter rejected its arguments")
        return out

    def fssim_pixel(self, mu1, mu2, xx, yy, xy):
        return np.float32(self.lib.fssimo_pixel(
            *[float(np.float32(v)) for v in (mu1, mu2, xx, yy, xy)]))

    def fssim_score(self, ref, dist, bpc, want=False):
        """Return out[2] (float_ssim, factor); with want=True also the SSIM
        map, the decimated planes (2, h', w') and the fp64 row sums."""
        ref = np.ascontiguousarray(ref)
        dist = np.ascontiguousarray(dist)
        if ref.shape != dist.shape or ref.ndim != 2:
            raise ValueError("ref and dist must be equal 2-D planes")
        wantt = np.uint8 if bpc == 8 else np.uint16
        if ref.dtype != wantt or dist.dtype != wantt:
            raise ValueError("bpc %d needs %s samples"
                             % (bpc, np.dtype(wantt).name))
        h, w = ref.shape
        f = self.fssim_scale(w, h)
        ow = self.fssim_decimated_size(w, f) if f > 1 else w
        oh = self.fssim_decimated_size(h, f) if f > 1 else h
        out = np.zeros(2, dtype=np.float64)
        smap = np.zeros((oh, ow), dtype=np.float32) if want else None
        planes = np.zeros((2, oh, ow), dtype=np.float32) if want else None
        rows = np.zeros(oh, dtype=np.float64) if want else None
        rc = self.lib.fssimo_score(
            ref.ctypes.data, dist.ctypes.data, w, h, int(bpc),
            out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
            _fp(smap) if want else None, _fp(planes) if want else None,
            rows.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
            if want else None)
        if rc != 0:
            raise ValueError("fssimo_score rejected its arguments (rc=%d)"
                             % rc)
        if want:
            return out, smap, planes, rows
        return out


def _load():
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build()
        _default = Oracle(_LIB)
    return _default


def taps(scale):
    return _load().taps(scale)


def log2(x):
    return _load().log2(x)


def log2_array(xs):
    return _load().log2_array(xs)


def ratios(a, sv, nsq=None):
    return _load().ratios(a, sv, nsq)


def statistic(mu1, mu2, xx, yy, xy, nsq=None, gain_limit=None):
    return _load().statistic(mu1, mu2, xx, yy, xy, nsq, gain_limit)


def statistic_array(mu1, mu2, xx, yy, xy, nsq=None, gain_limit=None):
    return _load().statistic_array(mu1, mu2, xx, yy, xy, nsq, gain_limit)


def normalise(plane, bpc):
    return _load().normalise(plane, bpc)


def filter2d(plane, tap):
    return _load().filter2d(plane, tap)


def decimate(plane, tap):
    return _load().decimate(plane, tap)


def ordered_sums(num_t, den_t):
    return _load().ordered_sums(num_t, den_t)


def total_rows(w, h):
    return _load().total_rows(w, h)


def score(ref, dist, bpc, want_rows=False, options=None):
    return _load().score(ref, dist, bpc, want_rows, options)


def fssim_scale(w, h):
    return _load().fssim_scale(w, h)


def fssim_decimated_size(n, f):
    return _load().fssim_decimated_size(n, f)


def fssim_symmetric(i, n):
    return _load().fssim_symmetric(i, n)


def fssim_decimate(plane, f):
    return _load().fssim_decimate(plane, f)


def fssim_taps():
    return _load().fssim_taps()


def fssim_filter(plane):
    return _load().fssim_filter(plane)


def fssim_pixel(mu1, mu2, xx, yy, xy):
    return _load().fssim_pixel(mu1, mu2, xx, yy, xy)


def fssim_score(ref, dist, bpc, want=False):
    return _load().fssim_score(ref, dist, bpc, want)
