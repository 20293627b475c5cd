"""MI355X-native float VIF (visual information fidelity) feature, and the
float SSIM feature with its exact decimation.

``Vif(w, h, bpc)`` wraps one scoring context of the C-ABI library
(include/vif.h); ``FloatSsim(w, h, bpc)`` one of include/fssim.h.  Frames
are device buffers (torch tensors on a ROCm device, or raw device
pointers); every step of either feature runs in the library's HIP kernels
for gfx950, and torch only supplies memory and streams.  There is no CPU
fallback: if the library is not built, using ``Vif`` or ``FloatSsim``
raises.

The synthetic workload generators live in ``vif_image_fidelity_amd.synth``
and need neither the library nor a GPU.
"""
import collections

import numpy as np

from . import _lib
from ._lib import (VIF_EHIP, VIF_EINVAL, VIF_ENOMEM, VIF_OK, VifError,
                   VIF_ETOOBIG, NOALLOC_SCRATCH,
                   DEBUG_NAMES, KERNEL_KINDS, QUEUE_DEPTH, MAX_BATCH,
                   MIN_SIDE, MAX_PIXELS, FSSIM_KERNEL_KINDS,
                   FSSIM_QUEUE_DEPTH, FSSIM_MAX_PIXELS, FSSIM_MAX_FACTOR)

__all__ = ["Vif", "VifError", "FloatSsim", "fssim_taps", "taps",
           "strip_geometry", "scores_from_rows", "score_noalloc",
           "make_options", "DEFAULT_OPTIONS",
           "VIF_OK", "VIF_EINVAL", "VIF_ENOMEM", "VIF_EHIP", "DEBUG_NAMES",
           "KERNEL_KINDS", "QUEUE_DEPTH", "MAX_BATCH", "MIN_SIDE",
           "MAX_PIXELS", "FSSIM_KERNEL_KINDS", "FSSIM_QUEUE_DEPTH",
           "FSSIM_MAX_PIXELS", "FSSIM_MAX_FACTOR"]

# Defaults of struct vif_options (include/vif.h states each option's
# meaning and range).
DEFAULT_OPTIONS = {"sigma_nsq": 2.0, "enhn_gain_limit": 100.0,
                   "kernelscale": 1.0, "scale_min_val": (0.0, 0.0, 0.0),
                   "skip_scale0": 0}


def make_options(options=None):
    """A struct vif_options from a dict of overrides of DEFAULT_OPTIONS."""
    d = dict(DEFAULT_OPTIONS)
    if options:
        unknown = set(options) - set(d)
        if unknown:
            raise ValueError("unknown options %s" % sorted(unknown))
        d.update(options)
    o = _lib.VifOptions()
    o.sigma_nsq = float(d["sigma_nsq"])
    o.enhn_gain_limit = float(d["enhn_gain_limit"])
    o.kernelscale = float(d["kernelscale"])
    floors = [float(v) for v in d["scale_min_val"]]
    if len(floors) != 3:
        raise ValueError("scale_min_val needs three floors")
    o.scale_min_val[:] = floors
    o.skip_scale0 = int(d["skip_scale0"])
    o.reserved = 0
    return o


def taps(scale):
    """Host Gaussian taps of scale 0..3 as the library computes them."""
    buf = np.zeros(_lib.MAX_TAPS, dtype=np.float32)
    n = _lib.vif_taps(scale, buf)
    if n < 0:
        raise VifError(n, "vif_taps")
    return buf[:n].copy()


def _ptr(x):
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if not x.is_cuda:
            raise ValueError("frames must be device tensors")
        if not x.is_contiguous():
            raise ValueError("frames must be contiguous")
        return x.data_ptr()
    raise TypeError("expected a device tensor or a device pointer")


class Vif:
    """One scoring context for w x h frames of bpc bits (8, 10, 12, 16).
    options: None or a dict of overrides of DEFAULT_OPTIONS."""

    def __init__(self, w, h, bpc, stream=None, options=None, max_batch=1,
                 strip=None):
        """strip: None, or (row0, row1) for a context that scores scale-0
        rows [row0, row1) of w x h frames (vif_create_strip): its frames are
        the strip's input rows, shape (in_rows, w) from input row in0
        (strip_geometry), and its outputs cover its own rows."""
        self.w, self.h, self.bpc = int(w), int(h), int(bpc)
        self.max_batch = int(max_batch)
        self.strip = None if strip is None else tuple(int(r) for r in strip)
        self.in0, self.in_rows = 0, self.h
        if self.strip is not None:
            g = strip_geometry(self.w, self.h, *self.strip)
            self.in0, self.in_rows = g["in0"], g["in_rows"]
            ctx = _lib.vif_create_strip(
                self.w, self.h, self.bpc,
                None if options is None else make_options(options),
                self.max_batch, *self.strip)
        elif self.max_batch != 1:
            ctx = _lib.vif_create_batch(
                self.w, self.h, self.bpc,
                None if options is None else make_options(options),
                self.max_batch)
        elif options is None:
            ctx = _lib.vif_create(self.w, self.h, self.bpc)
        else:
            ctx = _lib.vif_create_ex(self.w, self.h, self.bpc,
                                     make_options(options))
        if not ctx:
            raise VifError(_lib.vif_errno(), "vif_create")
        self._ctx = ctx
        # the frames of every pending submission, oldest first: held here
        # until their collect() returns, so the memory of a temporary frame
        # is not reused while the kernels still read it
        self._inflight = collections.deque()
        if self.strip is None:
            self.total_rows = sum((self.h >> s) for s in range(4))
        else:
            self.total_rows = sum(g["own_rows"])
        if stream is not None:
            self.set_stream(stream)

    def set_stream(self, stream):
        """stream: a torch.cuda.Stream, a raw hipStream_t (int) or None."""
        ptr = getattr(stream, "cuda_stream", stream)
        rc = _lib.vif_set_stream(self._ctx, ptr)
        if rc != VIF_OK:
            raise VifError(rc, "vif_set_stream")

    def _check_frame(self, t):
        if hasattr(t, "shape"):
            if tuple(t.shape) != (self.in_rows, self.w):
                raise ValueError("frame shape %s, context is (%d, %d)"
                                 % (tuple(t.shape), self.in_rows, self.w))
            want = 1 if self.bpc == 8 else 2
            if t.element_size() != want:
                raise ValueError("bpc %d needs %d-byte samples"
                                 % (self.bpc, want))

    def score(self, ref, dist):
        """Score one pair; returns float64[8]: vif_scale0..3, num, den,
        num/den, 0."""
        self._check_frame(ref)
        self._check_frame(dist)
        out = np.zeros(8, dtype=np.float64)
        rc = _lib.vif_score(self._ctx, _ptr(ref), _ptr(dist), out)
        if rc != VIF_OK:
            raise VifError(rc, "vif_score")
        return out

    def _host_ptr(self, a):
        """Address of a host plane: a C-contiguous numpy array (or a CPU
        tensor) of shape (h, w) with the context's sample width."""
        if hasattr(a, "data_ptr"):
            if a.is_cuda:
                raise ValueError("host frames must be CPU memory")
            if not a.is_contiguous():
                raise ValueError("frames must be contiguous")
            self._check_frame(a)
            return a.data_ptr()
        if not isinstance(a, np.ndarray):
            raise TypeError("expected a numpy array or a CPU tensor")
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("frames must be contiguous")
        if a.shape != (self.in_rows, self.w):
            raise ValueError("frame shape %s, context is (%d, %d)"
                             % (a.shape, self.in_rows, self.w))
        if a.dtype != (np.uint8 if self.bpc == 8 else np.uint16):
            raise ValueError("bpc %d needs %s samples"
                             % (self.bpc, "uint8" if self.bpc == 8
                                else "uint16"))
        return a.ctypes.data

    def score_host(self, ref, dist):
        """Score one pair held in host memory (copied by the library)."""
        out = np.zeros(8, dtype=np.float64)
        rc = _lib.vif_score_host(self._ctx, self._host_ptr(ref),
                                 self._host_ptr(dist), out)
        if rc != VIF_OK:
            raise VifError(rc, "vif_score_host")
        return out

    def submit_host(self, ref, dist):
        """Enqueue one pair held in host memory; the arrays must stay
        unchanged until the matching collect() returns (the context holds a
        reference to them until then)."""
        rc = _lib.vif_submit_host(self._ctx, self._host_ptr(ref),
                                  self._host_ptr(dist))
        if rc != VIF_OK:
            raise VifError(rc, "vif_submit_host")
        self._inflight.append((ref, dist))

    def submit(self, ref, dist):
        """Enqueue one pair (at most QUEUE_DEPTH pending); the frames must
        stay unchanged until the matching collect() returns (the context
        holds a reference to them until then)."""
        self._check_frame(ref)
        self._check_frame(dist)
        rc = _lib.vif_submit(self._ctx, _ptr(ref), _ptr(dist))
        if rc != VIF_OK:
            raise VifError(rc, "vif_submit")
        self._inflight.append((ref, dist))

    def submit_batch(self, refs, dists):
        """Enqueue len(refs) pairs (at most max_batch) as one submission:
        each kernel runs once for all of them.  collect() returns them one
        by one, in order."""
        for t in list(refs) + list(dists):
            self._check_frame(t)
        rc = _lib.vif_submit_batch(self._ctx, [_ptr(r) for r in refs],
                                   [_ptr(d) for d in dists])
        if rc != VIF_OK:
            raise VifError(rc, "vif_submit_batch")
        self._inflight.extend(zip(refs, dists))

    def collect(self):
        """Outputs of the oldest submitted pair (float64[8])."""
        out = np.zeros(8, dtype=np.float64)
        rc = _lib.vif_collect(self._ctx, out)
        # drop the frames the library no longer holds (after an error too)
        while len(self._inflight) > _lib.vif_pending(self._ctx):
            self._inflight.popleft()
        if rc != VIF_OK:
            raise VifError(rc, "vif_collect")
        return out

    def pending(self):
        return _lib.vif_pending(self._ctx)

    def sums(self):
        s = np.zeros(8, dtype=np.float32)
        rc = _lib.vif_get_sums(self._ctx, s)
        if rc != VIF_OK:
            raise VifError(rc, "vif_get_sums")
        return s

    def options(self):
        """The context's options as a dict."""
        o = _lib.VifOptions()
        rc = _lib.vif_get_options(self._ctx, o)
        if rc != VIF_OK:
            raise VifError(rc, "vif_get_options")
        return {"sigma_nsq": o.sigma_nsq,
                "enhn_gain_limit": o.enhn_gain_limit,
                "kernelscale": o.kernelscale,
                "scale_min_val": tuple(o.scale_min_val),
                "skip_scale0": o.skip_scale0}

    def debug(self):
        """The fifteen debug values of the last frame, {name: value} in
        DEBUG_NAMES order."""
        out = np.zeros(_lib.NDEBUG, dtype=np.float64)
        rc = _lib.vif_get_debug(self._ctx, out)
        if rc != VIF_OK:
            raise VifError(rc, "vif_get_debug")
        return dict(zip(DEBUG_NAMES, out.tolist()))

    def row_sums(self):
        rows = np.zeros((self.total_rows, 2), dtype=np.float32)
        rc = _lib.vif_get_row_sums(self._ctx, rows, self.total_rows)
        if rc < 0:
            raise VifError(rc, "vif_get_row_sums")
        return rows

    def set_profiling(self, kinds=0xF):
        """Time the kernel kinds in the bit mask (0xF all, 0 off); a list
        of kind names is accepted too."""
        if isinstance(kinds, (list, tuple)):
            kinds = sum(1 << KERNEL_KINDS.index(k) for k in kinds)
        elif kinds is True:
            kinds = (1 << len(KERNEL_KINDS)) - 1
        elif kinds is False or kinds is None:
            kinds = 0
        rc = _lib.vif_set_profiling(self._ctx, int(kinds))
        if rc != VIF_OK:
            raise VifError(rc, "vif_set_profiling")

    def kernel_times(self):
        """{kind: (total_ms, launches)} since profiling was enabled."""
        k = len(KERNEL_KINDS)
        ms = np.zeros(k, dtype=np.float64)
        n = np.zeros(k, dtype=np.int64)
        rc = _lib.vif_get_kernel_times(self._ctx, ms, n, k)
        if rc < 0:
            raise VifError(rc, "vif_get_kernel_times")
        return {k: (float(ms[i]), int(n[i]))
                for i, k in enumerate(KERNEL_KINDS)}

    def close(self):
        if getattr(self, "_ctx", None):
            _lib.vif_destroy(self._ctx)  # waits for pending work
            self._ctx = None
        getattr(self, "_inflight", collections.deque()).clear()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def score_noalloc(ref, dist, bpc, options=None, stream=None):
    """Score one pair with vif_score_noalloc: no context and no allocation
    (the library's fixed device array holds the intermediate buffers).
    ref, dist: device tensors (h, w) or device pointers with the sizes given
    by the tensors; returns float64[8] as Vif.score."""
    h, w = (int(v) for v in ref.shape)
    if tuple(dist.shape) != (h, w):
        raise ValueError("ref and dist differ in shape")
    out = np.zeros(8, dtype=np.float64)
    sp = getattr(stream, "cuda_stream", stream)
    rc = _lib.vif_score_noalloc(w, h, int(bpc),
                                None if options is None
                                else make_options(options),
                                _ptr(ref), _ptr(dist), sp, out)
    if rc != VIF_OK:
        raise VifError(rc, "vif_score_noalloc")
    return out


def strip_geometry(w, h, row0, row1):
    """The rows a strip of scale-0 rows [row0, row1) of w x h frames reads
    and owns (vif_strip_geometry): {"in0", "in_rows", "own0": [4],
    "own_rows": [4]}."""
    info = np.zeros(_lib.STRIP_INFO, dtype=np.int32)
    rc = _lib.vif_strip_geometry(w, h, row0, row1, info)
    if rc != VIF_OK:
        raise VifError(rc, "vif_strip_geometry")
    return {"in0": int(info[0]), "in_rows": int(info[1]),
            "own0": [int(v) for v in info[2::2]],
            "own_rows": [int(v) for v in info[3::2]]}


def scores_from_rows(w, h, rows, options=None):
    """out[8] and the eight fp32 sums of a w x h frame from its row sums
    (vif_scores_from_rows): rows is (h + h/2 + h/4 + h/8, 2) float32, scale
    by scale, top to bottom."""
    rows = np.ascontiguousarray(rows, dtype=np.float32)
    need = sum(int(h) >> s for s in range(4))
    if rows.shape != (need, 2):
        raise ValueError("rows must be (%d, 2)" % need)
    out = np.zeros(8, dtype=np.float64)
    sums = np.zeros(8, dtype=np.float32)
    rc = _lib.vif_scores_from_rows(w, h, None if options is None
                                   else make_options(options), rows, out,
                                   sums)
    if rc != VIF_OK:
        raise VifError(rc, "vif_scores_from_rows")
    return out, sums


def fssim_taps():
    """The 11 fp32 SSIM window taps as the library passes them."""
    buf = np.zeros(_lib.FSSIM_TAPS, dtype=np.float32)
    n = _lib.fssim_taps(buf)
    if n < 0:
        raise VifError(n, "fssim_taps")
    return buf


class FloatSsim:
    """One float SSIM scoring context for w x h frames of bpc bits (8, 10,
    12, 16).  The frame is decimated by factor() first when that is above
    1; geometry() gives (factor, w', h')."""

    def __init__(self, w, h, bpc, stream=None, max_batch=1):
        self.w, self.h, self.bpc = int(w), int(h), int(bpc)
        self.max_batch = int(max_batch)
        if self.max_batch != 1:
            ctx = _lib.fssim_create_batch(self.w, self.h, self.bpc,
                                          self.max_batch)
        else:
            ctx = _lib.fssim_create(self.w, self.h, self.bpc)
        if not ctx:
            raise VifError(_lib.vif_errno(), "fssim_create")
        self._ctx = ctx
        self._inflight = collections.deque()  # as in Vif
        g = np.zeros(3, dtype=np.int32)
        rc = _lib.fssim_geometry(ctx, g)
        if rc != VIF_OK:
            raise VifError(rc, "fssim_geometry")
        self.factor, self.ow, self.oh = (int(v) for v in g)
        if stream is not None:
            self.set_stream(stream)

    def geometry(self):
        return self.factor, self.ow, self.oh

    def set_stream(self, stream):
        ptr = getattr(stream, "cuda_stream", stream)
        rc = _lib.fssim_set_stream(self._ctx, ptr)
        if rc != VIF_OK:
            raise VifError(rc, "fssim_set_stream")

    def _check_frame(self, t):
        if hasattr(t, "shape"):
            if tuple(t.shape) != (self.h, self.w):
                raise ValueError("frame shape %s, context is (%d, %d)"
                                 % (tuple(t.shape), self.h, self.w))
            want = 1 if self.bpc == 8 else 2
            if t.element_size() != want:
                raise ValueError("bpc %d needs %d-byte samples"
                                 % (self.bpc, want))

    def score(self, ref, dist):
        """Score one pair; returns float64[2]: float_ssim, factor."""
        self._check_frame(ref)
        self._check_frame(dist)
        out = np.zeros(2, dtype=np.float64)
        rc = _lib.fssim_score(self._ctx, _ptr(ref), _ptr(dist), out)
        if rc != VIF_OK:
            raise VifError(rc, "fssim_score")
        return out

    def submit(self, ref, dist):
        self._check_frame(ref)
        self._check_frame(dist)
        rc = _lib.fssim_submit(self._ctx, _ptr(ref), _ptr(dist))
        if rc != VIF_OK:
            raise VifError(rc, "fssim_submit")
        self._inflight.append((ref, dist))

    def submit_batch(self, refs, dists):
        """Enqueue len(refs) pairs (at most max_batch) as one submission."""
        for t in list(refs) + list(dists):
            self._check_frame(t)
        rc = _lib.fssim_submit_batch(self._ctx, [_ptr(r) for r in refs],
                                     [_ptr(d) for d in dists])
        if rc != VIF_OK:
            raise VifError(rc, "fssim_submit_batch")
        self._inflight.extend(zip(refs, dists))

    def collect(self):
        out = np.zeros(2, dtype=np.float64)
        rc = _lib.fssim_collect(self._ctx, out)
        while len(self._inflight) > _lib.fssim_pending(self._ctx):
            self._inflight.popleft()
        if rc != VIF_OK:
            raise VifError(rc, "fssim_collect")
        return out

    def pending(self):
        return _lib.fssim_pending(self._ctx)

    def row_sums(self):
        rows = np.zeros(self.oh, dtype=np.float64)
        rc = _lib.fssim_get_row_sums(self._ctx, rows, self.oh)
        if rc < 0:
            raise VifError(rc, "fssim_get_row_sums")
        return rows

    def ssim_map(self):
        m = np.zeros((self.oh, self.ow), dtype=np.float32)
        rc = _lib.fssim_get_map(self._ctx, m, m.size)
        if rc < 0:
            raise VifError(int(rc), "fssim_get_map")
        return m

    def planes(self):
        p = np.zeros((2, self.oh, self.ow), dtype=np.float32)
        rc = _lib.fssim_get_planes(self._ctx, p, p.size)
        if rc < 0:
            raise VifError(int(rc), "fssim_get_planes")
        return p

    def set_profiling(self, kinds=0x7):
        rc = _lib.fssim_set_profiling(self._ctx, int(kinds))
        if rc != VIF_OK:
            raise VifError(rc, "fssim_set_profiling")

    def kernel_times(self):
        k = len(FSSIM_KERNEL_KINDS)
        ms = np.zeros(k, dtype=np.float64)
        n = np.zeros(k, dtype=np.int64)
        rc = _lib.fssim_get_kernel_times(self._ctx, ms, n, k)
        if rc < 0:
            raise VifError(rc, "fssim_get_kernel_times")
        return {kk: (float(ms[i]), int(n[i]))
                for i, kk in enumerate(FSSIM_KERNEL_KINDS)}

    def close(self):
        if getattr(self, "_ctx", None):
            _lib.fssim_destroy(self._ctx)  # waits for pending work
            self._ctx = None
        getattr(self, "_inflight", collections.deque()).clear()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
