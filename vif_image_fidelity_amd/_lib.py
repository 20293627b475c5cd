"""ctypes binding of libvif_amd.so (include/vif.h, include/vif_selftest.h,
include/fssim.h).

Argument marshalling only: every step of the feature runs in the library's
HIP kernels.  The functions keep the C names.  Loading fails loudly when the
library has not been built; there is no CPU fallback.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvif_amd.so")

VIF_OK = 0
VIF_EINVAL = -1
VIF_ENOMEM = -2
VIF_EHIP = -3
VIF_ETOOBIG = -4
NOALLOC_SCRATCH = 32 << 20
NSCALES = 4
MAX_TAPS = 17
QUEUE_DEPTH = 3
MAX_BATCH = 16
STRIP_INFO = 10
MIN_SIDE = 16
MAX_PIXELS = 1 << 27
NDEBUG = 15
KERNEL_KINDS = ("scale0", "scale1", "scale2", "scale3")
FSSIM_TAPS = 11
FSSIM_QUEUE_DEPTH = 3
FSSIM_MAX_PIXELS = 1 << 27
FSSIM_MAX_FACTOR = 128
FSSIM_KERNEL_KINDS = ("decimate", "ssim", "rowsum")
DEBUG_NAMES = ("vif_scale0", "vif_scale1", "vif_scale2", "vif_scale3",
               "vif", "vif_num", "vif_den",
               "vif_num_scale0", "vif_den_scale0", "vif_num_scale1",
               "vif_den_scale1", "vif_num_scale2", "vif_den_scale2",
               "vif_num_scale3", "vif_den_scale3")


class VifOptions(ctypes.Structure):
    """struct vif_options of include/vif.h."""
    _fields_ = [("sigma_nsq", ctypes.c_double),
                ("enhn_gain_limit", ctypes.c_double),
                ("kernelscale", ctypes.c_double),
                ("scale_min_val", ctypes.c_double * 3),
                ("skip_scale0", ctypes.c_int),
                ("reserved", ctypes.c_int)]

_lib = None


class VifError(RuntimeError):
    def __init__(self, code, what):
        self.code = code
        super().__init__("%s failed: %s (code %d)" % (what, vif_strerror(code),
                                                      code))


def load():
    """Load the built library (once); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libvif_amd.so is not built (%s); run "
            "`python -m vif_image_fidelity_amd.build` first" % LIB_PATH)
    # PyTorch ships its own copy of the HIP runtime under the soname the
    # library links against.  Importing torch first makes the dynamic loader
    # bind the library to that copy: loaded the other way round, the process
    # holds two runtimes, and device pointers and streams of one are invalid
    # in the other.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, ip, fp = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_float)
    dp = ctypes.POINTER(ctypes.c_double)
    lp = ctypes.POINTER(ctypes.c_long)
    sig = {
        "vif_create": ([ip, ip, ip], vp),
        "vif_create_ex": ([ip, ip, ip, ctypes.POINTER(VifOptions)], vp),
        "vif_create_batch": ([ip, ip, ip, ctypes.POINTER(VifOptions), ip],
                             vp),
        "vif_submit_batch": ([vp, ip, ctypes.POINTER(vp),
                              ctypes.POINTER(vp)], ip),
        "vif_create_strip": ([ip, ip, ip, ctypes.POINTER(VifOptions), ip,
                              ip, ip], vp),
        "vif_strip_geometry": ([ip, ip, ip, ip, ctypes.POINTER(ip)], ip),
        "vif_scores_from_rows": ([ip, ip, ctypes.POINTER(VifOptions), fp, dp,
                                  fp], ip),
        "vif_score_noalloc": ([ip, ip, ip, ctypes.POINTER(VifOptions), vp,
                               vp, vp, dp], ip),
        "vif_default_options": ([ctypes.POINTER(VifOptions)], None),
        "vif_get_options": ([vp, ctypes.POINTER(VifOptions)], ip),
        "vif_get_debug": ([vp, dp], ip),
        "vif_score": ([vp, vp, vp, dp], ip),
        "vif_submit": ([vp, vp, vp], ip),
        "vif_submit_host": ([vp, vp, vp], ip),
        "vif_score_host": ([vp, vp, vp, dp], ip),
        "vif_collect": ([vp, dp], ip),
        "vif_pending": ([vp], ip),
        "vif_destroy": ([vp], None),
        "vif_set_stream": ([vp, vp], ip),
        "vif_get_sums": ([vp, fp], ip),
        "vif_get_row_sums": ([vp, fp, ip], ip),
        "vif_taps": ([ip, fp], ip),
        "vif_set_profiling": ([vp, ip], ip),
        "vif_get_kernel_times": ([vp, dp, lp, ip], ip),
        "vif_errno": ([], ip),
        "vif_strerror": ([ip], ctypes.c_char_p),
        "vif_selftest_fp64": ([vp, vp, ctypes.c_double, ctypes.c_long, vp, vp,
                               vp, vp, vp], ip),
        "vif_selftest_div32": ([vp, vp, ctypes.c_long, vp, vp], ip),
        "vif_selftest_div32_in_range": ([vp, vp, ctypes.c_long, vp, vp], ip),
        "vif_selftest_log2": ([vp, ctypes.c_long, vp, vp], ip),
        "vif_selftest_ratios": ([vp, vp, ctypes.c_double, ctypes.c_long, vp,
                                 vp, vp], ip),
        "vif_selftest_statistic": ([vp, vp, vp, vp, vp, ctypes.c_long,
                                    ctypes.c_double, ctypes.c_double, vp, vp,
                                    vp], ip),
        "vif_selftest_carry_wait": ([ctypes.POINTER(ip), fp, vp], ip),
        "vif_selftest_valu_rate": ([ip, ip, ctypes.c_long, vp, dp, vp], ip),
        "vif_selftest_stage_loads": ([ctypes.POINTER(vp), ctypes.POINTER(vp),
                                      ip, ip, ip, ip, vp, vp], ip),
        "fssim_create": ([ip, ip, ip], vp),
        "fssim_create_batch": ([ip, ip, ip, ip], vp),
        "fssim_submit_batch": ([vp, ip, ctypes.POINTER(vp),
                                ctypes.POINTER(vp)], ip),
        "fssim_destroy": ([vp], None),
        "fssim_geometry": ([vp, ctypes.POINTER(ctypes.c_int)], ip),
        "fssim_score": ([vp, vp, vp, dp], ip),
        "fssim_submit": ([vp, vp, vp], ip),
        "fssim_collect": ([vp, dp], ip),
        "fssim_pending": ([vp], ip),
        "fssim_set_stream": ([vp, vp], ip),
        "fssim_get_row_sums": ([vp, dp, ip], ip),
        "fssim_get_map": ([vp, fp, ctypes.c_long], ctypes.c_long),
        "fssim_get_planes": ([vp, fp, ctypes.c_long], ctypes.c_long),
        "fssim_taps": ([fp], ip),
        "fssim_set_profiling": ([vp, ip], ip),
        "fssim_get_kernel_times": ([vp, dp, lp, ip], ip),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def exported_symbols():
    """Names of every C function this binding declares."""
    return ["vif_default_options", "vif_create", "vif_create_ex",
            "vif_create_batch", "vif_submit_batch", "vif_create_strip",
            "vif_strip_geometry", "vif_scores_from_rows",
            "vif_score_noalloc",
            "vif_get_options", "vif_score", "vif_submit", "vif_collect",
            "vif_submit_host", "vif_score_host",
            "vif_pending", "vif_get_debug",
            "vif_destroy", "vif_set_stream",
            "vif_get_sums", "vif_get_row_sums", "vif_taps",
            "vif_set_profiling", "vif_get_kernel_times", "vif_errno",
            "vif_strerror", "vif_selftest_fp64", "vif_selftest_div32",
            "vif_selftest_div32_in_range",
            "vif_selftest_log2", "vif_selftest_ratios",
            "vif_selftest_statistic", "vif_selftest_carry_wait",
            "vif_selftest_valu_rate", "vif_selftest_stage_loads",
            "fssim_create", "fssim_create_batch", "fssim_submit_batch",
            "fssim_destroy", "fssim_geometry", "fssim_score",
            "fssim_submit", "fssim_collect", "fssim_pending",
            "fssim_set_stream", "fssim_get_row_sums", "fssim_get_map",
            "fssim_get_planes", "fssim_taps", "fssim_set_profiling",
            "fssim_get_kernel_times"]


# ------------------------------------------------------- C-named wrappers

def vif_create(w, h, bpc):
    return load().vif_create(int(w), int(h), int(bpc))


def vif_default_options():
    o = VifOptions()
    load().vif_default_options(ctypes.byref(o))
    return o


def vif_create_ex(w, h, bpc, options):
    """options: a VifOptions or None (the defaults)."""
    return load().vif_create_ex(int(w), int(h), int(bpc),
                                None if options is None
                                else ctypes.byref(options))


def vif_create_batch(w, h, bpc, options, max_batch):
    """options: a VifOptions or None (the defaults)."""
    return load().vif_create_batch(int(w), int(h), int(bpc),
                                   None if options is None
                                   else ctypes.byref(options), int(max_batch))


def vif_create_strip(w, h, bpc, options, max_batch, row0, row1):
    """options: a VifOptions or None (the defaults)."""
    return load().vif_create_strip(int(w), int(h), int(bpc),
                                   None if options is None
                                   else ctypes.byref(options), int(max_batch),
                                   int(row0), int(row1))


def vif_strip_geometry(w, h, row0, row1, info):
    """info: a contiguous int32 numpy array of STRIP_INFO entries."""
    return load().vif_strip_geometry(
        int(w), int(h), int(row0), int(row1),
        ctypes.cast(info.ctypes.data, ctypes.POINTER(ctypes.c_int)))


def vif_scores_from_rows(w, h, options, rows, out, sums):
    """rows: float32 (h + h/2 + h/4 + h/8, 2); out: float64[8]; sums:
    float32[8] or None; options: a VifOptions or None."""
    return load().vif_scores_from_rows(
        int(w), int(h), None if options is None else ctypes.byref(options),
        _fptr(rows), _dptr(out), None if sums is None else _fptr(sums))


def vif_score_noalloc(w, h, bpc, options, ref_ptr, dist_ptr, stream, out):
    """options: a VifOptions or None; stream: a hipStream_t (int) or None;
    out: a float64[8] numpy array."""
    return load().vif_score_noalloc(
        int(w), int(h), int(bpc),
        None if options is None else ctypes.byref(options), ref_ptr,
        dist_ptr, stream, _dptr(out))


def vif_submit_batch(ctx, ref_ptrs, dist_ptrs):
    """ref_ptrs, dist_ptrs: equal-length sequences of device pointers."""
    n = len(ref_ptrs)
    if len(dist_ptrs) != n:
        raise ValueError("as many distorted as reference frames")
    arr = ctypes.c_void_p * max(n, 1)
    return load().vif_submit_batch(ctx, n, arr(*ref_ptrs), arr(*dist_ptrs))


def vif_get_options(ctx, options):
    return load().vif_get_options(ctx, ctypes.byref(options))


def vif_get_debug(ctx, out):
    return load().vif_get_debug(ctx, _dptr(out))


def vif_score(ctx, ref_ptr, dist_ptr, out):
    """out: a ctypes double[8] or a contiguous float64 numpy array."""
    return load().vif_score(ctx, ref_ptr, dist_ptr, _dptr(out))


def vif_submit(ctx, ref_ptr, dist_ptr):
    return load().vif_submit(ctx, ref_ptr, dist_ptr)


def vif_submit_host(ctx, ref_ptr, dist_ptr):
    return load().vif_submit_host(ctx, ref_ptr, dist_ptr)


def vif_score_host(ctx, ref_ptr, dist_ptr, out):
    return load().vif_score_host(ctx, ref_ptr, dist_ptr, _dptr(out))


def vif_collect(ctx, out):
    return load().vif_collect(ctx, _dptr(out))


def vif_pending(ctx):
    return load().vif_pending(ctx)


def vif_destroy(ctx):
    load().vif_destroy(ctx)


def vif_set_stream(ctx, stream_ptr):
    return load().vif_set_stream(ctx, stream_ptr)


def vif_get_sums(ctx, sums):
    return load().vif_get_sums(ctx, _fptr(sums))


def vif_get_row_sums(ctx, rows, capacity):
    return load().vif_get_row_sums(ctx, _fptr(rows), int(capacity))


def vif_taps(scale, taps):
    return load().vif_taps(int(scale), _fptr(taps))


def vif_set_profiling(ctx, enable):
    return load().vif_set_profiling(ctx, int(enable))


def vif_get_kernel_times(ctx, ms, launches, capacity):
    return load().vif_get_kernel_times(
        ctx, _dptr(ms), ctypes.cast(launches.ctypes.data,
                                    ctypes.POINTER(ctypes.c_long)),
        int(capacity))


def vif_errno():
    return load().vif_errno()


def vif_strerror(code):
    return load().vif_strerror(int(code)).decode()


def fssim_create(w, h, bpc):
    return load().fssim_create(int(w), int(h), int(bpc))


def fssim_create_batch(w, h, bpc, max_batch):
    return load().fssim_create_batch(int(w), int(h), int(bpc),
                                     int(max_batch))


def fssim_submit_batch(ctx, ref_ptrs, dist_ptrs):
    n = len(ref_ptrs)
    if len(dist_ptrs) != n:
        raise ValueError("as many distorted as reference frames")
    arr = ctypes.c_void_p * max(n, 1)
    return load().fssim_submit_batch(ctx, n, arr(*ref_ptrs), arr(*dist_ptrs))


def fssim_destroy(ctx):
    load().fssim_destroy(ctx)


def fssim_geometry(ctx, geom):
    """geom: a contiguous int32 numpy array of 3."""
    return load().fssim_geometry(
        ctx, ctypes.cast(geom.ctypes.data, ctypes.POINTER(ctypes.c_int)))


def fssim_score(ctx, ref_ptr, dist_ptr, out):
    return load().fssim_score(ctx, ref_ptr, dist_ptr, _dptr(out))


def fssim_submit(ctx, ref_ptr, dist_ptr):
    return load().fssim_submit(ctx, ref_ptr, dist_ptr)


def fssim_collect(ctx, out):
    return load().fssim_collect(ctx, _dptr(out))


def fssim_pending(ctx):
    return load().fssim_pending(ctx)


def fssim_set_stream(ctx, stream_ptr):
    return load().fssim_set_stream(ctx, stream_ptr)


def fssim_get_row_sums(ctx, rows, capacity):
    return load().fssim_get_row_sums(ctx, _dptr(rows), int(capacity))


def fssim_get_map(ctx, smap, capacity):
    return load().fssim_get_map(ctx, _fptr(smap), int(capacity))


def fssim_get_planes(ctx, planes, capacity):
    return load().fssim_get_planes(ctx, _fptr(planes), int(capacity))


def fssim_taps(taps):
    return load().fssim_taps(_fptr(taps))


def fssim_set_profiling(ctx, kinds):
    return load().fssim_set_profiling(ctx, int(kinds))


def fssim_get_kernel_times(ctx, ms, launches, capacity):
    return load().fssim_get_kernel_times(
        ctx, _dptr(ms), ctypes.cast(launches.ctypes.data,
                                    ctypes.POINTER(ctypes.c_long)),
        int(capacity))


def _fptr(a):
    return ctypes.cast(a.ctypes.data, ctypes.POINTER(ctypes.c_float))


def _dptr(a):
    if isinstance(a, ctypes.Array):
        return a
    return ctypes.cast(a.ctypes.data, ctypes.POINTER(ctypes.c_double))
