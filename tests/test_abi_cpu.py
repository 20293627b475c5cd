"""The C-ABI library on the CPU: it loads, exports every symbol the headers
declare, and its host logic (taps, argument checks, error strings, fault
injection) behaves as documented.  No kernel runs here."""
import ctypes
import os
import subprocess
import sys

import numpy as np
import pytest

from libutil import ROOT, ensure_built, header_functions


@pytest.fixture(scope="module")
def lib():
    return ensure_built()


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert "vif_create" in names and "vif_score" in names
    assert "vif_destroy" in names
    for n in names:
        assert hasattr(lib, n), n
    r = subprocess.run(["nm", "-D", "--defined-only",
                        os.path.join(ROOT, "vif_image_fidelity_amd",
                                     "libvif_amd.so")],
                       capture_output=True, text=True, check=True)
    exported = {ln.split()[-1] for ln in r.stdout.splitlines() if ln.strip()}
    for n in names:
        assert n in exported, n
    # the binding declares exactly the header's functions
    from vif_image_fidelity_amd import _lib
    assert sorted(_lib.exported_symbols()) == names


def test_library_taps_equal_oracle_taps(lib, orc):
    """The library's host tap generator and the oracle's, written separately
    from the same definition, agree bit for bit."""
    import vif_image_fidelity_amd as V
    for s in range(4):
        a = V.taps(s)
        b = orc.taps(s)
        assert a.tobytes() == b.tobytes(), s


def test_valu_rate_rejects_bad_arguments(lib):
    """The issue-rate microbenchmark refuses occupancies, round counts and
    grid sizes outside its ranges before it touches a device."""
    import ctypes
    from vif_image_fidelity_amd import _lib
    ms = ctypes.c_double(0.0)
    dummy = ctypes.c_void_p(256)   # never dereferenced: the checks come first
    for w, it, nb in ((2, 1, 1), (9, 1, 1), (6, 0, 1), (6, 1 << 25, 1),
                      (6, 1, 0), (6, 1, 1 << 25)):
        assert lib.vif_selftest_valu_rate(w, it, nb, dummy, ctypes.byref(ms),
                                          None) == _lib.VIF_EINVAL, (w, it, nb)
    assert lib.vif_selftest_valu_rate(6, 1, 1, None, ctypes.byref(ms),
                                      None) == _lib.VIF_EINVAL
    assert lib.vif_selftest_valu_rate(6, 1, 1, dummy, None,
                                      None) == _lib.VIF_EINVAL
    assert ms.value == 0.0


def test_taps_bad_scale(lib):
    buf = np.zeros(17, np.float32)
    from vif_image_fidelity_amd import _lib
    assert _lib.vif_taps(4, buf) == _lib.VIF_EINVAL
    assert _lib.vif_taps(-1, buf) == _lib.VIF_EINVAL
    assert _lib.vif_errno() == _lib.VIF_EINVAL


@pytest.mark.parametrize("w,h,bpc", [(15, 16, 8), (16, 15, 8), (0, 0, 8),
                                     (16, 16, 9), (16, 16, 0), (16, 16, 32),
                                     (1 << 14, 1 << 14, 8), (-16, 16, 8)])
def test_create_rejects_bad_arguments(lib, w, h, bpc):
    """Geometry and bit depth are refused at create time, before any device
    call (so this runs without a GPU)."""
    from vif_image_fidelity_amd import _lib
    ctx = _lib.vif_create(w, h, bpc)
    assert not ctx
    assert _lib.vif_errno() == _lib.VIF_EINVAL


def test_default_options(lib):
    from vif_image_fidelity_amd import _lib
    import vif_image_fidelity_amd as V
    o = _lib.vif_default_options()
    assert (o.sigma_nsq, o.enhn_gain_limit, o.kernelscale) == (2.0, 100.0,
                                                               1.0)
    assert tuple(o.scale_min_val) == (0.0, 0.0, 0.0)
    assert (o.skip_scale0, o.reserved) == (0, 0)
    m = V.make_options({})
    for f, _ in _lib.VifOptions._fields_:
        a, b = getattr(o, f), getattr(m, f)
        if f == "scale_min_val":
            a, b = tuple(a), tuple(b)
        assert a == b, f
    _lib.load().vif_default_options(None)  # NULL-safe


@pytest.mark.parametrize("opt", [{"kernelscale": 2.0}, {"kernelscale": 0.0},
                                 {"sigma_nsq": -1e-9},
                                 {"sigma_nsq": float("nan")},
                                 {"sigma_nsq": float("inf")},
                                 {"enhn_gain_limit": -1.0},
                                 {"enhn_gain_limit": float("nan")},
                                 {"scale_min_val": (0.0, 0.0, float("nan"))},
                                 {"skip_scale0": 2}, {"skip_scale0": -1}])
def test_create_ex_rejects_bad_options(lib, opt):
    """Options outside their ranges are refused at create time, before any
    device call (so this runs without a GPU)."""
    from vif_image_fidelity_amd import _lib
    import vif_image_fidelity_amd as V
    ctx = _lib.vif_create_ex(64, 64, 8, V.make_options(opt))
    assert not ctx
    assert _lib.vif_errno() == _lib.VIF_EINVAL


def test_create_ex_rejects_reserved_field(lib):
    from vif_image_fidelity_amd import _lib
    o = _lib.vif_default_options()
    o.reserved = 1
    assert not _lib.vif_create_ex(64, 64, 8, o)
    assert _lib.vif_errno() == _lib.VIF_EINVAL


def test_options_struct_layout(lib):
    """The ctypes mirror of struct vif_options has the C layout (six
    doubles, two ints: 56 bytes, no padding)."""
    import ctypes
    from vif_image_fidelity_amd import _lib
    assert ctypes.sizeof(_lib.VifOptions) == 56
    assert _lib.VifOptions.skip_scale0.offset == 48


def test_unknown_option_rejected(lib):
    import vif_image_fidelity_amd as V
    with pytest.raises(ValueError):
        V.make_options({"nsq": 1.0})


def test_null_handling(lib):
    from vif_image_fidelity_amd import _lib
    out = np.zeros(8)
    assert _lib.vif_score(None, 1, 1, out) == _lib.VIF_EINVAL
    assert _lib.vif_set_stream(None, None) == _lib.VIF_EINVAL
    assert _lib.vif_get_sums(None, np.zeros(8, np.float32)) == _lib.VIF_EINVAL
    assert _lib.vif_set_profiling(None, 1) == _lib.VIF_EINVAL
    assert _lib.vif_submit(None, 1, 1) == _lib.VIF_EINVAL
    assert _lib.vif_collect(None, out) == _lib.VIF_EINVAL
    assert _lib.vif_pending(None) == _lib.VIF_EINVAL
    assert _lib.vif_submit_host(None, 1, 1) == _lib.VIF_EINVAL
    assert _lib.vif_score_host(None, 1, 1, out) == _lib.VIF_EINVAL
    assert _lib.vif_get_debug(None, np.zeros(15)) == _lib.VIF_EINVAL
    assert _lib.vif_get_options(None, _lib.VifOptions()) == _lib.VIF_EINVAL
    _lib.vif_destroy(None)  # no-op


def test_selftests_reject_bad_arguments(lib):
    from vif_image_fidelity_amd import _lib
    L = _lib.load()
    assert L.vif_selftest_log2(None, 10, None, None) == _lib.VIF_EINVAL
    assert L.vif_selftest_log2(None, -1, None, None) == _lib.VIF_EINVAL
    assert L.vif_selftest_div32(None, None, 5, None, None) == _lib.VIF_EINVAL
    assert L.vif_selftest_fp64(None, None, 2.0, 3, None, None, None, None,
                               None) == _lib.VIF_EINVAL
    # n == 0 is a no-op success without touching the device
    assert L.vif_selftest_log2(None, 0, None, None) == _lib.VIF_OK


def test_strerror(lib):
    from vif_image_fidelity_amd import _lib
    for code in (0, -1, -2, -3, 7):
        s = _lib.vif_strerror(code)
        assert isinstance(s, str) and s
    assert "invalid" in _lib.vif_strerror(-1)
    assert "alloc" in _lib.vif_strerror(-2)


def test_fault_injection_alloc(lib):
    """VIF_FAULT_INJECT=alloc makes vif_create fail with VIF_ENOMEM before
    any allocation (a host-side path, no GPU needed)."""
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from vif_image_fidelity_amd import _lib\n"
            "c = _lib.vif_create(64, 64, 8)\n"
            "print(bool(c), _lib.vif_errno())\n" % ROOT)
    env = dict(os.environ, VIF_FAULT_INJECT="alloc")
    r = subprocess.run([sys.executable, "-c", code], env=env,
                       capture_output=True, text=True, check=True)
    assert r.stdout.split() == ["False", "-2"]


def test_binding_constants_match_headers():
    """The Python binding's constants are the headers' #defines."""
    import re
    from vif_image_fidelity_amd import _lib
    defs = {}
    for fn in ("vif.h", "fssim.h"):
        text = open(os.path.join(ROOT, "include", fn)).read()
        for m in re.finditer(r"#define\s+(\w+)\s+\(?(\d+)L?(?:\s*<<\s*(\d+))?\)?",
                             text):
            v = int(m.group(2))
            if m.group(3):
                v <<= int(m.group(3))
            defs[m.group(1)] = v
    pairs = {"VIF_QUEUE_DEPTH": _lib.QUEUE_DEPTH,
             "VIF_MAX_BATCH": _lib.MAX_BATCH,
             "VIF_MIN_SIDE": _lib.MIN_SIDE,
             "VIF_MAX_PIXELS": _lib.MAX_PIXELS,
             "FSSIM_TAPS": _lib.FSSIM_TAPS,
             "FSSIM_QUEUE_DEPTH": _lib.FSSIM_QUEUE_DEPTH,
             "FSSIM_MAX_BATCH": _lib.MAX_BATCH,
             "FSSIM_MAX_PIXELS": _lib.FSSIM_MAX_PIXELS,
             "FSSIM_MAX_FACTOR": _lib.FSSIM_MAX_FACTOR}
    for name, value in pairs.items():
        assert defs[name] == value, name


def test_package_import_needs_no_gpu():
    import vif_image_fidelity_amd as V
    assert V.VIF_OK == 0
    assert len(V.KERNEL_KINDS) == 4
    assert V.QUEUE_DEPTH == 3
    assert len(V.DEBUG_NAMES) == 15 and V.DEBUG_NAMES[4] == "vif"


def test_one_hip_runtime_in_the_process():
    """Loading the library before anything imports torch still leaves one
    HIP runtime mapped: torch bundles its own copy under the same soname,
    and two copies in one process make torch's device pointers and streams
    invalid in the library's calls."""
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from vif_image_fidelity_amd import _lib\n"
            "_lib.load()\n"
            "import torch\n"
            "p = {l.split()[-1] for l in open('/proc/self/maps')"
            " if 'libamdhip64' in l}\n"
            "print(len(p), sorted(p))\n" % ROOT)
    ensure_built()
    r = subprocess.run([sys.executable, "-c", code], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("1 "), r.stdout


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    from vif_image_fidelity_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load()


def test_fssim_taps_equal_oracle_taps(lib, orc):
    """The library's SSIM window taps and the oracle's, written separately,
    agree bit for bit and are symmetric bit for bit (the kernel reads
    t[min(k, 10-k)])."""
    import vif_image_fidelity_amd as V
    a = V.fssim_taps()
    assert a.tobytes() == orc.fssim_taps().tobytes()
    assert a.tobytes() == a[::-1].copy().tobytes()


@pytest.mark.parametrize("w,h,bpc", [(0, 5, 8), (5, 0, 8), (-1, 5, 8),
                                     (16, 16, 9), (16, 16, 7), (16, 16, 0),
                                     (1 << 14, 1 << 14, 8)])
def test_fssim_create_rejects_bad_arguments(lib, w, h, bpc):
    from vif_image_fidelity_amd import _lib
    assert not _lib.fssim_create(w, h, bpc)
    assert _lib.vif_errno() == _lib.VIF_EINVAL


def test_fssim_null_context_calls(lib):
    from vif_image_fidelity_amd import _lib
    out = np.zeros(2)
    assert _lib.fssim_score(None, None, None, out) == _lib.VIF_EINVAL
    assert _lib.fssim_collect(None, out) == _lib.VIF_EINVAL
    assert _lib.fssim_pending(None) == _lib.VIF_EINVAL
    assert _lib.fssim_geometry(None, np.zeros(3, np.int32)) == _lib.VIF_EINVAL
    _lib.fssim_destroy(None)


@pytest.mark.parametrize("mb", [0, -1, 17, 1000])
def test_create_batch_rejects_bad_capacity(lib, mb):
    """A batch capacity outside 1..VIF_MAX_BATCH is refused at create time,
    before any device call."""
    from vif_image_fidelity_amd import _lib
    assert not _lib.vif_create_batch(64, 64, 8, None, mb)
    assert _lib.vif_errno() == _lib.VIF_EINVAL


def test_submit_batch_null_context(lib):
    from vif_image_fidelity_amd import _lib
    assert _lib.vif_submit_batch(None, [0], [0]) == _lib.VIF_EINVAL


@pytest.mark.parametrize("mb", [0, 17])
def test_fssim_create_batch_rejects_bad_capacity(lib, mb):
    from vif_image_fidelity_amd import _lib
    assert not _lib.fssim_create_batch(64, 64, 8, mb)
    assert _lib.vif_errno() == _lib.VIF_EINVAL
