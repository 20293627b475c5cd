"""The scale-0 kernel's input staging on its own (GPU): the load-only probe
that calibrates the HBM counters for that kernel's access shape
(vif_selftest_stage_loads) stages each tile with the scale kernel's own code
and stores the sum of the raw samples it loaded.  Those sums must equal the
host's sums over the tile's 32 rows x 128 columns with the kernels' edge rule
(one reflection about the edge sample, then a clamp; ADR-1444 "float_vif_hip
runs the arithmetic of the CUDA twin ...", Decision), for the 8-samples-per-
load path and the one-sample path, ragged and tiny planes, 8- and 16-bit
samples and batches of frames."""
import ctypes
import os
import sys

import numpy as np
import pytest

from libutil import ensure_built

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import bench  # noqa: E402  (the host model of the probe lives with its mode)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    L = ensure_built()
    assert torch.cuda.is_available()
    return L


def _planes(g, w, h, bpc, n):
    hi = (1 << bpc) - 1
    dt = np.uint8 if bpc == 8 else np.uint16
    return [(g.integers(0, hi + 1, (h, w)).astype(dt),
             g.integers(0, hi + 1, (h, w)).astype(dt)) for _ in range(n)]


def _dev(a, shift):
    """Device copy of plane a starting `shift` bytes into its allocation."""
    import torch
    flat = np.ascontiguousarray(a).reshape(-1).view(np.uint8)
    buf = torch.zeros(flat.size + 64, dtype=torch.uint8, device="cuda:0")
    buf[shift:shift + flat.size].copy_(torch.from_numpy(flat))
    return buf, buf.data_ptr() + shift


@pytest.mark.parametrize("w,h,bpc,n,shift", [
    (304, 70, 8, 2, 0),      # interior tiles 8 samples per load
    (304, 70, 8, 1, 1),      # misaligned planes: one sample per load
    (300, 70, 8, 1, 0),      # width not a multiple of 8
    (16, 16, 8, 1, 0),       # smallest frame: mirror and clamp everywhere
    (232, 33, 10, 3, 0),     # 16-bit containers, ragged last strip
    (72, 1200, 12, 1, 2),    # tall, 16-bit misaligned by one sample
    (1000, 40, 16, 4, 0),
])
def test_probe_reads_the_tiles(lib, w, h, bpc, n, shift):
    import torch
    from vif_image_fidelity_amd import _lib
    g = np.random.default_rng(w * h + bpc + n + shift)
    frames = _planes(g, w, h, bpc, n)
    keep, refs, dists = [], [], []
    for r, d in frames:
        br, pr = _dev(r, shift)
        bd, pd = _dev(d, shift)
        keep += [br, bd]
        refs.append(pr)
        dists.append(pd)
    strips, ntx = -(-h // 16), -(-w // 112)
    out = torch.full((n * strips * ntx,), -1, dtype=torch.int32,
                     device="cuda:0")
    rc = lib.vif_selftest_stage_loads((ctypes.c_void_p * n)(*refs),
                                      (ctypes.c_void_p * n)(*dists), n, w, h,
                                      bpc, out.data_ptr(), None)
    assert rc == _lib.VIF_OK
    got = out.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, bench.stage_tile_sums(frames, w, h))


def test_probe_rejects_bad_arguments(lib):
    import torch
    from vif_image_fidelity_amd import _lib
    buf = torch.zeros(64 * 64, dtype=torch.uint8, device="cuda:0")
    out = torch.zeros(64, dtype=torch.int32, device="cuda:0")
    p = (ctypes.c_void_p * 1)(buf.data_ptr())
    nul = (ctypes.c_void_p * 1)(None)
    for args in ((p, p, 0, 64, 64, 8), (p, p, 17, 64, 64, 8),
                 (p, p, 1, 15, 64, 8), (p, p, 1, 64, 64, 9),
                 (nul, p, 1, 64, 64, 8), (p, nul, 1, 64, 64, 8)):
        assert lib.vif_selftest_stage_loads(*args, out.data_ptr(), None) == \
            _lib.VIF_EINVAL
    assert lib.vif_selftest_stage_loads(p, p, 1, 64, 64, 8, None, None) == \
        _lib.VIF_EINVAL
