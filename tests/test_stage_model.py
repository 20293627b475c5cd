"""The host model of the staging probe (CPU): the tile sums it expects and
the lines each XCD must fetch, against brute force on small cases."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402


def _mc(i, n):
    m = abs(i)
    m = 2 * (n - 1) - m if m > n - 1 else m
    return min(max(m, 0), n - 1)


@pytest.mark.parametrize("w,h", [(300, 70), (16, 16), (113, 17)])
def test_tile_sums_brute_force(w, h):
    g = np.random.default_rng(w + h)
    pairs = [(g.integers(0, 65536, (h, w)).astype(np.uint16),
              g.integers(0, 65536, (h, w)).astype(np.uint16))
             for _ in range(2)]
    strips, ntx = -(-h // 16), -(-w // 112)
    want = []
    for c in range(ntx):
        for ref, dist in pairs:
            for r in range(strips):
                t = 0
                for j in range(32):
                    yy = _mc(16 * r - 8 + j, h)
                    for k in range(128):
                        xx = _mc(112 * c - 8 + k, w)
                        t += int(ref[yy, xx]) + int(dist[yy, xx])
                want.append(t & 0xFFFFFFFF)
    assert np.array_equal(bench.stage_tile_sums(pairs, w, h),
                          np.array(want, dtype=np.uint32))


@pytest.mark.parametrize("w,h,n,bps,shift", [(300, 70, 3, 1, 0),
                                             (232, 100, 5, 2, 7),
                                             (16, 16, 1, 1, 0)])
def test_fetch_lines_brute_force(w, h, n, bps, shift):
    """Distinct (XCD, 128-byte line) pairs over every byte every block
    reads, block by block, against the vectorised model."""
    ptrs = [(1 << 30) + z * (1 << 24) + shift for z in range(2 * n)]
    pairs = [(ptrs[2 * z], ptrs[2 * z + 1]) for z in range(n)]
    strips, ntx = -(-h // 16), -(-w // 112)
    slots = n * strips
    gx = (slots + 7) & ~7
    seen = set()
    for x in range(gx):
        sp = (x % 8) * (gx // 8) + x // 8
        if sp >= slots:
            continue
        z, r = divmod(sp, strips)
        for c in range(ntx):
            for base in pairs[z]:
                for j in range(32):
                    yy = _mc(16 * r - 8 + j, h)
                    for k in range(128):
                        xx = _mc(112 * c - 8 + k, w)
                        a = base + (yy * w + xx) * bps
                        for b in range(bps):
                            seen.add((x % 8, (a + b) >> 7))
    fetch, planes = bench.stage_probe_fetch_bytes(pairs, w, h, bps)
    assert fetch == 128 * len(seen)
    assert planes == 2 * n * w * h * bps
