"""Seeded synthetic luma frame pairs shaped like the pages' fixtures.

The pages measure on the Netflix 576x324 pair (8 to 16 bits), two 1920x1080
checkerboard pairs and Big Buck Bunny at 3840x2160 (ADR-1422, Consequences;
Research-1434, Sources).  Those files are not available here, so each
workload below is a seeded stand-in with the same shape, bit depth and value
structure.  This module holds no VIF arithmetic: it only draws pixels.  Both
the GPU path and the CPU oracle are fed from it.

Conventions: numpy ``Generator(PCG64(seed))``; rounding is ``np.rint`` (half
to even); box means pad by whole-sample reflection (``np.pad`` mode
"reflect"); every plane is (h, w), row-major, uint8 for 8-bit, uint16
holding the low ``bpc`` bits otherwise.

Workloads (name -> list of frames, each ``(ref, dist, bpc)``):
  netflix_576x324_8bit     576x324 8-bit, 3 frames, seed 0
  tiny_frames_8bit         40x40, 56x56, 64x64, 71x71, 73x41, 2 frames each,
                           seed 2
  checker_1080p_10bit      1920x1080 10-bit checkerboard, 1 px shift, seed 3
  bright_1080p_16bit       1920x1080 16-bit bright gradient, seed 4
  pink_4k_8bit             3840x2160 8-bit 1/f noise, seed = frame index

For the float SSIM decimation, whose factor max(1, round(min(w, h) / 256))
depends only on the frame size, ``noisy_pair`` draws one pair of any size
and bit depth (uniform reference, noisy distorted frame), so that every
factor 1..10 and odd sizes can be exercised.
"""
import numpy as np


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _box_mean(plane, k):
    """k x k box mean with whole-sample reflection, float64 result."""
    p = k // 2
    a = np.pad(plane.astype(np.float64), p, mode="reflect")
    h, w = plane.shape
    out = np.zeros((h, w), dtype=np.float64)
    for dy in range(k):
        for dx in range(k):
            out += a[dy:dy + h, dx:dx + w]
    return out / (k * k)


def netflix_576x324_8bit(frames=3, seed=0):
    """Ref: uniform integers on [16, 235], 5x5 box mean, rint.
    Dist: ref + N(0, 6^2), rint, clipped to [0, 255]."""
    g = _rng(seed)
    h, w = 324, 576
    out = []
    for _ in range(frames):
        raw = g.integers(16, 236, size=(h, w))
        ref = np.rint(_box_mean(raw, 5)).astype(np.uint8)
        noisy = ref.astype(np.float64) + g.normal(0.0, 6.0, size=(h, w))
        dist = np.clip(np.rint(noisy), 0, 255).astype(np.uint8)
        out.append((ref, dist, 8))
    return out


TINY_SIZES = ((40, 40), (56, 56), (64, 64), (71, 71), (73, 41))  # (w, h)


def tiny_frames_8bit(frames_each=2, seed=2, sizes=TINY_SIZES):
    """Ref: uniform integers on [0, 255].  Dist: 3x3 box mean of ref, rint."""
    g = _rng(seed)
    out = []
    for (w, h) in sizes:
        for _ in range(frames_each):
            ref = g.integers(0, 256, size=(h, w)).astype(np.uint8)
            dist = np.clip(np.rint(_box_mean(ref, 3)), 0, 255).astype(np.uint8)
            out.append((ref, dist, 8))
    return out


def checker_pattern(h, w, shift=0, square=10, lo=64, hi=940):
    """c(y, x) = lo if (floor((x - shift)/square) + floor(y/square)) even."""
    y = np.arange(h)[:, None]
    x = np.arange(w)[None, :] - shift
    par = (np.floor_divide(x, square) + np.floor_divide(y, square)) % 2
    return np.where(par == 0, lo, hi).astype(np.int64)


def checker_1080p_10bit(frames=3, seed=3, h=1080, w=1920):
    """Ref: 10 px squares alternating 64 / 940.  Dist: the pattern shifted
    1 px right (c(y, x - 1), extended to x = -1) + N(0, 2^2), rint, clipped to
    [0, 1023]."""
    g = _rng(seed)
    ref = checker_pattern(h, w).astype(np.uint16)
    shifted = checker_pattern(h, w, shift=1).astype(np.float64)
    out = []
    for _ in range(frames):
        noisy = shifted + g.normal(0.0, 2.0, size=(h, w))
        dist = np.clip(np.rint(noisy), 0, 1023).astype(np.uint16)
        out.append((ref.copy(), dist, 10))
    return out


def bright_1080p_16bit(frames=3, seed=4, h=1080, w=1920):
    """Ref: rint(49152 + 16383 x / (w-1)) + N(0, 300^2), rint, clipped to
    [0, 65535].  Dist: 3x3 box mean of ref, then 64 rint(v / 64), clipped."""
    g = _rng(seed)
    ramp = np.rint(49152.0 + 16383.0 * np.arange(w) / (w - 1))
    out = []
    for _ in range(frames):
        noisy = ramp[None, :] + g.normal(0.0, 300.0, size=(h, w))
        ref = np.clip(np.rint(noisy), 0, 65535).astype(np.uint16)
        blur = _box_mean(ref, 3)
        dist = np.clip(64.0 * np.rint(blur / 64.0), 0, 65535).astype(np.uint16)
        out.append((ref, dist, 16))
    return out


def _pink_plane(g, h, w, mean=128.0, sd=40.0):
    white = g.normal(0.0, 1.0, size=(h, w))
    spec = np.fft.rfft2(white)
    fy = np.fft.fftfreq(h)[:, None]
    fx = np.fft.rfftfreq(w)[None, :]
    f = np.sqrt(fy * fy + fx * fx)
    amp = np.zeros_like(f)
    nz = f > 0
    amp[nz] = 1.0 / f[nz]
    img = np.fft.irfft2(spec * amp, s=(h, w))
    img = (img - img.mean()) / img.std()
    return np.clip(np.rint(mean + sd * img), 0, 255)


def _bilinear_up2(small, h, w):
    """2x bilinear upscale with half-pixel centres and edge clamping."""
    sh, sw = small.shape
    ys = (np.arange(h) + 0.5) / 2.0 - 0.5
    xs = (np.arange(w) + 0.5) / 2.0 - 0.5
    y0 = np.floor(ys).astype(np.int64)
    x0 = np.floor(xs).astype(np.int64)
    wy = (ys - y0)[:, None]
    wx = (xs - x0)[None, :]
    y0c = np.clip(y0, 0, sh - 1)
    y1c = np.clip(y0 + 1, 0, sh - 1)
    x0c = np.clip(x0, 0, sw - 1)
    x1c = np.clip(x0 + 1, 0, sw - 1)
    a = small[y0c][:, x0c]
    b = small[y0c][:, x1c]
    c = small[y1c][:, x0c]
    d = small[y1c][:, x1c]
    top = a * (1.0 - wx) + b * wx
    bot = c * (1.0 - wx) + d * wx
    return top * (1.0 - wy) + bot * wy


def pink_4k_frame(index, h=2160, w=3840):
    """One 1/f-noise frame pair; the seed is the frame index."""
    g = _rng(index)
    ref = _pink_plane(g, h, w)
    small = ref.reshape(h // 2, 2, w // 2, 2).mean(axis=(1, 3))
    up = _bilinear_up2(small, h, w)
    dist = np.clip(np.rint(up), 0, 255)
    return (np.ascontiguousarray(ref, dtype=np.uint8),
            np.ascontiguousarray(dist, dtype=np.uint8), 8)


def pink_4k_8bit(frames=20, first=0, h=2160, w=3840):
    """Ref: white N(0,1) -> rfft2 -> amplitude x 1/|f| (DC zeroed) -> irfft2
    -> standardised to mean 128, sd 40 -> rint, clipped.  Dist: 2x2 box-mean
    downscale, bilinear 2x upscale, rint, clipped."""
    return [pink_4k_frame(first + i, h, w) for i in range(frames)]


def noisy_pair(w, h, bpc, seed, sd_frac=0.05):
    """Ref: uniform integers on [0, 2^bpc - 1].  Dist: ref + N(0, (sd_frac *
    2^bpc)^2), rint, clipped to the bit depth's range."""
    g = _rng(seed)
    top = (1 << bpc) - 1
    dt = np.uint8 if bpc == 8 else np.uint16
    ref = g.integers(0, top + 1, size=(h, w))
    noisy = ref.astype(np.float64) + g.normal(0.0, sd_frac * (top + 1),
                                               size=(h, w))
    dist = np.clip(np.rint(noisy), 0, top)
    return ref.astype(dt), dist.astype(dt), bpc


WORKLOADS = {
    "netflix_576x324_8bit": netflix_576x324_8bit,
    "tiny_frames_8bit": tiny_frames_8bit,
    "checker_1080p_10bit": checker_1080p_10bit,
    "bright_1080p_16bit": bright_1080p_16bit,
    "pink_4k_8bit": pink_4k_8bit,
}
