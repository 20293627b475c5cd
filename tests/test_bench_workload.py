"""Facts about the benchmark's workload that its operation count relies on
(CPU only, the oracle's own filter and decimation): on the 3840x2160 1/f
frames every scale-0 pixel takes the statistic's high-variance branch
(sigma1_sq >= 2 compared in fp64), so the scale-0 kernel performs the
statistic's operations for every pixel and the roofline counts them per
pixel; at scales 1-3 at least 99.9% of the pixels do."""
import numpy as np
import pytest


@pytest.mark.parametrize("index", [0, 7])
def test_every_pixel_takes_the_high_branch(orc, index):
    from vif_image_fidelity_amd import synth
    r, _, _ = synth.pink_4k_frame(index)
    x = orc.normalise(r, 8)
    for s in range(4):
        t = orc.taps(s)
        if s > 0:
            x = orc.decimate(x, t)
        mu = orc.filter2d(x, t)
        xx = orc.filter2d((x * x).astype(np.float32), t)
        s1 = np.maximum((xx - (mu * mu).astype(np.float32))
                        .astype(np.float32), np.float32(0))
        high = np.mean(s1.astype(np.float64) >= 2.0)
        if s == 0:
            assert high == 1.0, (index, s, high)
        else:
            assert high >= 0.999, (index, s, high)


def test_kernel_hash_ignores_comments_only():
    """The traffic record stays valid across comment edits of the kernel
    sources and becomes invalid with any code edit."""
    import bench
    src = "int f(int a) {  // one\n  /* two\n lines */ return a + 1;\n}\n"
    same = "// header\nint f(int a) {  // changed\n  return a + 1;\n}\n"
    other = "int f(int a) {\n  return a + 2;\n}\n"
    assert bench._code_only(src) == bench._code_only(same)
    assert bench._code_only(src) != bench._code_only(other)
