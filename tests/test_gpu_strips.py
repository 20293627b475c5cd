"""Row strips on the GPU (the one-device share of a frame split by rows):
each strip context scores its strip's input rows, and the strips' own row
sums, concatenated scale by scale, equal the whole frame's row sums bit for
bit -- those of a whole-frame context and the oracle's -- and give the
oracle's out[8] and sums through vif_scores_from_rows.  The host adds the
rows top to bottom after the concatenation, as for a whole frame (ADR-1422
"float_vif_sycl computes the CPU's arithmetic ...", Decision); the strip's
kernels mirror only at the frame's edges (ADR-1444 "float_vif_hip runs the
arithmetic of the CUDA twin ...", Decision).
"""
import numpy as np
import pytest

from libutil import ensure_built, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def V():
    import torch
    ensure_built()
    assert torch.cuda.is_available()
    import vif_image_fidelity_amd as V
    return V


def _tiling(h, step):
    b = list(range(0, h, step)) + [h]
    return list(zip(b[:-1], b[1:]))


def _split(rows, h):
    """Whole-frame row sums (scale after scale) as a list per scale."""
    out, base = [], 0
    for s in range(4):
        out.append(rows[base:base + (h >> s)])
        base += h >> s
    return out


def _score_strips(V, ref_d, dist_d, w, h, bpc, tiling, options=None,
                  host=None):
    """Scores every strip of one frame with its own context; returns the
    concatenated own rows (scale by scale) and each strip's out[8]."""
    per_scale = [[] for _ in range(4)]
    outs = []
    for row0, row1 in tiling:
        ctx = V.Vif(w, h, bpc, options=options, strip=(row0, row1))
        a, b = ctx.in0, ctx.in0 + ctx.in_rows
        if host is None:
            out = ctx.score(ref_d[a:b], dist_d[a:b])
        else:
            out = ctx.score_host(np.ascontiguousarray(host[0][a:b]),
                                 np.ascontiguousarray(host[1][a:b]))
        rows = ctx.row_sums()
        g = V.strip_geometry(w, h, row0, row1)
        base = 0
        for s in range(4):
            n = g["own_rows"][s]
            per_scale[s].append(rows[base:base + n])
            base += n
        assert base == rows.shape[0]
        outs.append(out)
        ctx.close()
    return np.concatenate([np.concatenate(p) for p in per_scale]), outs


def _check_frame(V, orc, ref, dist, bpc, tiling, label, options=None,
                 host=False):
    h, w = ref.shape
    print("strip case %s %dx%d bpc %d, %d strips" % (label, w, h, bpc,
                                                     len(tiling)), flush=True)
    out, sums, rows = orc.score(ref, dist, bpc, want_rows=True,
                                options=options)
    rd, dd = to_device(ref), to_device(dist)
    cat, _ = _score_strips(V, rd, dd, w, h, bpc, tiling, options,
                           host=(ref, dist) if host else None)
    bad = np.nonzero(cat.view(np.uint32) != rows.view(np.uint32))
    assert bad[0].size == 0, (label, bad[0][:10])
    got, gsums = V.scores_from_rows(w, h, cat, options)
    assert float(np.max(np.abs(got - out))) <= 5e-5, label
    assert got.tobytes() == out.tobytes(), (label, got, out)
    assert gsums.tobytes() == sums.tobytes(), label
    # the whole-frame context returns the same rows
    whole = V.Vif(w, h, bpc, options=options)
    whole.score(rd, dd)
    assert whole.row_sums().tobytes() == cat.tobytes(), label
    whole.close()


def test_4k_frames_in_eight_strips(V, orc):
    """3840x2160, the 1/f workload: eight strips on 272-row boundaries
    (strip boundaries fall on multiples of 8 rows; the last strip has
    256)."""
    from vif_image_fidelity_amd import synth
    for i in range(2):
        ref, dist, bpc = synth.pink_4k_frame(i)
        _check_frame(V, orc, ref, dist, bpc, _tiling(2160, 272),
                     "pink_4k_8bit[%d]" % i)


def test_1080p_10bit_frames_in_eight_strips(V, orc):
    from vif_image_fidelity_amd import synth
    for i, (ref, dist, bpc) in enumerate(synth.checker_1080p_10bit()):
        _check_frame(V, orc, ref, dist, bpc, _tiling(1080, 136),
                     "checker_1080p_10bit[%d]" % i)


def _noisy(seed, w, h, bpc):
    g = np.random.Generator(np.random.PCG64(seed))
    top = 256 if bpc == 8 else 1 << bpc
    dt = np.uint8 if bpc == 8 else np.uint16
    ref = g.integers(0, top, size=(h, w)).astype(dt)
    dist = np.clip(ref.astype(np.int64) +
                   g.integers(-top // 10, top // 10 + 1, size=(h, w)),
                   0, top - 1).astype(dt)
    return ref, dist


@pytest.mark.parametrize("w,h,bpc,step", [
    (64, 300, 8, 40), (40, 203, 8, 16), (73, 91, 10, 24),
    (96, 1083, 12, 136), (48, 160, 16, 8), (3841, 33, 8, 16),
    (16, 16, 8, 8)])
def test_ragged_strips(V, orc, w, h, bpc, step):
    """Heights that are not multiples of 8 (the last strip ends at the
    frame's bottom), a last strip of 3 rows with no rows of its own at scale
    3, strips of one 8-row block, a wide frame and the smallest one."""
    ref, dist = _noisy(w + 3 * h, w, h, bpc)
    _check_frame(V, orc, ref, dist, bpc, _tiling(h, step),
                 "ragged %dx%d" % (w, h))


def test_strips_with_options_and_host_frames(V, orc):
    ref, dist = _noisy(9, 200, 120, 8)
    opts = {"sigma_nsq": 4.7, "enhn_gain_limit": 0.8, "skip_scale0": 1,
            "scale_min_val": (0.5, 0.0, 0.99)}
    _check_frame(V, orc, ref, dist, 8, _tiling(120, 32), "options",
                 options=opts)
    _check_frame(V, orc, ref, dist, 8, _tiling(120, 48), "host frames",
                 host=True)


def test_strip_batch_in_the_queue(V, orc):
    """One share at its real shape, as a device holding it would run it:
    the strip [272, 544) of 3840x2160 frames (309 input rows) for four
    frames per submission, several submissions through the queue.  Each
    frame's own rows equal the oracle's rows of the whole frame."""
    from vif_image_fidelity_amd import synth
    frames = [synth.pink_4k_frame(i) for i in range(6)]
    want = [_split(orc.score(r, d, b, want_rows=True)[2], 2160)
            for r, d, b in frames]
    ctx = V.Vif(3840, 2160, 8, max_batch=4, strip=(272, 544))
    assert (ctx.in0, ctx.in_rows) == (248, 309)
    g = V.strip_geometry(3840, 2160, 272, 544)
    a, b = ctx.in0, ctx.in0 + ctx.in_rows
    dev = [(to_device(r)[a:b], to_device(d)[a:b]) for r, d, _ in frames]
    order = [0, 1, 2, 3, 4, 5, 2, 0, 1, 3, 5, 4]
    for k in range(0, len(order), 4):
        sel = [dev[i] for i in order[k:k + 4]]
        ctx.submit_batch([x for x, _ in sel], [y for _, y in sel])
    for k, i in enumerate(order):
        ctx.collect()
        rows = ctx.row_sums()
        base = 0
        for s in range(4):
            n = g["own_rows"][s]
            o = g["own0"][s]
            assert rows[base:base + n].tobytes() == \
                want[i][s][o:o + n].tobytes(), (k, i, s)
            base += n
    ctx.close()


def test_strip_frame_shape_checked(V):
    ctx = V.Vif(256, 256, 8, strip=(64, 128))
    import torch
    wrong = torch.zeros((256, 256), dtype=torch.uint8, device="cuda:0")
    with pytest.raises(ValueError):
        ctx.score(wrong, wrong)
    ctx.close()
