"""Full-pipeline parity (GPU): the HIP path through the C ABI against the CPU
oracle on the same seeded frames, bit for bit: every output of every frame
(out[0..7]), the eight per-scale fp32 sums and every per-row fp32 sum.  The
largest absolute difference is always computed and anything above the
pages' 5e-5 gate fails on its own (Research-2130, Findings; ADR-1444,
Context), before the 0-ULP assertion.

Workloads: the five synthetic stand-ins of vif_image_fidelity_amd.synth,
plus edge geometries (16x16, ragged tiles, tall and wide frames, odd sizes)
and bit-depth invariance.  The 3840x2160 workload runs its first two frames
in full in the launch configuration the benchmark times.
"""
import json
import os
import sys

import numpy as np
import pytest

from libutil import ensure_built, to_device

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
FACTS = json.load(open(os.path.join(HERE, "golden", "page_facts.json")))
GATE = FACTS["parity_gate"]["value"]


@pytest.fixture(scope="module")
def V():
    import torch
    ensure_built()
    assert torch.cuda.is_available()
    import vif_image_fidelity_amd as V
    return V


_ctx_cache = {}


def _ctx(V, w, h, bpc):
    key = (w, h, bpc)
    if key not in _ctx_cache:
        _ctx_cache[key] = V.Vif(w, h, bpc)
    return _ctx_cache[key]


def _compare(V, orc, ref, dist, bpc, label, ctx=None):
    h, w = ref.shape
    print("parity case %s %dx%d bpc %d" % (label, w, h, bpc), flush=True)
    if ctx is None:
        ctx = _ctx(V, w, h, bpc)
    got = ctx.score(to_device(ref), to_device(dist))
    gsums = ctx.sums()
    grows = ctx.row_sums()
    exp, esums, erows = orc.score(ref, dist, bpc, want_rows=True)
    maxdiff = float(np.max(np.abs(got - exp)))
    print("  max|diff| = %.3g" % maxdiff, flush=True)
    assert maxdiff <= GATE, (label, maxdiff)
    assert got.view(np.uint64).tolist() == exp.view(np.uint64).tolist(), \
        (label, got, exp)
    assert gsums.view(np.uint32).tolist() == esums.view(np.uint32).tolist()
    bad = np.nonzero(grows.view(np.uint32) != erows.view(np.uint32))
    assert bad[0].size == 0, (label, bad[0][:10])
    return got


@pytest.mark.parametrize("name", ["netflix_576x324_8bit", "tiny_frames_8bit",
                                  "checker_1080p_10bit",
                                  "bright_1080p_16bit"])
def test_workload_parity(V, orc, name):
    from vif_image_fidelity_amd import synth
    for i, (ref, dist, bpc) in enumerate(synth.WORKLOADS[name]()):
        _compare(V, orc, ref, dist, bpc, "%s[%d]" % (name, i))


def test_4k_parity_first_frames(V, orc):
    from vif_image_fidelity_amd import synth
    for i in range(2):
        ref, dist, bpc = synth.pink_4k_frame(i)
        _compare(V, orc, ref, dist, bpc, "pink_4k_8bit[%d]" % i)


EDGE_SHAPES = [(16, 16), (17, 16), (16, 17), (112, 16), (113, 17), (224, 32),
               (225, 33), (16, 300), (300, 16), (71, 71), (72, 72), (73, 41),
               (129, 97), (1000, 37), (37, 1000), (3841, 33)]


def _noisy8(seed, w, h, spread=20):
    g = np.random.Generator(np.random.PCG64(seed))
    ref = g.integers(0, 256, size=(h, w)).astype(np.uint8)
    dist = np.clip(ref.astype(np.int16) +
                   g.integers(-spread, spread + 1, size=(h, w), dtype=np.int16),
                   0, 255).astype(np.uint8)
    return ref, dist


@pytest.mark.parametrize("wh", [(16, 1048704), (1048704, 16), (7400000, 16)])
def test_extreme_aspect_frames(V, orc, wh):
    """A frame 16 pixels wide has 65 544 strips of 16 rows at scale 0, all in
    grid x (strips of every frame).  Its transpose has 9364 tiles in a row.
    7 400 000 x 16 has 66 072 tiles in a row at scale 0, more than a grid's
    y dimension allows (65 535): scale 0 takes two launches, and each row's
    sum is handed from the first launch's last tile to the second launch's
    first."""
    w, h = wh
    ref, dist = _noisy8(w + 3 * h, w, h)
    ctx = V.Vif(w, h, 8)
    _compare(V, orc, ref, dist, 8, "extreme aspect", ctx=ctx)
    ctx.close()


def test_max_pixels_parity(V, orc):
    """The largest frame a context accepts: 2^27 pixels (16384 x 8192)."""
    w, h = 16384, 8192
    assert w * h == V.MAX_PIXELS
    ref, dist = _noisy8(27, w, h)
    ctx = V.Vif(w, h, 8)
    _compare(V, orc, ref, dist, 8, "max pixels", ctx=ctx)
    ctx.close()


OPTION_SETS = [
    {"sigma_nsq": 4.7},
    {"sigma_nsq": 1.5, "enhn_gain_limit": 1.0},
    {"sigma_nsq": 0.5, "enhn_gain_limit": 0.25},
    {"sigma_nsq": 0.0},
    {"enhn_gain_limit": 0.0},
    {"skip_scale0": 1},
    {"scale_min_val": (0.999, 0.5, 2.0)},
    {"sigma_nsq": 4.7, "enhn_gain_limit": 1.2, "skip_scale0": 1,
     "scale_min_val": (0.9, 0.0, 1.5)},
]


@pytest.mark.parametrize("opt", OPTION_SETS,
                         ids=["o%d" % i for i in range(len(OPTION_SETS))])
def test_options_parity(V, orc, opt):
    """Every option of struct vif_options against the oracle's reading of
    it, bit for bit (out[8], sums, rows, and the fifteen debug values), on
    the 576x324 8-bit workload's first frame, a bright 16-bit frame and a
    ragged 8-bit frame with a flat region (zero variances, where nsq = 0
    divides by zero)."""
    from vif_image_fidelity_amd import synth
    ref0, dist0, bpc0 = synth.WORKLOADS["netflix_576x324_8bit"]()[0]
    g = np.random.Generator(np.random.PCG64(77))
    wide = g.integers(40000, 65536, size=(70, 130)).astype(np.uint16)
    wdist = np.clip(wide.astype(np.int64) + g.integers(-3000, 3000,
                                                       size=wide.shape),
                    0, 65535).astype(np.uint16)
    flat = g.integers(0, 256, size=(61, 203)).astype(np.uint8)
    flat[10:50, 20:120] = 77
    fdist = flat.copy()
    fdist[:, 150:] = np.clip(fdist[:, 150:].astype(int) + 9, 0, 255)
    for ref, dist, bpc, label in ((ref0, dist0, bpc0, "netflix"),
                                  (wide, wdist, 16, "bright16"),
                                  (flat, fdist, 8, "flat")):
        h, w = ref.shape
        print("options case %s %s" % (label, opt), flush=True)
        with V.Vif(w, h, bpc, options=opt) as ctx:
            got = ctx.score(to_device(ref), to_device(dist))
            gsums, grows, gdbg = ctx.sums(), ctx.row_sums(), ctx.debug()
            back = ctx.options()
        exp, esums, erows = orc.score(ref, dist, bpc, want_rows=True,
                                      options=opt)
        assert got.view(np.uint64).tolist() == exp.view(np.uint64).tolist(), \
            (label, got, exp)
        assert gsums.view(np.uint32).tolist() == esums.view(np.uint32).tolist()
        assert np.array_equal(grows.view(np.uint32), erows.view(np.uint32))
        want = list(exp[:4]) + [exp[6], exp[4], exp[5]] + \
            [float(v) for v in esums]
        assert [gdbg[k] for k in V.DEBUG_NAMES] == want
        for k, v in opt.items():
            assert back[k] == (tuple(v) if k == "scale_min_val" else v)


@pytest.mark.parametrize("opt", [{"kernelscale": 2.0}, {"sigma_nsq": -1.0},
                                 {"enhn_gain_limit": float("nan")},
                                 {"skip_scale0": 3}])
def test_bad_options_refused(V, opt):
    with pytest.raises(V.VifError):
        V.Vif(64, 64, 8, options=opt)


@pytest.mark.parametrize("wh", EDGE_SHAPES)
def test_edge_geometry_parity(V, orc, wh):
    w, h = wh
    g = np.random.Generator(np.random.PCG64(w * 7919 + h))
    ref = g.integers(0, 256, size=(h, w)).astype(np.uint8)
    dist = np.clip(ref.astype(np.int64) + g.integers(-25, 26, size=(h, w)),
                   0, 255).astype(np.uint8)
    _compare(V, orc, ref, dist, 8, "edge")


@pytest.mark.parametrize("bpc", [10, 12, 16])
def test_wide_samples_parity_and_invariance(V, orc, bpc):
    """Random wide samples at parity; and a frame whose codes are 4/16/256
    times an 8-bit frame's scores bit-identically to the 8-bit frame."""
    g = np.random.Generator(np.random.PCG64(bpc))
    h, w = 90, 150
    top = (1 << bpc) - 1
    ref = g.integers(0, top + 1, size=(h, w)).astype(np.uint16)
    dist = np.clip(ref.astype(np.int64) + g.integers(-top // 20, top // 20,
                                                      size=(h, w)),
                   0, top).astype(np.uint16)
    _compare(V, orc, ref, dist, bpc, "wide%d" % bpc)
    r8 = g.integers(0, 256, size=(h, w)).astype(np.uint8)
    d8 = np.clip(r8.astype(np.int64) + g.integers(-9, 10, size=(h, w)), 0,
                 255).astype(np.uint8)
    mul = 1 << (bpc - 8)
    a = _compare(V, orc, r8, d8, 8, "inv8")
    b = _compare(V, orc, (r8.astype(np.uint32) * mul).astype(np.uint16),
                 (d8.astype(np.uint32) * mul).astype(np.uint16), bpc,
                 "inv%d" % bpc)
    assert a.tobytes() == b.tobytes()


def _offset_view(t, k):
    """The frame t copied into a larger buffer k samples from its start."""
    import torch
    flat = torch.zeros(t.numel() + 16, dtype=t.dtype, device=t.device)
    flat[k:k + t.numel()] = t.reshape(-1)
    return flat[k:k + t.numel()].view(t.shape)


@pytest.mark.parametrize("bpc", [8, 16])
def test_input_load_paths(V, orc, bpc):
    """Scale 0 loads interior tiles 8 samples at a time when the width is a
    multiple of 8 and the planes are aligned to 8 samples, and one sample at
    a time otherwise (edge tiles, other widths, planes at any other offset).
    Every combination scores bit for bit as the oracle: width 360 (tiles 1
    and 2 interior) with aligned planes and with planes one sample off, width
    364, and a batch whose second frame is off."""
    g = np.random.Generator(np.random.PCG64(360 + bpc))
    top = (1 << bpc) - 1
    dt = np.uint8 if bpc == 8 else np.uint16
    for w in (360, 364):
        h = 100
        ref = g.integers(0, top + 1, size=(h, w)).astype(dt)
        dist = np.clip(ref.astype(np.int64) +
                       g.integers(-(top // 10), top // 10 + 1, size=(h, w)),
                       0, top).astype(dt)
        exp = orc.score(ref, dist, bpc)[0]
        ctx = V.Vif(w, h, bpc, max_batch=2)
        dr, dd = to_device(ref), to_device(dist)
        for k in (0, 1, 3):
            print("load paths: bpc %d width %d offset %d" % (bpc, w, k),
                  flush=True)
            a = dr if k == 0 else _offset_view(dr, k)
            b = dd if k == 0 else _offset_view(dd, k)
            got = ctx.score(a, b)
            assert got.tobytes() == exp.tobytes(), (w, k)
        ro, do = _offset_view(dr, 1), _offset_view(dd, 1)
        ctx.submit_batch([dr, ro], [dd, do])
        assert ctx.collect().tobytes() == exp.tobytes()
        assert ctx.collect().tobytes() == exp.tobytes()
        ctx.close()


def _random_pair(g, w, h, bpc):
    """One seeded pair of a randomly chosen kind: noise, smooth, a flat
    region, or a gradient; the distorted frame noisy or blurred."""
    top = (1 << bpc) - 1
    kind = int(g.integers(0, 4))
    if kind == 0:
        ref = g.integers(0, top + 1, size=(h, w))
    elif kind == 1:
        base = g.integers(0, top + 1, size=(h + 4, w + 4)).astype(np.float64)
        ref = np.rint(sum(base[i:i + h, j:j + w] for i in range(5)
                          for j in range(5)) / 25.0)
    elif kind == 2:
        ref = g.integers(0, top + 1, size=(h, w))
        ref[h // 4:3 * h // 4, w // 4:3 * w // 4] = top // 3
    else:
        ref = np.rint(np.linspace(0, top, w)[None, :] +
                      g.normal(0, top / 50.0, size=(h, w)))
    ref = np.clip(ref, 0, top)
    if g.integers(0, 2):
        dist = ref + np.rint(g.normal(0, top * g.uniform(0.005, 0.1),
                                      size=(h, w)))
    else:
        pad = np.pad(ref.astype(np.float64), 1, mode="edge")
        dist = np.rint(sum(pad[i:i + h, j:j + w] for i in range(3)
                           for j in range(3)) / 9.0)
    dt = np.uint8 if bpc == 8 else np.uint16
    return (ref.astype(dt), np.clip(dist, 0, top).astype(dt))


def test_random_sweep(V, orc):
    """A seeded sweep of 40 random cases: frame sizes 16..499 x 16..399,
    bit depths 8/10/12/16, frame content, options (a third of the cases)
    and submissions of 1 to 3 frames; every output and every per-scale sum
    bit for bit as the oracle, and the row sums of each submission's last
    frame."""
    g = np.random.Generator(np.random.PCG64(2026))
    for case in range(40):
        w = int(g.integers(16, 500))
        h = int(g.integers(16, 400))
        bpc = int(g.choice([8, 10, 12, 16]))
        n = int(g.integers(1, 4))
        opt = None
        if g.uniform() < 1 / 3:
            opt = {"sigma_nsq": float(g.choice([0.5, 1.5, 2.0, 3.0, 4.7])),
                   "enhn_gain_limit": float(g.choice([0.5, 1.0, 100.0])),
                   "skip_scale0": int(g.integers(0, 2)),
                   "scale_min_val": tuple(float(v) for v in
                                          g.choice([0.0, 0.5, 0.99], 3))}
        pairs = [_random_pair(g, w, h, bpc) for _ in range(n)]
        print("sweep case %d: %dx%d bpc %d, %d frame(s), options %s"
              % (case, w, h, bpc, n, opt), flush=True)
        with V.Vif(w, h, bpc, options=opt, max_batch=n) as ctx:
            dev = [(to_device(r), to_device(d)) for r, d in pairs]
            ctx.submit_batch([a for a, _ in dev], [b for _, b in dev])
            for i, (r, d) in enumerate(pairs):
                got = ctx.collect()
                exp, esums, erows = orc.score(r, d, bpc, want_rows=True,
                                              options=opt)
                assert got.view(np.uint64).tolist() == \
                    exp.view(np.uint64).tolist(), (case, i, got, exp)
                assert ctx.sums().view(np.uint32).tolist() == \
                    esums.view(np.uint32).tolist(), (case, i)
            grows = ctx.row_sums()
            assert (grows.view(np.uint32) == erows.view(np.uint32)).all(), \
                case


def test_flat_and_identical_frames(V, orc):
    f = np.full((64, 80), 200, np.uint8)
    out = _compare(V, orc, f, f, 8, "flat")
    assert np.all(out[:4] == 1.0) and out[6] == 1.0
    assert out[4] == out[5] == 80 * 64 + 40 * 32 + 20 * 16 + 10 * 8
    g = np.random.Generator(np.random.PCG64(9))
    r = g.integers(0, 256, size=(64, 80)).astype(np.uint8)
    out = _compare(V, orc, r, r, 8, "self")
    assert abs(out[4] - out[5]) <= 1e-6 * out[5]


def test_repeat_is_deterministic_and_stream_aware(V, orc):
    import torch
    from vif_image_fidelity_amd import synth
    ref, dist, bpc = synth.netflix_576x324_8bit(frames=1)[0]
    ctx = V.Vif(576, 324, 8)
    dr, dd = to_device(ref), to_device(dist)
    a = ctx.score(dr, dd)
    s = torch.cuda.Stream()
    ctx.set_stream(s)
    b = ctx.score(dr, dd)
    ctx.set_stream(None)
    c = ctx.score(dr, dd)
    assert a.tobytes() == b.tobytes() == c.tobytes()
    ctx.close()


def test_async_queue_matches_oracle(V, orc):
    """submit/collect with the queue full, frames collected in order."""
    from vif_image_fidelity_amd import synth
    frames = synth.netflix_576x324_8bit(frames=3) * 3
    exps = [orc.score(r, d, b)[0] for (r, d, b) in frames[:3]]
    dev = [(to_device(r), to_device(d)) for (r, d, _) in frames]
    ctx = V.Vif(576, 324, 8)
    outs = []
    for i, (r, d) in enumerate(dev):
        if ctx.pending() == V.QUEUE_DEPTH:
            outs.append(ctx.collect())
        ctx.submit(r, d)
    assert ctx.pending() == V.QUEUE_DEPTH
    with pytest.raises(V.VifError):
        ctx.submit(*dev[0])      # the queue is full
    with pytest.raises(V.VifError):
        ctx.score(*dev[0])       # frames are pending
    while ctx.pending():
        outs.append(ctx.collect())
    with pytest.raises(V.VifError):
        ctx.collect()            # nothing pending
    assert len(outs) == len(frames)
    for i, o in enumerate(outs):
        assert o.tobytes() == exps[i % 3].tobytes(), i
    ctx.close()


def test_queue_holds_temporary_frames(V, orc):
    """Frames passed to submit() as temporaries (no other reference) stay
    alive until their collect(): the binding holds them, so the caching
    allocator cannot hand their memory to the tensors allocated and filled
    in between while the kernels read it."""
    import torch
    from vif_image_fidelity_amd import synth
    frames = synth.netflix_576x324_8bit(frames=3)
    exps = [orc.score(r, d, b)[0] for (r, d, b) in frames]
    ctx = V.Vif(576, 324, 8)
    order = [0, 1, 2, 2, 1, 0, 1]
    outs = []
    for i in order:
        if ctx.pending() == V.QUEUE_DEPTH:
            outs.append(ctx.collect())
        r, d, _ = frames[i]
        ctx.submit(to_device(r), to_device(d))
        assert len(ctx._inflight) == ctx.pending()
        junk = [torch.full(r.shape, 255, dtype=torch.uint8, device="cuda:0")
                for _ in range(4)]
        del junk
    while ctx.pending():
        outs.append(ctx.collect())
    assert len(ctx._inflight) == 0
    for i, got in zip(order, outs):
        assert got.tobytes() == exps[i].tobytes(), i
    ctx.close()


def test_contexts_in_two_threads(V, orc):
    """Separate contexts are independent: two host threads, each with its
    own context (one 576x324, one 1920x1080 10-bit), score their frames
    through full queues at the same time (ctypes releases the interpreter
    lock during library calls), and every output matches the oracle."""
    import threading
    from vif_image_fidelity_amd import synth
    work = {"small": synth.netflix_576x324_8bit(frames=3),
            "1080p": synth.checker_1080p_10bit(frames=2)}
    want = {k: [orc.score(r, d, b)[0] for (r, d, b) in fr]
            for k, fr in work.items()}
    dev = {k: [(to_device(r), to_device(d)) for (r, d, _) in fr]
           for k, fr in work.items()}
    got = {}
    errors = []

    def run(key):
        try:
            r0 = work[key][0][0]
            ctx = V.Vif(r0.shape[1], r0.shape[0], work[key][0][2])
            outs = []
            order = list(range(len(dev[key]))) * 6
            for i in order:
                if ctx.pending() == V.QUEUE_DEPTH:
                    outs.append(ctx.collect())
                ctx.submit(*dev[key][i])
            while ctx.pending():
                outs.append(ctx.collect())
            ctx.close()
            got[key] = (order, outs)
        except Exception as e:  # reported below, in the main thread
            errors.append((key, repr(e)))

    threads = [threading.Thread(target=run, args=(k,)) for k in work]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert sorted(got) == sorted(work), "a thread did not finish"
    for key, (order, outs) in got.items():
        assert len(outs) == len(order)
        for i, out in zip(order, outs):
            assert out.tobytes() == want[key][i].tobytes(), (key, i)


def test_timed_and_untimed_launches_interleave(V, orc):
    """Frames submitted with and without kernel timing (the timed ones
    record HIP events around each launch) interleave over changing frames,
    with host synchronisation between rounds: every frame must give the
    oracle's bits whichever way it was launched."""
    from vif_image_fidelity_amd import synth
    frames = synth.netflix_576x324_8bit(frames=3)
    exps = [orc.score(r, d, b)[0] for (r, d, b) in frames]
    dev = [(to_device(r), to_device(d)) for (r, d, _) in frames]
    ctx = V.Vif(576, 324, 8)
    for rnd in range(4):
        ctx.set_profiling(0xF if rnd % 2 else 0)
        for i in range(7):
            k = (i * 2 + rnd) % 3
            got = ctx.score(*dev[k])
            assert got.tobytes() == exps[k].tobytes(), (rnd, i)
        for i in range(6):
            k = (i + rnd) % 3
            if ctx.pending() == V.QUEUE_DEPTH:
                ctx.collect()
            ctx.submit(*dev[k])
        while ctx.pending():
            ctx.collect()
    ctx.close()


def test_profiling_counts_launches(V):
    from vif_image_fidelity_amd import synth
    ref, dist, bpc = synth.netflix_576x324_8bit(frames=1)[0]
    ctx = V.Vif(576, 324, 8)
    ctx.set_profiling(True)
    dr, dd = to_device(ref), to_device(dist)
    for _ in range(3):
        ctx.score(dr, dd)
    kt = ctx.kernel_times()
    for kind in V.KERNEL_KINDS:
        ms, n = kt[kind]
        assert n == 3 and ms > 0, kind
    ctx.close()


def test_score_rejects_misaligned_wide_pointer(V):
    import torch
    ctx = V.Vif(64, 64, 10)
    buf = torch.zeros(64 * 64 * 2 + 2, dtype=torch.uint8, device="cuda:0")
    from vif_image_fidelity_amd import _lib
    out = np.zeros(8)
    p = buf.data_ptr() + 1
    assert _lib.vif_score(ctx._ctx, p, p, out) == _lib.VIF_EINVAL
    ctx.close()


def test_host_frames_match_device_frames(V, orc):
    """Frames in host memory (pageable numpy arrays and pinned tensors) go
    through the per-slot upload and score bit for bit as the same frames in
    device memory; the queue keeps order over more frames than slots, and a
    host buffer refilled after its frame was collected is scored anew."""
    import torch
    from vif_image_fidelity_amd import synth
    frames = synth.WORKLOADS["netflix_576x324_8bit"]()
    h, w = frames[0][0].shape
    ctx = _ctx(V, w, h, 8)
    want = [orc.score(r, d, 8)[0] for r, d, _ in frames]
    print("host frames: pageable", flush=True)
    for (r, d, _), exp in zip(frames, want):
        got = ctx.score_host(r, d)
        assert got.tobytes() == exp.tobytes()
    print("host frames: pinned queue", flush=True)
    pinned = []
    for r, d, _ in frames:
        pr = torch.empty((h, w), dtype=torch.uint8, pin_memory=True)
        pd = torch.empty((h, w), dtype=torch.uint8, pin_memory=True)
        pr.numpy()[:] = r
        pd.numpy()[:] = d
        pinned.append((pr, pd))
    order = [0, 1, 2, 1, 0, 2, 2]
    outs = []
    for k, i in enumerate(order):
        if ctx.pending() == V.QUEUE_DEPTH:
            outs.append(ctx.collect())
        ctx.submit_host(*pinned[i])
    while ctx.pending():
        outs.append(ctx.collect())
    for i, got in zip(order, outs):
        assert got.tobytes() == want[i].tobytes(), i
    # refill a host buffer once nothing is pending and score it again
    pinned[0][1].numpy()[:] = frames[1][1]
    got = ctx.score_host(*pinned[0])
    exp = orc.score(frames[0][0], frames[1][1], 8)[0]
    assert got.tobytes() == exp.tobytes()
    with pytest.raises(ValueError):
        ctx.score_host(frames[0][0][:, :-1], frames[0][1][:, :-1])
    with pytest.raises(ValueError):
        ctx.score_host(frames[0][0].astype(np.uint16), frames[0][1])


def _check_outputs(got, exp, label):
    maxdiff = float(np.max(np.abs(got - exp)))
    assert maxdiff <= GATE, (label, maxdiff)
    assert got.view(np.uint64).tolist() == exp.view(np.uint64).tolist(), \
        (label, got, exp)


@pytest.mark.parametrize("name,n", [("netflix_576x324_8bit", 16),
                                    ("checker_1080p_10bit", 3),
                                    ("bright_1080p_16bit", 5)])
def test_batch_matches_oracle(V, orc, name, n):
    """One submission of n frames (each kernel launched once for all of
    them): every frame's outputs, sums and row sums equal the oracle's."""
    from vif_image_fidelity_amd import synth
    frames = synth.WORKLOADS[name]()
    h, w = frames[0][0].shape
    bpc = frames[0][2]
    print("batch case %s n=%d" % (name, n), flush=True)
    exps = {}
    for k, (r, d, b) in enumerate(frames):
        exps[k] = orc.score(r, d, b, want_rows=True)
    dev = [(to_device(r), to_device(d)) for r, d, _ in frames]
    ctx = V.Vif(w, h, bpc, max_batch=n)
    idx = [(3 * i + 1) % len(frames) for i in range(n)]
    ctx.submit_batch([dev[k][0] for k in idx], [dev[k][1] for k in idx])
    assert ctx.pending() == n
    for i, k in enumerate(idx):
        got = ctx.collect()
        exp, esums, erows = exps[k]
        _check_outputs(got, exp, "%s[%d]" % (name, i))
        assert ctx.sums().view(np.uint32).tolist() == \
            esums.view(np.uint32).tolist()
        assert (ctx.row_sums().view(np.uint32) ==
                erows.view(np.uint32)).all()
    assert ctx.pending() == 0
    ctx.close()


def test_batch_4k_bench_configuration(V, orc):
    """The benchmark's launch configuration: four 3840x2160 frames of the 1/f
    workload in one submission (every kernel launched once for them)."""
    from vif_image_fidelity_amd import synth
    frames = [synth.pink_4k_frame(i) for i in range(4)]
    ctx = V.Vif(3840, 2160, 8, max_batch=4)
    dev = [(to_device(r), to_device(d)) for r, d, _ in frames]
    ctx.submit_batch([a for a, _ in dev], [b for _, b in dev])
    for i, (r, d, b) in enumerate(frames):
        got = ctx.collect()
        _check_outputs(got, orc.score(r, d, b)[0], "pink_4k_8bit[%d]" % i)
    ctx.close()


def test_4k_ordered_stream_paths(V, orc):
    """At 3840x2160 one scale-0 kernel fills the GPU twice over, so
    consecutive submissions' scale-0 kernels are ordered: each slot's stream
    waits for the previous slot's scale-0 event.  Every way in is checked on
    that path: a full queue of device frames with every kernel timed, a
    queue of pinned host frames (copied on the slot's own stream ahead of
    its kernels), and frames written on the caller's stream just before the
    submit, behind other work on that stream."""
    import torch
    from vif_image_fidelity_amd import synth
    frames = [synth.pink_4k_frame(i) for i in range(2)]
    want = [orc.score(r, d, b)[0] for r, d, b in frames]
    dev = [(to_device(r), to_device(d)) for r, d, _ in frames]
    ctx = V.Vif(3840, 2160, 8)
    print("ordered paths: device queue, profiling on", flush=True)
    ctx.set_profiling(True)
    order = [0, 1, 0, 1, 1, 0]
    outs = []
    for i in order:
        if ctx.pending() == V.QUEUE_DEPTH:
            outs.append(ctx.collect())
        ctx.submit(*dev[i])
    while ctx.pending():
        outs.append(ctx.collect())
    for i, got in zip(order, outs):
        assert got.tobytes() == want[i].tobytes(), i
    kt = ctx.kernel_times()
    for kind in V.KERNEL_KINDS:
        ms, n = kt[kind]
        assert n == len(order) and ms > 0, kind
    ctx.set_profiling(False)
    print("ordered paths: pinned host queue", flush=True)
    pinned = []
    for r, d, _ in frames:
        pr = torch.empty(r.shape, dtype=torch.uint8, pin_memory=True)
        pd = torch.empty(d.shape, dtype=torch.uint8, pin_memory=True)
        pr.numpy()[:] = r
        pd.numpy()[:] = d
        pinned.append((pr, pd))
    outs = []
    for i in order:
        if ctx.pending() == V.QUEUE_DEPTH:
            outs.append(ctx.collect())
        ctx.submit_host(*pinned[i])
    while ctx.pending():
        outs.append(ctx.collect())
    for i, got in zip(order, outs):
        assert got.tobytes() == want[i].tobytes(), i
    print("ordered paths: frames written on the caller's stream", flush=True)
    s = torch.cuda.Stream()
    a = torch.ones(2048, 2048, device="cuda:0")
    for k in range(2):
        src = dev[k]
        dr = dev[1 - k][0].clone()
        dd = dev[1 - k][1].clone()
        torch.cuda.synchronize()
        ctx.set_stream(s)
        with torch.cuda.stream(s):
            for _ in range(8):
                a = torch.mm(a, a) * (1.0 / 2048)
            dr.copy_(src[0])
            dd.copy_(src[1])
        ctx.submit(dr, dd)
        got = ctx.collect()
        ctx.set_stream(None)
        assert got.tobytes() == want[k].tobytes(), k
    torch.cuda.synchronize()
    ctx.close()


def test_batch_tiny_frames(V, orc):
    """Every tiny geometry in batches of two and of one."""
    from vif_image_fidelity_amd import synth
    frames = synth.tiny_frames_8bit()
    by_size = {}
    for r, d, b in frames:
        by_size.setdefault(r.shape, []).append((r, d, b))
    for shape, fr in by_size.items():
        h, w = shape
        ctx = V.Vif(w, h, 8, max_batch=2)
        dev = [(to_device(r), to_device(d)) for r, d, _ in fr]
        ctx.submit_batch([a for a, _ in dev], [b for _, b in dev])
        ctx.submit(*dev[1])
        for i, (r, d, b) in enumerate(fr + [fr[1]]):
            got = ctx.collect()
            _check_outputs(got, orc.score(r, d, b)[0],
                           "tiny %dx%d[%d]" % (w, h, i))
        ctx.close()


def test_batch_mixed_queue_and_limits(V, orc):
    """Batches and single frames share the three slots: a fourth submission
    is refused until a slot's frames are all collected; order is kept."""
    from vif_image_fidelity_amd import synth
    frames = synth.netflix_576x324_8bit()
    exps = [orc.score(r, d, b)[0] for r, d, b in frames]
    dev = [(to_device(r), to_device(d)) for r, d, _ in frames]
    ctx = V.Vif(576, 324, 8, max_batch=4)
    order = []
    ctx.submit_batch([dev[0][0], dev[1][0], dev[2][0]],
                     [dev[0][1], dev[1][1], dev[2][1]])
    order += [0, 1, 2]
    ctx.submit(*dev[2])
    order += [2]
    ctx.submit_batch([dev[1][0]] * 4, [dev[1][1]] * 4)
    order += [1] * 4
    assert ctx.pending() == 8
    with pytest.raises(V.VifError):
        ctx.submit(*dev[0])          # all three slots in use
    with pytest.raises(V.VifError):
        ctx.submit_batch([dev[0][0]] * 5, [dev[0][1]] * 5)  # above capacity
    for i in range(3):
        assert ctx.collect().tobytes() == exps[order[i]].tobytes()
    # the first slot is free again
    ctx.submit_batch([dev[0][0]], [dev[0][1]])
    order += [0]
    for i in range(3, len(order)):
        assert ctx.collect().tobytes() == exps[order[i]].tobytes(), i
    assert ctx.pending() == 0
    ctx.close()


def test_batch_with_options(V, orc):
    """Non-default noise variance and gain limit through a batched
    submission."""
    from vif_image_fidelity_amd import synth
    frames = synth.netflix_576x324_8bit()
    opt = {"sigma_nsq": 1.5, "enhn_gain_limit": 1.0}
    ctx = V.Vif(576, 324, 8, options=opt, max_batch=3)
    dev = [(to_device(r), to_device(d)) for r, d, _ in frames]
    ctx.submit_batch([a for a, _ in dev], [b for _, b in dev])
    for i, (r, d, b) in enumerate(frames):
        got = ctx.collect()
        _check_outputs(got, orc.score(r, d, b, options=opt)[0],
                       "options[%d]" % i)
    ctx.close()


def test_batch_profiling_counts_one_launch_per_kind(V):
    from vif_image_fidelity_amd import synth
    frames = synth.netflix_576x324_8bit()
    dev = [(to_device(r), to_device(d)) for r, d, _ in frames]
    ctx = V.Vif(576, 324, 8, max_batch=3)
    ctx.set_profiling(0xF)
    for _ in range(2):
        ctx.submit_batch([a for a, _ in dev], [b for _, b in dev])
        for _ in dev:
            ctx.collect()
    t = ctx.kernel_times()
    assert [t[k][1] for k in V.KERNEL_KINDS] == [2] * 4
    ctx.close()


def test_4k_every_frame_bench_configuration(V, orc):
    """Every frame of the 3840x2160 1/f workload (20 pairs), as the benchmark
    scores them: submissions of four frames (each kernel launched once for
    the four) through the full three-slot queue.  Every frame's out[8], its
    eight sums and all 4050 row sums equal the oracle's bit for bit
    (ADR-1422, Consequences: every output of every frame equals the CPU's).
    The oracle runs in threads (its C calls release the interpreter)."""
    from concurrent.futures import ThreadPoolExecutor
    from vif_image_fidelity_amd import synth
    frames = synth.pink_4k_8bit(frames=20)
    print("oracle on 20 frames of pink_4k_8bit", flush=True)
    with ThreadPoolExecutor(max_workers=8) as ex:
        exps = list(ex.map(lambda f: orc.score(f[0], f[1], f[2],
                                               want_rows=True), frames))
    dev = [(to_device(r), to_device(d)) for r, d, _ in frames]
    ctx = V.Vif(3840, 2160, 8, max_batch=4)
    nxt = 0
    for k in range(len(frames)):
        while nxt < len(frames) and ctx.pending() + 4 <= 4 * V.QUEUE_DEPTH:
            sel = dev[nxt:nxt + 4]
            ctx.submit_batch([a for a, _ in sel], [b for _, b in sel])
            nxt += 4
        got = ctx.collect()
        exp, esums, erows = exps[k]
        print("pink_4k_8bit[%d] collected" % k, flush=True)
        _check_outputs(got, exp, "pink_4k_8bit[%d]" % k)
        assert ctx.sums().view(np.uint32).tolist() == \
            esums.view(np.uint32).tolist(), k
        bad = np.nonzero(ctx.row_sums().view(np.uint32) !=
                         erows.view(np.uint32))
        assert bad[0].size == 0, (k, bad[0][:10])
    assert ctx.pending() == 0
    ctx.close()
