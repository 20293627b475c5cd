"""Throughput of the float VIF feature on one MI355X.

  python bench.py [--gpus 1] [--steps K] [--warmup W]

One step scores one batch of --batch (default 4) 3840x2160 8-bit luma frame
pairs: the whole path (four scales of filtering, statistic, decimation and
ordered row sums, the read-back and the host sums) with each kernel launched
once for the batch (vif_submit_batch).  The 20 synthetic 1/f-noise frame
pairs are resident in HBM before the timed region; steps cycle through them
and go through the context's asynchronous queue (up to three batches in
flight), so consecutive batches overlap their read-back and host work with
the next batch's kernels.  `value` is frames/s.  Prints one JSON line.

The line carries, besides the contract fields:
  roofline      the dominant kernel (the scale-0 filter/statistic kernel, one
                launch per batch): algorithmic operations per launch (fp32
                and fp64, each IEEE operation once) / its average duration,
                timed with HIP events on the slot's stream during the timed
                region, against the VALU peak for plain operations;
                `traffic` is the kernel's HBM bytes per launch from committed
                rocprofv3 counters taken at the same batch size, when the
                kernel source and flags have not changed since, else null.
  cpu_baseline  the CPU oracle on this host, one core, on a bounded sample of
                the same workload.
  extra         1920x1080 and 576x324 frames/s, the rates with batched
                submissions (vif_submit_batch: one launch per kernel for 4, 8
                or 16 frames), the 4K rate when the frames
                come from pinned host memory (PCIe copies included, never the
                headline value), HBM GB/s of the whole frame from counters
                when available, and the per-kernel split; under "fssim" the
                float SSIM feature on the same 4K frames and on the 1080p
                10-bit frames: frames/s, the decimation kernel's HBM
                roofline (algorithmic bytes: both sample planes read once,
                both decimated fp32 planes written once) and the CPU
                oracle's rate.
"""
import argparse
import collections
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("VIF frames/sec at 1080p and 4K on 1 MI355X; achieved HBM GB/s vs "
          "peak")

# Algorithmic operations of the scale-0 kernel per scale-0 pixel, counted
# from the definition: every IEEE operation once (separate multiply and add,
# no fused multiply-add, no packing; fp64 operations and conversions count
# as one like fp32 ones).
#   filter: 3 products + 5 quantities x 2 passes x (17 mul + 16 add) + 8 for
#     the variances (3 mul, 3 sub, 2 clamps) = 341;
#   the next scale's 9-tap low-pass of both planes at even rows (two columns
#     per decimated pixel) and even columns: 2 planes x 3 x (9 mul + 8 add)
#     = 102 per scale-1 pixel = 25.5 per scale-0 pixel;
#   the statistic of a pixel in the high-variance branch = 78: fp64
#     conversion and comparison of sigma1_sq (2); g = sigma12 / sigma1_sq,
#     g * sigma12, sv_sq (3); the comparisons with eps and 0, the floor at
#     eps and the gain limit (4) with their four selects (4); g * g and
#     a = g*g * sigma1_sq (2); the numerator ratio: two conversions, the sum
#     with nsq, the quotient, the sum with 1, the conversion to fp32 (6); the
#     denominator ratio: quotient, sum, conversion (3); two log2
#     polynomials of 27 each (exponent field, bias, mantissa bits, t = m - 1,
#     9 Horner steps of multiply and add, the last product, the exponent's
#     conversion and the final sum).
# On the benchmark's frames every scale-0 pixel takes that branch
# (tests/test_bench_workload.py), so the statistic counts for every pixel.
FILTER_OPS_PER_PIXEL_SCALE0 = 341.0 + 102.0 / 4.0
STAT_OPS_PER_PIXEL = 78.0
OPS_PER_PIXEL_SCALE0 = FILTER_OPS_PER_PIXEL_SCALE0 + STAT_OPS_PER_PIXEL

# VALU peak for plain (unfused, unpacked) fp32 operations.  MI355X's fp32
# vector figure, 157.3 TFLOP/s, is 256 CUs x 4 SIMDs x 32 lanes x 2 flops (an
# FMA) x 2.4 GHz: a SIMD retires two wave64 VALU instructions per four
# cycles.  Unpacked code reaches that rate too, by dual issue (the SIMD
# issues VALU instructions of two waves in one quad-cycle; rocprofv3's
# SQ_ACTIVE_INST_VALU2 counts those quad-cycles, and the scale-0 kernel
# retires more wave instructions than one per quad-cycle per SIMD allows).
# A plain add or multiply is one operation, so the ceiling is
# 256 x 4 x 32 x 2.4e9 = 78.6e12 operations/s.
VALU_CLOCK_HZ = 2.4e9
VALU_PEAK_OPS = 256 * 4 * 32 * VALU_CLOCK_HZ

HBM_PEAK_GBS = 8000.0

# The pages' parity gate: an output further than this from the CPU's fails
# (ADR-1422 and ADR-1444, Context).  Bit identity is reported beside it.
PARITY_GATE = 5e-5

# The other workloads of frames mode: generator in synth, w, h, bpc.
SMALL_WORKLOADS = {"1080p10": ("checker_1080p_10bit", 1920, 1080, 10),
                   "1080p16": ("bright_1080p_16bit", 1920, 1080, 16),
                   "576x324": ("netflix_576x324_8bit", 576, 324, 8)}

# One device's share when 3840x2160 frames are split in eight row strips on
# 272-row boundaries (strip boundaries fall on multiples of 8 rows): rows
# 272..543, read with their halo as input rows 248..556.
STRIP_SHARE = (272, 544)

PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic_scale0_4k.json")
PROFILE_TRAFFIC_1080P = os.path.join(ROOT, "profiles", "traffic_1080p_10bit.json")


def _code_only(text):
    """C++ source without its comments and blank lines, each line's
    whitespace runs collapsed (comments and layout do not change the
    machine code)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(" ".join(ln.split()) for ln in text.split("\n")
                     if ln.strip())


def kernel_source_hash():
    """SHA-256 of what the VIF kernels' machine code depends on: their
    sources (comments removed) and the compiler flags of the build."""
    from vif_image_fidelity_amd import build
    h = hashlib.sha256()
    for rel in ("vif_image_fidelity_amd/csrc/vif_kernels.hip",
                "vif_image_fidelity_amd/csrc/vif_device_math.h",
                "vif_image_fidelity_amd/csrc/vif_internal.h"):
        with open(os.path.join(ROOT, rel)) as f:
            h.update(_code_only(f.read()).encode())
    h.update(" ".join(build.FLAGS).encode())
    return h.hexdigest()


def load_traffic(batch, path=PROFILE_TRAFFIC):
    """Counter-derived HBM bytes per launch of the scale-0 kernel (a launch
    of `batch` frames) and per frame of the whole path, if taken on the
    current kernel source at that batch size."""
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None, None
    if (rec.get("kernel_source_sha256") != kernel_source_hash() or
            rec.get("batch") != batch):
        return None, None
    return rec.get("scale0_bytes_per_launch"), rec.get("frame_bytes")


def ensure_lib():
    from vif_image_fidelity_amd import _lib, build
    if not os.path.exists(_lib.LIB_PATH):
        build.build()
    _lib.load()


def _device_pairs(frames):
    import torch
    dev = torch.device("cuda:0")

    def td(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    pairs = [(td(r), td(d)) for (r, d, _) in frames]
    torch.cuda.synchronize()
    return pairs


def steady_state(V, frames, w, h, bpc, steps, warmup, batch=1, reps=5,
                 prof_kinds=0, settle_s=0.25, strip=None):
    """Scores the resident frames (cycling over them) through one context's
    queue, `batch` frames per submission (each kernel launched once for the
    batch), and times the queue in steady state.

    The queue is kept full throughout: a new submission goes in as soon as
    the oldest one's frames have been collected.  `warmup` submissions run
    first, untimed, and more after them until `settle_s` seconds have
    passed since the first (the device's clocks rise over the first tens of
    milliseconds of work after an idle spell; the number run is returned);
    the queue is then filled, if it is not yet.  Each
    of the `reps` timed repetitions then counts exactly `steps`
    submissions: t0 is taken with the queue full, each step collects the
    oldest submission (a collect waits for that submission's completion
    event on the device, so its work is finished) and submits the next, and
    t1 follows the last step's collect and submit.  The repetitions run back
    to back, and the queue is drained after the last, untimed.  So the
    region covers `steps` submission completions of a pipeline that neither
    fills nor drains inside it.

    strip: None, or (row0, row1): a strip context (vif_create_strip) fed
    the strip's input rows of each frame, one device's share of a frame
    split by rows.

    Returns {"seconds": [per repetition], "kernel": {kind: (ms, launches)}
    over the timed repetitions, "host_us": per-frame host time of submit and
    collect calls, "outputs": {frame index: set of out[8] byte strings},
    "warmup_run": warm-up submissions run}."""
    import torch
    from vif_image_fidelity_amd import _lib
    pairs = _device_pairs(frames)
    ctx = V.Vif(w, h, bpc, max_batch=batch, strip=strip)
    a, b = ctx.in0, ctx.in0 + ctx.in_rows
    pairs = [(r[a:b], d[a:b]) for r, d in pairs]
    ptrs = [(r.data_ptr(), d.data_ptr()) for r, d in pairs]
    ctx.set_profiling(prof_kinds)
    nf = len(ptrs)
    pending = collections.deque()  # frame index of every pending frame
    outputs = {}
    state = {"next": 0, "submit": 0.0, "collect": 0.0}
    clock = time.perf_counter

    def submit():
        idx = [(state["next"] + j) % nf for j in range(batch)]
        state["next"] = (state["next"] + batch) % nf
        c0 = clock()
        if batch == 1:
            rc = _lib.vif_submit(ctx._ctx, *ptrs[idx[0]])
        else:
            rc = _lib.vif_submit_batch(ctx._ctx, [ptrs[i][0] for i in idx],
                                       [ptrs[i][1] for i in idx])
        state["submit"] += clock() - c0
        if rc != 0:
            raise V.VifError(rc, "vif_submit_batch")
        pending.extend(idx)

    def collect():
        c0 = clock()
        got = [ctx.collect() for _ in range(batch)]
        state["collect"] += clock() - c0
        for out in got:
            outputs.setdefault(pending.popleft(), set()).add(out.tobytes())

    depth = V.QUEUE_DEPTH
    warm0 = clock()
    warm_run = 0
    while warm_run < warmup or clock() - warm0 < settle_s:
        if len(pending) == depth * batch:
            collect()
        submit()
        warm_run += 1
    while len(pending) < depth * batch:
        submit()
    k0 = ctx.kernel_times()
    state["submit"] = state["collect"] = 0.0
    seconds = []
    for _ in range(reps):
        t0 = clock()
        for _ in range(steps):
            collect()
            submit()
        seconds.append(clock() - t0)
    k1 = ctx.kernel_times()
    host = {"submit": 1e6 * state["submit"] / (reps * steps * batch),
            "collect": 1e6 * state["collect"] / (reps * steps * batch)}
    while pending:
        collect()
    torch.cuda.synchronize()
    ctx.close()
    kernel = {k: (k1[k][0] - k0[k][0], k1[k][1] - k0[k][1]) for k in k1}
    return {"seconds": seconds, "kernel": kernel, "host_us": host,
            "outputs": outputs, "warmup_run": warm_run}


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def rate(res, steps, batch):
    """Frames/s of the median repetition."""
    return steps * batch / median(res["seconds"])


def time_fssim(V, frames, w, h, bpc, steps, warmup, prof_kinds=0, batch=1):
    """The float SSIM queue over resident frames, timed in steady state as
    steady_state() times VIF: the queue is full at t0, and the region counts
    `steps` frames' completions (steps a multiple of `batch`).  Returns
    (seconds, kernel times, geometry)."""
    import torch
    pairs = _device_pairs(frames)
    ctx = V.FloatSsim(w, h, bpc, max_batch=batch)
    ctx.set_profiling(prof_kinds)
    state = {"next": 0}

    def submit():
        sel = [pairs[(state["next"] + j) % len(pairs)] for j in range(batch)]
        state["next"] += batch
        if batch == 1:
            ctx.submit(*sel[0])
        else:
            ctx.submit_batch([a for a, _ in sel], [b for _, b in sel])

    full = V.FSSIM_QUEUE_DEPTH * batch
    for _ in range(max(warmup // batch, 1)):
        if ctx.pending() == full:
            for _ in range(batch):
                ctx.collect()
        submit()
    while ctx.pending() < full:
        submit()
    k0 = ctx.kernel_times()
    t0 = time.perf_counter()
    for _ in range(max(steps // batch, 1)):
        for _ in range(batch):
            ctx.collect()
        submit()
    t1 = time.perf_counter()
    k1 = ctx.kernel_times()
    while ctx.pending():
        ctx.collect()
    torch.cuda.synchronize()
    geom = ctx.geometry()
    ctx.close()
    kt = {k: (k1[k][0] - k0[k][0], k1[k][1] - k0[k][1]) for k in k1}
    return (t1 - t0), kt, geom


def fssim_kernel_us(V, frames, w, h, bpc, n=300, batch=1):
    """Average kernel durations (HIP events on the slot's stream around each
    launch) with one submission of `batch` frames at a time, so that no other
    submission's kernels share the GPU during a timed launch."""
    import torch
    dev = torch.device("cuda:0")

    def td(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    pairs = [(td(r), td(d)) for (r, d, _) in frames[:4]]
    ctx = V.FloatSsim(w, h, bpc, max_batch=batch)

    def one(i):
        sel = [pairs[(i + j) % len(pairs)] for j in range(batch)]
        ctx.submit_batch([a for a, _ in sel], [b for _, b in sel])
        for _ in range(batch):
            ctx.collect()

    for i in range(10):
        one(i)
    ctx.set_profiling(0x7)
    for i in range(n):
        one(i)
    kt = ctx.kernel_times()
    ctx.close()
    return {k: 1000.0 * v[0] / max(v[1], 1) for k, v in kt.items()}


def fssim_leg(V, frames, w, h, bpc, steps, cpu_budget_s, batch=8):
    """frames/s of the float SSIM queue (no timing events), one frame and
    `batch` frames per submission; the kernels' average durations with one
    submission at a time; the decimation kernel against the HBM peak (per
    launch of one frame and of a batch); and the oracle on this host."""
    dt, _, (f, ow, oh) = time_fssim(V, frames, w, h, bpc, steps, 20)
    dtb, _, _ = time_fssim(V, frames, w, h, bpc, steps, 4 * batch,
                           batch=batch)
    avg = fssim_kernel_us(V, frames, w, h, bpc)
    avgb = fssim_kernel_us(V, frames, w, h, bpc, n=100, batch=batch)
    bps = 1 if bpc == 8 else 2
    dec_bytes = 2 * w * h * bps + 2 * ow * oh * 4
    rec = {"workload": "%dx%d %d-bit, factor %d -> %dx%d" % (w, h, bpc, f,
                                                             ow, oh),
           "fps": round(steps / dt, 1),
           "fps_batch%d" % batch: round(steps / dtb, 1),
           "kernel_avg_us": {k: round(v, 2) for k, v in avg.items()},
           "kernel_avg_us_batch%d" % batch: {k: round(v, 2)
                                             for k, v in avgb.items()}}
    if f > 1 and avg["decimate"] > 0:
        for key, us, nb in (("decimate_roofline", avg["decimate"], 1),
                            ("decimate_roofline_batch%d" % batch,
                             avgb["decimate"], batch)):
            gbs = nb * dec_bytes / (us * 1e-6) / 1e9
            rec[key] = {"bound": "hbm", "achieved": round(gbs, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "algorithmic_bytes": nb * dec_bytes}
    if cpu_budget_s > 0:
        import oracle
        n, t0 = 0, time.perf_counter()
        while True:
            r, d, b = frames[n % len(frames)]
            oracle.fssim_score(r, d, b)
            n += 1
            if time.perf_counter() - t0 >= cpu_budget_s:
                break
        rec["cpu_oracle"] = {"fps": round(n / (time.perf_counter() - t0), 2),
                             "cores": 1, "frames": n}
    return rec


def time_host_frames(V, frames, w, h, bpc, steps, warmup):
    """The queue fed from host memory: pinned host planes, each frame copied
    to the slot's device buffers by the library (vif_submit_host).  The
    rate includes the host-to-device copies over PCIe."""
    import torch
    dt = torch.uint8 if bpc == 8 else torch.int16
    pairs = []
    for r, d, _ in frames[:4]:
        pr = torch.empty((h, w), dtype=dt, pin_memory=True)
        pd = torch.empty((h, w), dtype=dt, pin_memory=True)
        pr.numpy().view(r.dtype)[:] = r
        pd.numpy().view(d.dtype)[:] = d
        pairs.append((pr, pd))
    ctx = V.Vif(w, h, bpc)

    def run(n):
        for i in range(n):
            if ctx.pending() == V.QUEUE_DEPTH:
                ctx.collect()
            ctx.submit_host(*pairs[i % len(pairs)])
        while ctx.pending():
            ctx.collect()

    run(warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ctx.close()
    return steps / (t1 - t0)


def isolated_scale0_us(V, frames, w, h, bpc, n=50):
    """Scale-0 kernel duration with one frame at a time (vif_score), i.e.
    without the next frame's kernels sharing the GPU."""
    import torch
    dev = torch.device("cuda:0")
    r, d, _ = frames[0]
    tr = torch.from_numpy(np.ascontiguousarray(r)).to(dev)
    tdd = torch.from_numpy(np.ascontiguousarray(d)).to(dev)
    ctx = V.Vif(w, h, bpc)
    for _ in range(5):
        ctx.score(tr, tdd)
    ctx.set_profiling(["scale0"])
    for _ in range(n):
        ctx.score(tr, tdd)
    ms, cnt = ctx.kernel_times()["scale0"]
    ctx.close()
    return 1000.0 * ms / max(cnt, 1)


def path_ops(w, h):
    """Algorithmic operations the definition needs per frame: per scale the
    3 products, 5 quantities x 2 passes x (N mul + N-1 add) and 8 for the
    variances per pixel, the statistic (STAT_OPS_PER_PIXEL, every pixel
    counted in the high-variance branch, which at least 99.9% of the
    benchmark's pixels take at every scale), the next scale's low-pass
    (2 planes x 3 x (2N'-1) per decimated pixel) and 2 row-sum adds per
    pixel."""
    widths = (17, 9, 5, 3)
    ops, ws, hs = 0.0, w, h
    for s in range(4):
        n = widths[s]
        ops += (3 + 10 * (2 * n - 1) + 8 + STAT_OPS_PER_PIXEL + 2) * ws * hs
        if s < 3:
            ops += 6 * (2 * widths[s + 1] - 1) * (ws // 2) * (hs // 2)
        ws, hs = ws // 2, hs // 2
    return ops


COPY_BYTES = 256 << 20


def copy_calibration(launches):
    """A plain device-to-device copy of COPY_BYTES, `launches` times: each
    launch reads and writes exactly COPY_BYTES, the reference against which
    the FETCH_SIZE and WRITE_SIZE counters are scaled."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(max(launches, 1)):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("copied %d x %d bytes" % (max(launches, 1), COPY_BYTES),
          file=sys.stderr, flush=True)


# The scale-0 kernel's tile: 16 x 112 output pixels, with a halo of its
# filter's radius (8) on every side.
STAGE_TILE_H, STAGE_TILE_W, STAGE_R = 16, 112, 8


def _mirror_clamp(i, n):
    """The kernels' edge rule: reflect about the edge sample once, then
    clamp into [0, n)."""
    m = np.abs(i)
    m = np.where(m > n - 1, 2 * (n - 1) - m, m)
    return np.clip(m, 0, n - 1)


def _stage_rows_cols(w, h):
    strips = -(-h // STAGE_TILE_H)
    ntx = -(-w // STAGE_TILE_W)
    rows = _mirror_clamp(STAGE_TILE_H * np.arange(strips)[:, None] - STAGE_R +
                         np.arange(STAGE_TILE_H + 2 * STAGE_R)[None, :], h)
    cols = _mirror_clamp(STAGE_TILE_W * np.arange(ntx)[:, None] - STAGE_R +
                         np.arange(STAGE_TILE_W + 2 * STAGE_R)[None, :], w)
    return strips, ntx, rows, cols


def stage_tile_sums(pairs, w, h):
    """What vif_selftest_stage_loads stores for the frame pairs `pairs`
    (host arrays): for tile column c, frame z and strip r, at
    [(c * n + z) * strips + r], the sum of the raw samples of the tile's 32
    mirrored rows x 128 mirrored columns of both planes, mod 2^32."""
    strips, ntx, rows, cols = _stage_rows_cols(w, h)
    out = np.zeros((ntx, len(pairs), strips), dtype=np.int64)
    for z, (ref, dist) in enumerate(pairs):
        for plane in (ref, dist):
            rs = plane.astype(np.int64)[rows].sum(axis=1)  # strips x w
            out[:, z, :] += rs[:, cols].sum(axis=2).T
    return (out.reshape(-1) & 0xFFFFFFFF).astype(np.uint32)


def stage_probe_fetch_bytes(ptr_pairs, w, h, bytes_per_sample):
    """HBM bytes one launch of the staging probe must fetch when every
    128-byte line reaches each XCD's L2 once: the launch's blocks go to XCDs
    round-robin (block x to XCD x % 8; the grid's x dimension is padded to a
    multiple of 8), block x takes slot (x % 8) * (gridDim.x / 8) + x / 8
    (frame z = slot / strips, strip slot % strips), and each block reads, in
    each of its 32 rows and each plane, the samples from its tile's first to
    its last (mirrored) column.  Returns (bytes summed over the XCDs' distinct
    lines, bytes of the planes themselves).  ptr_pairs: device addresses of
    the frames' planes."""
    n = len(ptr_pairs)
    strips, ntx, rows, cols = _stage_rows_cols(w, h)
    slots = n * strips
    per = ((slots + 7) & ~7) >> 3
    slot = np.arange(slots)
    xcd = slot // per
    z, r = slot // strips, slot % strips
    lo, hi = cols.min(axis=1), cols.max(axis=1)            # per tile column
    bps = bytes_per_sample
    keys = []
    for p in range(2):
        base = np.array([pp[p] for pp in ptr_pairs], dtype=np.int64)[z]
        # [slot, row, column of tiles]
        row_off = (rows[r].astype(np.int64) * w)[:, :, None]
        a0 = base[:, None, None] + (row_off + lo[None, None, :]) * bps
        a1 = base[:, None, None] + (row_off + hi[None, None, :]) * bps + \
            bps - 1
        l0, l1 = a0 >> 7, a1 >> 7
        span = int((l1 - l0).max()) + 1
        xk = (xcd.astype(np.int64) << 44)[:, None, None]
        for d in range(span):
            ln = l0 + d
            keys.append((xk + ln)[ln <= l1])
    lines = np.unique(np.concatenate(keys)).size
    return lines * 128, 2 * n * w * h * bps


def stage_probe(frames, w, h, bpc, batch, launches):
    """Runs the staging probe (vif_selftest_stage_loads) `launches` times on
    the resident frames, batch frames per launch, alternating between two
    groups of frames (so one launch's lines are gone from the L2 when the
    next group is read again); checks the first launch of each group against
    the host's tile sums and prints the bytes each launch must fetch."""
    import ctypes
    import torch
    from vif_image_fidelity_amd import _lib
    lib = _lib.load()
    pairs = _device_pairs(frames)
    groups = [list(range(g * batch, (g + 1) * batch)) for g in range(2)]
    strips, ntx = -(-h // STAGE_TILE_H), -(-w // STAGE_TILE_W)
    out = torch.empty(batch * strips * ntx, dtype=torch.int32,
                      device="cuda:0")
    bps = 1 if bpc == 8 else 2
    expect = []
    for g in groups:
        ptrs = [(pairs[i][0].data_ptr(), pairs[i][1].data_ptr()) for i in g]
        expect.append(stage_probe_fetch_bytes(ptrs, w, h, bps))
    for k in range(launches):
        g = groups[k % 2]
        refs = (ctypes.c_void_p * batch)(*[pairs[i][0].data_ptr() for i in g])
        dists = (ctypes.c_void_p * batch)(*[pairs[i][1].data_ptr()
                                            for i in g])
        rc = lib.vif_selftest_stage_loads(refs, dists, batch, w, h, bpc,
                                          out.data_ptr(), None)
        if rc != 0:
            raise RuntimeError("vif_selftest_stage_loads: %d" % rc)
        if k < 2:
            want = stage_tile_sums([(frames[i][0], frames[i][1]) for i in g],
                                   w, h)
            got = out.cpu().numpy().view(np.uint32)
            if not np.array_equal(got, want):
                raise AssertionError("staging probe read the wrong samples")
    torch.cuda.synchronize()
    for i, (fetch, planes) in enumerate(expect):
        print("staging probe, frames %s: %d launches; each must fetch %d "
              "bytes (%.1f KiB; the planes alone are %d bytes, x%.4f)"
              % (groups[i], (launches - i + 1) // 2, fetch, fetch / 1024.0,
                 planes, fetch / planes), file=sys.stderr, flush=True)


VALU_WAVES = (4, 5, 6, 7, 8)


def valu_rate(iters):
    """The issue rate of the filter's multiply-and-add pair (a multiply by a
    uniform tap, a VGPR add) at 4..8 waves per SIMD, from the library's
    microbenchmark (vif_selftest_valu_rate): 16 rounds of full occupancy,
    `iters` rounds of 32 VALU instructions per thread.  Prints wave
    instructions per SIMD per quad-cycle at the nominal 2.4 GHz (the counters
    SQ_INSTS_VALU and GRBM_GUI_ACTIVE give the rate at the clock the chip
    actually ran)."""
    import ctypes
    import torch
    from vif_image_fidelity_amd import _lib
    lib = _lib.load()
    for w in VALU_WAVES:
        blocks = 256 * w * 16
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
        ms = ctypes.c_double(0.0)
        best = None
        for _ in range(3):
            rc = lib.vif_selftest_valu_rate(w, iters, blocks, out.data_ptr(),
                                            ctypes.byref(ms), None)
            if rc != 0:
                raise RuntimeError("vif_selftest_valu_rate: %d" % rc)
            best = ms.value if best is None else min(best, ms.value)
        insts = blocks * 4.0 * iters * 32
        quads = best * 1e-3 * VALU_CLOCK_HZ / 4.0
        print("%d waves/SIMD: %.3f ms, %.3f wave instructions per SIMD per "
              "quad-cycle at 2.4 GHz" % (w, best, insts / (1024 * quads)),
              file=sys.stderr, flush=True)


def _oracle_frames(args):
    """Worker of the all-cores oracle figure: generates two frames of the
    1/f workload, then scores them in turn for budget_s seconds; returns
    (frames scored, seconds)."""
    first, step, budget_s = args
    import oracle
    from vif_image_fidelity_amd import synth
    frames = [synth.pink_4k_frame((first + j * step) % 20) for j in range(2)]
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        r, d, b = frames[n % 2]
        oracle.score(r, d, b)
        n += 1
    return n, time.perf_counter() - t0


def cpu_baseline_all_cores(budget_s=12.0, procs=None):
    """The oracle on several host cores at once: one process per core (at
    most 16), each scoring whole frames of the same workload.  Returns
    (frames/s summed over the processes, processes)."""
    import multiprocessing as mp
    procs = procs or min(16, os.cpu_count() or 1)
    with mp.get_context("spawn").Pool(procs) as pool:
        res = pool.map(_oracle_frames,
                       [(k, procs, budget_s) for k in range(procs)])
    return sum(n / t for n, t in res), procs


def cpu_baseline(frames, budget_s=40.0):
    """The oracle, single-threaded, over the frames in order (one pass,
    stopping early once budget_s is spent).  Returns (frames/s, the oracle's
    out[8] of each frame scored, seconds)."""
    import oracle
    outs = []
    t0 = time.perf_counter()
    for r, d, b in frames:
        outs.append(oracle.score(r, d, b)[0])
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return len(outs) / dt, outs, dt


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=150,
                    help="timed steps; a step is one batch of --batch frames")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=5,
                    help="timed repetitions of --steps steps each; the "
                    "median one gives the value")
    ap.add_argument("--frames", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--steps-1080p", type=int, default=500)
    ap.add_argument("--batch", type=int, default=4,
                    help="frames per step (one submission, each kernel "
                    "launched once for them); the fssim mode defaults to 1")
    ap.add_argument("--workload", choices=list(SMALL_WORKLOADS) + ["4k"],
                    default="4k",
                    help="frames mode only: the 3840x2160 8-bit frames, or "
                    "the 1920x1080 10-bit checkerboard pairs, the 1920x1080 "
                    "16-bit bright pairs, the 576x324 8-bit pairs")
    ap.add_argument("--mode", choices=["full", "frames", "strip", "copy",
                                       "fssim", "valu", "stageprobe"],
                    default="full",
                    help="full: the JSON line; frames: only the timed 4K "
                    "loop (for profiler runs); strip: the same for one "
                    "device's share of 4K frames split in eight row strips "
                    "(rows 272..543, 309 input rows); copy: a plain device "
                    "copy of "
                    "known size (counter calibration); fssim: only the 4K "
                    "float SSIM loop (for profiler runs); valu: the issue "
                    "rate of the filter's multiply-and-add pair at 4..8 "
                    "waves per SIMD; stageprobe: the scale-0 kernel's input "
                    "staging alone on 8 of the 4K frames in two groups of "
                    "--batch, --steps launches (counter calibration for its "
                    "access shape)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library scores frames on "
              "a single MI355X (frames shard across GPUs with no exchange, "
              "one context per GPU).  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    cpu_all = None
    if args.mode == "full" and not args.no_cpu_baseline:
        # before this process touches the GPU: the oracle on every core at
        # once, one process per core
        afps, aprocs = cpu_baseline_all_cores()
        cpu_all = {"value": round(afps, 3), "unit": "frames/s",
                   "processes": aprocs, "host_cpus": os.cpu_count(),
                   "kind": "oracle"}
        print("oracle on %d processes: %.2f frames/s" % (aprocs, afps),
              file=sys.stderr, flush=True)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.mode == "copy":
        copy_calibration(args.steps)
        return
    if args.mode == "valu":
        ensure_lib()
        valu_rate(4096)
        return
    ensure_lib()
    import vif_image_fidelity_amd as V
    from vif_image_fidelity_amd import synth

    batch = args.batch
    if not 1 <= batch <= V.MAX_BATCH:
        print("--batch must be 1..%d" % V.MAX_BATCH, file=sys.stderr)
        sys.exit(2)
    reps = args.reps
    if args.mode == "frames" and args.workload in SMALL_WORKLOADS:
        gen, w, h, bpc = SMALL_WORKLOADS[args.workload]
        frames = getattr(synth, gen)()
        res = steady_state(V, frames, w, h, bpc, args.steps, args.warmup,
                           batch=batch, reps=reps, prof_kinds=["scale0"])
        s0_ms, s0_n = res["kernel"]["scale0"]
        print("%s: %.1f frames/s, %.3f ms/step of %d frames; "
              "scale-0 kernel %.1f us per launch"
              % (gen, rate(res, args.steps, batch),
                 1000.0 * median(res["seconds"]) / args.steps, batch,
                 1000.0 * s0_ms / max(s0_n, 1)), file=sys.stderr, flush=True)
        return

    print("generating %d synthetic 3840x2160 frame pairs" % args.frames,
          file=sys.stderr, flush=True)
    frames4k = synth.pink_4k_8bit(frames=args.frames)
    w, h, bpc = 3840, 2160, 8
    if args.mode == "stageprobe":
        stage_probe(frames4k, w, h, bpc, batch, args.steps)
        return
    if args.mode == "fssim":
        fb = batch if "--batch" in sys.argv else 1
        dt, _, geom = time_fssim(V, frames4k, w, h, bpc, args.steps * fb,
                                 args.warmup * fb, batch=fb)
        print("4K float SSIM (factor %d, %d per submission): %.1f frames/s"
              % (geom[0], fb, args.steps * fb / dt), file=sys.stderr,
              flush=True)
        return

    if args.mode == "strip":
        res = steady_state(V, frames4k, w, h, bpc, args.steps, args.warmup,
                           batch=batch, reps=reps, prof_kinds=0xF,
                           strip=STRIP_SHARE)
        kt = {k: round(1000.0 * v[0] / max(v[1], 1), 2)
              for k, v in res["kernel"].items()}
        print("4K strip share %s: %.1f shares/s, kernels (us per launch of "
              "%d): %s" % (STRIP_SHARE, rate(res, args.steps, batch), batch,
                           kt), file=sys.stderr, flush=True)
        return

    # the headline: steps of `batch` frames, median of the repetitions
    main_res = steady_state(V, frames4k, w, h, bpc, args.steps, args.warmup,
                            batch=batch, reps=reps, prof_kinds=["scale0"])
    fps = rate(main_res, args.steps, batch)
    ms_step = 1000.0 * median(main_res["seconds"]) / args.steps
    s0_ms, s0_n = main_res["kernel"]["scale0"]
    s0_avg_ms = s0_ms / max(s0_n, 1)
    print("4K: %.1f frames/s (repetitions: %s), %.3f ms/step of %d frames; "
          "scale-0 kernel %.1f us per launch"
          % (fps, ", ".join("%.1f" % (args.steps * batch / t)
                            for t in main_res["seconds"]),
             ms_step, batch, 1000 * s0_avg_ms), file=sys.stderr, flush=True)
    if args.mode == "frames":
        return

    # one frame per submission (the pages' per-frame call), same frames
    one = steady_state(V, frames4k, w, h, bpc, 500, 20, reps=3,
                       prof_kinds=["scale0"])
    fps_one = rate(one, 500, 1)
    s0_one_ms = one["kernel"]["scale0"][0] / max(one["kernel"]["scale0"][1],
                                                 1)
    print("4K one frame per submission: %.1f frames/s" % fps_one,
          file=sys.stderr, flush=True)
    iso_s0_us = isolated_scale0_us(V, frames4k, w, h, bpc)

    # per-kernel split (all kinds timed; separate run, not the headline)
    allk = steady_state(V, frames4k, w, h, bpc, min(args.steps, 100), 5,
                        batch=batch, reps=1, prof_kinds=0xF)
    split = {k: round(1000.0 * v[0] / max(v[1], 1), 2)
             for k, v in allk["kernel"].items()}

    # 1080p (10-bit checkerboard workload) for the metric's second size, and
    # the bright 16-bit pairs of the same size; 576x324
    f1080 = synth.checker_1080p_10bit()
    r1080 = steady_state(V, f1080, 1920, 1080, 10, args.steps_1080p, 10,
                         reps=3)
    f1080b = synth.bright_1080p_16bit()
    r1080b = steady_state(V, f1080b, 1920, 1080, 16, args.steps_1080p, 10,
                          reps=3)
    fsmall = synth.netflix_576x324_8bit()
    rsmall = steady_state(V, fsmall, 576, 324, 8, 2000, 50, reps=3)

    # batched submissions: each kernel launched once for several frames
    batched = {}
    for key, fr, bw, bh, bb, nb, steps in (
            ("1080p_10bit_batch8", f1080, 1920, 1080, 10, 8, 375),
            ("1080p_16bit_batch8", f1080b, 1920, 1080, 16, 8, 375),
            ("576x324_8bit_batch16", fsmall, 576, 324, 8, 16, 500)):
        rb = steady_state(V, fr, bw, bh, bb, steps, 4, batch=nb, reps=3)
        batched[key] = round(rate(rb, steps, nb), 1)
    fps_host = time_host_frames(V, frames4k, w, h, bpc, 200, 10)
    # one device's share of 4K frames split in eight row strips
    rstrip = steady_state(V, frames4k, w, h, bpc, 100, 5, batch=batch,
                          reps=3, prof_kinds=["scale0"], strip=STRIP_SHARE)
    sg = V.strip_geometry(w, h, *STRIP_SHARE)
    strip_leg = {
        "strip_rows": list(STRIP_SHARE), "input_rows": sg["in_rows"],
        "frames_per_submission": batch,
        "shares_per_s": round(rate(rstrip, 100, batch), 1),
        "scale0_launch_avg_us": round(
            1000.0 * rstrip["kernel"]["scale0"][0] /
            max(rstrip["kernel"]["scale0"][1], 1), 2)}
    print("side figures done", file=sys.stderr, flush=True)

    # float SSIM with its exact decimation, on the same 4K frames and on the
    # 1080p 10-bit frames
    fssim = {"4k_8bit": fssim_leg(V, frames4k, w, h, bpc, 2000,
                                  0 if args.no_cpu_baseline else 5.0),
             "1080p_10bit": fssim_leg(V, f1080, 1920, 1080, 10, 2000, 0)}

    ops = OPS_PER_PIXEL_SCALE0 * w * h  # per frame
    fops = FILTER_OPS_PER_PIXEL_SCALE0 * w * h
    achieved = batch * ops / (s0_avg_ms / 1000.0) / 1e12
    peak = VALU_PEAK_OPS / 1e12
    traffic, frame_bytes = load_traffic(batch)
    roofline = {"bound": "alu", "achieved": round(achieved, 3),
                "peak": round(peak, 2), "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic}

    pops = path_ops(w, h)
    extra = {"timing": {
                 "repetitions": reps,
                 "frames_per_s_each": [round(args.steps * batch / t, 1)
                                       for t in main_res["seconds"]],
                 "warmup_steps_run": main_res["warmup_run"],
                 "method": "untimed warm-up of at least `warmup` steps and "
                           "0.25 s; queue full at t0; each repetition counts "
                           "exactly `steps` submission completions in "
                           "steady state; value = median repetition"},
             "roofline_unit_note": "roofline.achieved and peak count plain "
                                   "IEEE operations per second, 1e12 per "
                                   "unit: fp32/fp64 multiplies and adds and "
                                   "the statistic's compares, selects and "
                                   "conversions, one each (no fused "
                                   "multiply-add); the unit keeps the name "
                                   "TFLOP/s",
             "scale0_ops_per_pixel": {
                 "filter_and_decimation": FILTER_OPS_PER_PIXEL_SCALE0,
                 "statistic": STAT_OPS_PER_PIXEL},
             "scale0_frac_filter_ops_only": round(
                 batch * fops / (s0_avg_ms / 1000.0) / VALU_PEAK_OPS, 4),
             "fps_4k_one_frame_per_submission": round(fps_one, 1),
             "scale0_frac_one_frame_per_submission": round(
                 ops / (s0_one_ms / 1000.0) / VALU_PEAK_OPS, 4),
             "fps_1080p_10bit": round(rate(r1080, args.steps_1080p, 1), 1),
             "fps_1080p_16bit": round(rate(r1080b, args.steps_1080p, 1), 1),
             "fps_576x324_8bit": round(rate(rsmall, 2000, 1), 1),
             "fps_4k_host_frames_pinned_pcie": round(fps_host, 1),
             "fps_batched": batched,
             "strip_share_4k": strip_leg,
             "host_us_per_frame_576x324": {
                 k: round(v, 2) for k, v in rsmall["host_us"].items()},
             "kernel_avg_us_4k": split,
             "scale0_launch_avg_us": round(1000 * s0_avg_ms, 2),
             "scale0_frames_per_launch": batch,
             "scale0_kernel_isolated_us": round(iso_s0_us, 2),
             "scale0_isolated_frac_of_valu_peak": round(
                 ops / (iso_s0_us * 1e-6) / VALU_PEAK_OPS, 4),
             "path_ops_per_frame": pops,
             "path_frac_of_valu_peak": round(pops * fps / VALU_PEAK_OPS, 4),
             "host_us_per_frame_4k": {
                 k: round(v, 2) for k, v in one["host_us"].items()},
             "host_us_per_frame_1080p": {
                 k: round(v, 2) for k, v in r1080["host_us"].items()},
             "fssim": fssim}
    if frame_bytes:
        gbs = frame_bytes * fps / 1e9
        extra["hbm_gbs_per_frame_counters"] = round(gbs, 1)
        extra["hbm_frac_of_peak"] = round(gbs / HBM_PEAK_GBS, 4)
    # the same for the 1920x1080 10-bit pairs in batches of 8
    _, fb1080 = load_traffic(8, PROFILE_TRAFFIC_1080P)
    if fb1080:
        gbs = fb1080 * batched["1080p_10bit_batch8"] / 1e9
        extra["hbm_1080p_10bit_batch8"] = {
            "gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "frame_bytes": fb1080}

    # every timed frame gave one output, the same every time it was scored
    stable = all(len(v) == 1 for v in main_res["outputs"].values())
    cpu = None
    parity_fail = False
    if not args.no_cpu_baseline:
        cfps, ref_outs, cdt = cpu_baseline(frames4k)
        cn = len(ref_outs)
        cpu = {"value": round(cfps, 4), "unit": "frames/s", "cores": 1,
               "kind": "oracle",
               "sample": "frames 0..%d of the 3840x2160 8-bit frame pairs "
                         "the GPU timed, one pass, single thread, %.1f s"
                         % (cn - 1, cdt)}
        extra["cpu_oracle_all_cores"] = cpu_all
        # the GPU's outputs of the same frames, from the timed loop
        maxd, same = 0.0, stable
        for i, want in enumerate(ref_outs):
            for got_b in main_res["outputs"].get(i, ()):
                got = np.frombuffer(got_b, dtype=np.float64)
                maxd = max(maxd, float(np.max(np.abs(got - want))))
                same = same and got.tobytes() == want.tobytes()
            if i not in main_res["outputs"]:
                same = False
        extra["parity_vs_oracle"] = {
            "frames": cn, "bit_identical": bool(same),
            "max_abs_diff": maxd, "gate": PARITY_GATE}
        parity_fail = not maxd <= PARITY_GATE
    else:
        extra["outputs_stable_across_repeats"] = stable

    line = {
        "metric": METRIC,
        "value": round(fps, 2),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "pink_4k_8bit: 3840x2160 8-bit luma pairs, "
                               "1/f-noise ref, 2x down/up-scaled dist, %d "
                               "frames resident in HBM, %d frames per step "
                               "(one batched submission)" % (args.frames,
                                                              batch),
                   "w": w, "h": h, "bpc": bpc, "scales": 4,
                   "frames_per_step": batch},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)
    if parity_fail:
        print("PARITY FAILURE: the GPU's outputs differ from the oracle's by "
              "more than %g" % PARITY_GATE, file=sys.stderr, flush=True)
        sys.exit(3)


if __name__ == "__main__":
    main()
