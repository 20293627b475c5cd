"""The library called from plain C (vif_image_fidelity_amd/csrc/score_raw.c,
built with gcc as C11 against include/vif.h and include/fssim.h): frames
written to raw files, scored by the C program with device frames
(vif_score, fssim_score) and host frames (vif_score_host), every output bit
for bit equal to the oracle's.  The program runs in a child process."""
import os
import subprocess
import struct

import numpy as np
import pytest

from libutil import ensure_built

pytestmark = pytest.mark.gpu


def _binary():
    ensure_built()
    from vif_image_fidelity_amd import build
    if not os.path.exists(build.EXAMPLE):
        build.build_example()
    return build.EXAMPLE


def _bits(values):
    return [struct.unpack("<Q", struct.pack("<d", float(v)))[0]
            for v in values]


@pytest.mark.parametrize("name,index", [("netflix_576x324_8bit", 0),
                                        ("checker_1080p_10bit", 1),
                                        ("bright_1080p_16bit", 2)])
def test_c_caller_matches_oracle(orc, tmp_path, name, index):
    from vif_image_fidelity_amd import synth
    ref, dist, bpc = synth.WORKLOADS[name]()[index]
    h, w = ref.shape
    rp, dp = tmp_path / "ref.raw", tmp_path / "dist.raw"
    np.ascontiguousarray(ref).astype("<u%d" % ref.itemsize).tofile(rp)
    np.ascontiguousarray(dist).astype("<u%d" % dist.itemsize).tofile(dp)
    print("C caller case %s[%d] %dx%d bpc %d" % (name, index, w, h, bpc),
          flush=True)
    r = subprocess.run([_binary(), str(w), str(h), str(bpc), str(rp),
                        str(dp)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    got = {}
    for line in r.stdout.split("\n"):
        if line.strip():
            key, *vals = line.split()
            got[key] = [int(v, 16) for v in vals]
    exp = orc.score(ref, dist, bpc)[0]
    assert got["vif"] == _bits(exp)
    assert got["vif_host"] == _bits(exp)
    assert got["fssim"] == _bits(orc.fssim_score(ref, dist, bpc))
