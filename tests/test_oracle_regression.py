"""Regression guard: the oracle still returns the outputs frozen in
tests/golden/oracle_regression.json (written by make_golden.py from the
oracle alone).  A deliberate change to the oracle's arithmetic regenerates
the file in the same commit, whose message names the passage or reading
that justifies it.  CPU only."""
import json
import os
import struct

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "oracle_regression.json")))


def _frames(name):
    from vif_image_fidelity_amd import synth
    return synth.WORKLOADS[name]()


@pytest.mark.parametrize("name", ["netflix_576x324_8bit", "tiny_frames_8bit"])
def test_oracle_matches_frozen_outputs(orc, name):
    frames = _frames(name)
    cases = [c for c in GOLD["cases"] if c["workload"] == name]
    assert len(cases) == len(frames)
    for c, (ref, dist, bpc) in zip(cases, frames):
        assert (c["w"], c["h"], c["bpc"]) == (ref.shape[1], ref.shape[0], bpc)
        out, sums = orc.score(ref, dist, bpc)
        assert [struct.pack(">d", float(v)).hex() for v in out] == c["out_hex"]
        assert [struct.pack(">f", float(v)).hex() for v in sums] == \
            c["sums_hex"]


def test_oracle_matches_frozen_option_outputs(orc):
    ref, dist, bpc = _frames("netflix_576x324_8bit")[0]
    cases = GOLD["option_cases"]
    assert len(cases) >= 6
    for c in cases:
        out, sums = orc.score(ref, dist, bpc, options=c["options"])
        assert [struct.pack(">d", float(v)).hex() for v in out] == \
            c["out_hex"], c["options"]
        assert [struct.pack(">f", float(v)).hex() for v in sums] == \
            c["sums_hex"], c["options"]
