"""Writes tests/golden/oracle_regression.json from the CPU oracle only.

The file freezes the oracle's outputs (as IEEE hex) on the two small
workloads so an accidental change to the oracle's arithmetic shows up as a
test failure.  It is a regression guard of the oracle against its own past,
not a pin of the oracle to the pages (those are in test_oracle_pins.py).

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import struct
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from vif_image_fidelity_amd import synth  # noqa: E402


def dhex(v):
    return struct.pack(">d", float(v)).hex()


def fhex(v):
    return struct.pack(">f", float(v)).hex()


def main():
    cases = []
    for name in ("netflix_576x324_8bit", "tiny_frames_8bit"):
        frames = synth.WORKLOADS[name]()
        for i, (ref, dist, bpc) in enumerate(frames):
            out, sums = oracle.score(ref, dist, bpc)
            cases.append({
                "workload": name, "frame": i, "w": int(ref.shape[1]),
                "h": int(ref.shape[0]), "bpc": bpc,
                "out_hex": [dhex(v) for v in out],
                "sums_hex": [fhex(v) for v in sums],
                "out": [float(v) for v in out],
            })
    path = os.path.join(HERE, "oracle_regression.json")
    with open(path, "w") as f:
        json.dump({"_comment": "written by tests/golden/make_golden.py from "
                   "oracle/ only; regression guard of the oracle",
                   "cases": cases}, f, indent=1)
    print("wrote %d cases to %s" % (len(cases), path))


if __name__ == "__main__":
    main()
