"""Writes rope_bands.json: rotary tables for the GPU tests of an explicit
frequency table, computed by the oracle only.

    python tests/golden/make_rope_bands.py

Table: the decoupled key takes the highest-frequency bands of the dense
backbone's per-axis rotary spectrum (VideoMLA paper, sections 3.2 and 4.1).  The
pages do not print the backbone's per-axis channel counts; the reading here is
the near-equal split of the 128 head channels with t taking the remainder,
(44, 42, 42) -- the split this repository's dense baseline uses.  Two
allocations of the 16 key pairs: the layer geometries' (4, 6, 6) and the
paper's (6, 5, 5) (section 4.1).
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import mla  # noqa: E402

AXIS_DIMS = (44, 42, 42)
THETA = 10000.0


def main():
    out = {"source": "oracle.mla.backbone_band_frequencies", "theta": THETA, "axis_dims": list(AXIS_DIMS),
           "tables": {}}
    for pairs in ((4, 6, 6), (6, 5, 5)):
        f = mla.backbone_band_frequencies(pairs, AXIS_DIMS, THETA)
        out["tables"]["%d,%d,%d" % pairs] = [float(v) for v in f]
    with open(os.path.join(HERE, "rope_bands.json"), "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")


if __name__ == "__main__":
    main()
