"""The oracle against the values the pages print (tests/golden/)."""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_e4m3_range_matches_the_page():
    with open(os.path.join(GOLDEN, "e4m3_range.json")) as f:
        g = json.load(f)
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    finite = vals[np.isfinite(vals)]
    # the largest and smallest finite E4M3 values are the page's saturation bounds
    assert finite.max() == g["e4m3_max_finite"] and finite.min() == g["e4m3_min_finite"]
    # the bounds round to themselves, and a block whose amax is the bound needs no scaling
    assert oracle.e4m3_round(np.array([g["e4m3_max_finite"]]))[0] == g["e4m3_max_finite"]
    assert oracle.block_exponent(np.array([g["e4m3_max_finite"]]))[0] == 0
    assert oracle.block_exponent(np.array([np.nextafter(g["e4m3_max_finite"], np.inf)]))[0] == 1
