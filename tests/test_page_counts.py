"""Work/traffic accounting against the counts the pages print (tests/golden)."""
import json
import os

import pytest

from fp32_gemm_major_amd import roofline as rf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_counts.json")
ENTRIES = json.load(open(GOLDEN, encoding="utf-8"))["entries"]


def _value(q, x):
    if q == "flops":
        return rf.flops(x["M"], x["N"], x["K"])
    if q == "alg_bytes":
        return rf.alg_bytes(x["M"], x["N"], x["K"], x["beta"])
    if q == "arithmetic_intensity":
        return rf.arithmetic_intensity(x["M"], x["N"], x["K"], x["beta"])
    if q == "seconds_at_peak":
        return rf.seconds_at_peak(x["M"], x["N"], x["K"], x["peak"])
    if q == "tile_loads_per_block":
        return rf.tile_loads(x["BM"], x["BN"], x["K"], x["BM"], x["BN"])
    if q == "tiles":
        return rf.tiles(x["M"], x["N"], x["BM"], x["BN"])
    if q == "tile_loads":
        return rf.tile_loads(x["M"], x["N"], x["K"], x["BM"], x["BN"])
    if q == "naive_intensity":
        # one output of the one-thread-per-element kernel: 2K flops over 2K floats
        return rf.flops(1, 1, x["K"]) / (2 * x["K"] * rf.FP32)
    if q == "ridge_point":
        return rf.ridge_point(x["peak_flops"], x["peak_bytes"])
    raise KeyError(q)


@pytest.mark.parametrize("e", ENTRIES, ids=[e["id"] for e in ENTRIES])
def test_page_count(e):
    got = _value(e["quantity"], e["inputs"])
    want = e["printed"]
    assert abs(got - want) <= e["rel_tol"] * abs(want) + 1e-12, (got, want, e["page"],
                                                                  e["section"])
