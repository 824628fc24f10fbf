"""The roofline byte counts of bench.py follow the library's work split:
the constants it mirrors equal those in the streaming kernels' source, and
the dense units it counts cover the dense branch exactly once."""
import os
import re

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_moe_transformer_amd", "csrc")


def constant(fname, name):
    src = open(os.path.join(CSRC, fname)).read()
    m = re.search(r"constexpr int " + name + r" = (\d+);", src)
    assert m, name
    return int(m.group(1))


def test_mirrored_split_constants():
    assert bench.DENSE_ROUTE_EIGHTHS == constant("stream.hip", "kDenseRouteEighths")
    assert bench.DENSE_KSLICES == constant("common.h", "kDenseKS")


def test_dense_units_partition_the_branch():
    """With every unit in the routed launch the count is the whole dense
    gate/up pair; with the split it is the complement of the router's share."""
    s = synth.DECODE
    old = bench.DENSE_ROUTE_EIGHTHS
    try:
        bench.DENSE_ROUTE_EIGHTHS = 0
        whole, cols = bench.dense_units_in_gateup(s)
        assert whole == 2 * s.hidden * s.dense_dim * 2
        assert cols == 2 * s.dense_dim
        bench.DENSE_ROUTE_EIGHTHS = 8
        assert bench.dense_units_in_gateup(s) == (0, 0)
    finally:
        bench.DENSE_ROUTE_EIGHTHS = old
    part, _ = bench.dense_units_in_gateup(s)
    assert 0 < part < whole
