"""The cost model reproduces the ScaNN page's worked example (golden fixture)."""
import os

from mips_ah_partition_amd import costs

GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_example_costs.txt")


def test_worked_example():
    g = {}
    for line in open(GOLD):
        if line.strip() and not line.startswith("#"):
            k, v = line.split()
            g[k] = int(v)
    c = costs.per_query(g["n"], g["d"], g["dpb"], g["num_leaves"], g["leaves_to_search"], g["reorder"])
    assert c.raw_bytes == g["raw_bytes"]
    assert c.blocks == g["blocks"]
    assert c.code_bytes_per_point == g["code_bytes_per_point"]
    assert c.code_bytes_total == g["code_bytes_total"]
    assert c.partition_macs == g["partition_macs"]
    assert c.lut_macs == g["lut_macs"]
    assert c.scan_lookups == g["scan_lookups"]
    assert c.reorder_macs == g["reorder_macs"]
    # "The scan is about fifty times the next-largest term"
    assert 40 < c.scan_lookups / max(c.partition_macs, c.lut_macs, c.reorder_macs) < 60
