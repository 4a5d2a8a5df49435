"""The benchmark's byte accounting against the one figure the pages print for
this path (tests/golden/kv_row_bytes.json)."""

import json
import os

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_row_bytes.json")


def test_kv_bytes_per_context_row_matches_the_pages():
    g = json.load(open(GOLDEN))
    assert g["heads"] * g["head_dim"] == g["hidden"]
    assert bench.kv_bytes_per_row(g["layers"], g["heads"], g["head_dim"], g["elem_bytes"]) == g["bytes_per_row"]
    assert g["bytes_per_row"] == 48 * 1024
