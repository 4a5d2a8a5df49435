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


def _fake_workload(pool_dtype):
    import types

    import torch

    ctx = torch.tensor([100, 0, 17], dtype=torch.int32)
    return types.SimpleNamespace(dtype=torch.bfloat16, pool_dtype=pool_dtype, ctx_lens=ctx, H=4, Dh=128,
                                 total_q=48, page_size=16, bs=3)


def test_cross_bytes_count_pool_elements_at_their_width():
    import torch

    bf = bench.cross_bytes(_fake_workload(torch.bfloat16))
    e4 = bench.cross_bytes(_fake_workload(torch.float8_e4m3fn))
    kv_bf16 = 117 * 4 * 128 * 2 * 2
    assert bf - e4 == kv_bf16 // 2          # only the key/value reads shrink
    assert e4 == kv_bf16 // 2 + 2 * 48 * 4 * 128 * 2 + 4 * (7 + 0 + 2) + 4 * 7 + 4 * 128


def test_traffic_record_is_per_workload(tmp_path, monkeypatch):
    import types

    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "t.json"))
    args = types.SimpleNamespace(config=5, layout="head_major", candidates=1, kv_fp8=False, upstream=False,
                                 dit=False)
    key = bench.workload_key(args)
    rec = {"workload": key, "sources_sha256": bench.kernel_sources_hash(), "traffic_bytes_per_launch": 123.0}
    json.dump({"records": {key: rec}}, open(tmp_path / "t.json", "w"))
    assert bench.measured_traffic(key) == 123.0
    args.kv_fp8 = True
    assert bench.measured_traffic(bench.workload_key(args)) is None
    rec["sources_sha256"] = "0" * 64
    json.dump({"records": {key: rec}}, open(tmp_path / "t.json", "w"))
    assert bench.measured_traffic(key) is None


def test_bench_refuses_more_than_one_gpu():
    # The path runs on one GPU: --gpus above 1 ends with a message and status 2,
    # before torch or the GPU is touched.
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["requested_gpus"] == 2 and "one GPU" in line["error"]
