"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic
byte and flop counts the roofline figures divide by, and the counter-traffic
report."""

import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_attention_bytes_count_every_key_and_value_once():
    cfg = dict(bench.CFG)
    ctx = np.array([1000, 2000])
    cfg["C"] = 2
    R = 2 * cfg["N"]
    kv = (1000 + R + 2000 + R) * 8 * 128 * 2 * 2  # K and V, bf16, 8 KV heads of 128
    q = 2 * R * 32 * 128 * 2
    o = 2 * R * 32 * 128 * 4
    assert bench.attention_bytes(ctx, cfg) == kv + q + o


def test_accept_bytes_read_each_row_once_plus_the_residual_rows():
    cfg = dict(bench.CFG)
    n_draft = np.array([3, 0, 3])   # FULL, FRESH, FULL
    accepted = np.array([3, 0, 1])  # the last one rejected its second draft
    V, N = cfg["V"], cfg["N"]
    want = ((3 + N) + (0 + N) + (3 + N) + 2) * V * 2
    assert bench.accept_bytes(n_draft, accepted, cfg) == want


def test_projection_flops_at_the_8b_step():
    qkv, o = bench.projection_flops(dict(bench.CFG))
    # base GEMM over 512 rows plus the rank-32 delta on the 256 MASK rows
    assert qkv == 2 * 512 * 4096 * 6144 + 2 * 256 * 32 * (3 * 4096 + 6144)
    assert o == 2 * 512 * 4096 * 4096 + 2 * 256 * 32 * (4096 + 4096)
    assert qkv == pytest.approx(26.07e9, rel=1e-3) and o == pytest.approx(17.31e9, rel=1e-3)


def _counter_tree(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_traffic_report_scales_by_the_copy_and_compares_with_the_algorithmic_bytes(tmp_path, capsys):
    att, mrg, cp = "void isd::attention_kernel<x>(p)", "void isd::attention_merge_kernel<128>(p)", "copyBuffer"
    gib_kib = (1 << 30) / 1024
    _counter_tree(tmp_path / "f", [(att, "FETCH_SIZE", 1000.0), (att, "FETCH_SIZE", 1200.0),
                                   (mrg, "FETCH_SIZE", 100.0)])
    _counter_tree(tmp_path / "w", [(att, "WRITE_SIZE", 50.0), (mrg, "WRITE_SIZE", 10.0)])
    # the copy reads half of what it copied by this counter (scale 2), writes all (scale 1)
    _counter_tree(tmp_path / "cf", [(cp, "FETCH_SIZE", gib_kib / 2)])
    _counter_tree(tmp_path / "cw", [(cp, "WRITE_SIZE", gib_kib)])
    algo = tmp_path / "algo.json"
    algo.write_text(json.dumps({"attention_bytes_per_step": [2.0e6, 2.6e6], "accept_bytes_per_step": [1.0],
                                "layers": 1, "copy_probe_bytes": 1 << 30}))
    bench.traffic_report(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"), str(tmp_path / "cw"),
                         str(algo))
    out = capsys.readouterr().out
    rec = json.loads([l for l in out.splitlines() if l.startswith("RESULT ")][-1][len("RESULT "):])
    # per call: (mean fetch 1100 + 100) KiB x 2 + (50 + 10) KiB x 1
    want = ((1100.0 + 100.0) * 2 + 60.0) * 1024
    assert rec["hbm_bytes_per_call"] == int(want)
    assert rec["algorithmic_bytes_per_call"] == int(2.3e6)
    assert rec["ratio_to_algorithmic"] == round(want / 2.3e6, 4)
    assert rec["kernel_source_sha256"] == bench.kernel_source_hash()


def test_committed_traffic_is_quoted_only_for_the_current_attention_source(tmp_path, monkeypatch):
    rec = bench.committed_traffic()
    if rec is not None:  # the committed counters belong to this source
        assert rec["kernel_source_sha256"] == bench.kernel_source_hash()
        assert 1.0 < rec["ratio_to_algorithmic"] < 1.2
    # a record for another source is not quoted
    stale = tmp_path / "traffic.txt"
    stale.write_text("RESULT " + json.dumps({"kernel_source_sha256": "0" * 64, "hbm_bytes_per_call": 1}) + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.committed_traffic() is None
