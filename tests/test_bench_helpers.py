"""bench.py's measurement plumbing, on the CPU: the kernel source hash that
keys the stored counter records ignores comments and whitespace but not
code, a record is used only while that hash matches, and the counted-bytes
rate is bytes over duration."""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_source_hash_ignores_comments_not_code(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("// header\nint f(int x) {\n  return x + 1;  // one\n}\n/* block\n comment */\n")
    b.write_text("int f(int x) { return x + 1; }\n")
    c.write_text("int f(int x) { return x + 2; }\n")
    ha, hb, hc = (bench.kernel_source_hash(str(p)) for p in (a, b, c))
    assert ha == hb
    assert hb != hc


def test_stored_traffic_follows_the_hash(tmp_path, monkeypatch):
    rec = {"workload": "w1", "kernel_source_sha256_16": bench.kernel_source_hash(),
           "hbm_bytes_per_dispatch": {"k": 1234}}
    path = tmp_path / "pmc_kf_w1.txt"
    path.write_text("summary text\n" + json.dumps(rec) + "\n")
    monkeypatch.setattr(bench, "PMC_FILE", str(tmp_path / "pmc_{kernel}_{workload}.txt"))
    assert bench.stored_traffic("w1", "k", kernel_file="kf") == (1234, None)
    assert bench.stored_traffic("w1", "other", kernel_file="kf")[0] is None
    assert bench.stored_traffic("w2", "k", kernel_file="kf")[0] is None
    rec["kernel_source_sha256_16"] = "0" * 16
    path.write_text(json.dumps(rec) + "\n")
    t, why = bench.stored_traffic("w1", "k", kernel_file="kf")
    assert t is None and "changed" in why


def test_measured_gbs():
    assert bench.measured_gbs(2e9, 1000.0) == pytest.approx(2000.0)
    assert bench.measured_gbs(None, 1000.0) is None
    assert bench.measured_gbs(1e9, 0) is None

