"""bench.py's measurement plumbing, on the CPU: the kernel source hash that
keys the stored counter records ignores comments and whitespace but not
code, a record is used only while that hash matches, the counted-bytes
rate is bytes over duration, the batch order puts the shared prefix's
members first, and the shared-prefix call's byte count takes the prefix
once."""
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



def test_members_first():
    import numpy as np
    cl = np.array([100, 3000, 2048, 2049, 17, 5000, 2047], np.int32)
    got = bench.members_first(cl, 2048)
    assert got.tolist() == [3000, 2049, 5000, 100, 2048, 17, 2047]
    assert bench.members_first(cl, 0).tolist() == cl.tolist()


def test_prefix_call_alg_bytes():
    """Counted from the definition, sequence by sequence: a member past the
    prefix reads its tokens after the prefix, everyone else its whole
    context, and the prefix is read once."""
    import numpy as np

    class Sh:
        n_kv, d, n_q = 8, 128, 32

    class S:
        shape = Sh()
        prefix_blocks = 4        # 64 tokens
        prefix_members = 3

    ctx = np.array([65, 64, 300, 500, 40], np.int64)
    per_tok = 2 * 8 * 128 * 2
    own_tokens = (65 - 64) + 64 + (300 - 64) + 500 + 40   # sequence 1 ends inside the prefix
    tiles = (5 - 4) + 4 + (19 - 4) + 32 + 3
    want = (per_tok * (own_tokens + 64) + 5 * 32 * 128 * 6 + 4 * (tiles + 4) + 4 * 5
            + 2 * 2 * 5 * 8 * 128 * 2)
    assert bench.prefix_call_alg_bytes(S, ctx) == want
