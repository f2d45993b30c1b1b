"""bench.py's measurement plumbing, on the CPU: the kernel source hash that
keys the stored counter records ignores comments and whitespace but not
code, a record is used only while that hash matches, the counted-bytes
rate is bytes over duration, the batch order puts the shared prefix's
members first, the shared-prefix call's byte count takes the prefix
once, and the prefill bench's oracle leg finds a planted row error."""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import numpy as np  # noqa: E402
import workload as w  # noqa: E402


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


def test_cpu_baseline_reports_both_oracles():
    """The CPU baseline's plumbing on a tiny state held in host tensors: the
    float64 oracle's one-core and threaded runs and its single-precision
    twin over the same pairs. The state's outputs are the float64 oracle's
    own rows, so both parity figures of that oracle are 0 and the twin's
    difference from it is its own rounding (well under 1e-5 here)."""
    import types

    import numpy as np
    import torch

    import oracle
    import workload as w
    sh = w.Shape("tiny", 2, 8, 2, 64, 3, 20, 90)
    S = types.SimpleNamespace(shape=sh, B=3, k_pool=[], v_pool=[], q=[], out=[])
    cases = [w.host_case(sh, 40 + l, context_lens=[20, 55, 90], share=False, permute=False)
             for l in range(2)]
    S.tables = cases[0].tables.block_tables
    S.ctx = cases[0].tables.context_lens
    as_t = lambda a: torch.from_numpy(a.view(np.int16).copy())
    for c in cases:
        assert np.array_equal(c.tables.block_tables, S.tables)
        S.k_pool.append(as_t(c.k_pool))
        S.v_pool.append(as_t(c.v_pool))
        S.q.append(as_t(c.q))
        want, rc = oracle.default().decode(c.q, c.k_pool, c.v_pool, S.tables, S.ctx, sh.n_kv,
                                           sh.scale)
        assert rc == 0
        S.out.append(torch.from_numpy(want.astype(np.float32)))
    multi, worst, done, worst_p = bench.cpu_baseline(torch, S, 0.05, 0.05)
    single = multi["single_core"]
    assert single["cores"] == 1 and single["kind"] == "oracle" and done >= 1
    assert multi["cores"] >= 1 and multi["full_layers_checked"] >= 1
    assert worst < 1e-6 and worst_p < 1e-6   # the fp32 copy of the oracle's own rows
    twin = single["fp32_twin"]
    assert twin["value"] > 0 and twin["cores"] == 1
    assert 0 < twin["max_abs_vs_float64_oracle"] < 1e-5


def test_prefill_cpu_baseline_checks_rows_against_the_oracle():
    """The prefill bench's oracle leg recomputes sampled rows one by one:
    against the verification oracle's own rows it finds no difference
    beyond fp32 rounding, and it reports its rate, core count and sample."""
    import torch
    import oracle
    sh = w.Shape("x", 1, 8, 2, 64, 1, 1, 1)
    ctx = np.array([40, 90], np.int32)
    C = 8
    hc = w.host_case(sh, 5, context_lens=ctx)
    qv = w.normal_bf16(w.rng(5, 15), (2, C, 8, 64))
    want, rc = oracle.default().verify(qv, hc.k_pool, hc.v_pool, hc.tables.block_tables, ctx, 2,
                                       sh.scale)
    assert rc == 0
    tt = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    res = bench.rows_cpu_baseline(torch, tt(hc.k_pool), tt(hc.v_pool), tt(qv),
                                     torch.from_numpy(want.astype(np.float32)),
                                     hc.tables.block_tables, ctx, C, 2, sh.scale, 0, 0.05)
    assert res["kind"] == "oracle" and res["cores"] == 1 and res["value"] > 0
    assert res["parity_rows"] >= 4 and res["parity_max_abs"] <= 1e-6
    # a planted error in one row is found when that row is sampled
    bad = want.astype(np.float32).copy()
    bad[0, 0, 0, 3] += 0.01
    res = bench.rows_cpu_baseline(torch, tt(hc.k_pool), tt(hc.v_pool), tt(qv), torch.from_numpy(bad),
                                     hc.tables.block_tables, ctx, C, 2, sh.scale, 0, 0.05)
    assert res["parity_max_abs"] >= 0.009
