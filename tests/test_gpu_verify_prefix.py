"""The verification pass for a batch that shares a prompt prefix
(pkv_paged_attn_verify_prefix): the prefix's tiles are read once for every
member whose query tokens all lie after the prefix (prefix units of the
split, 32 member rows (query token, head) per tile), each member's own tiles
after the prefix by its own unit, and the merge kernel combines both.

The bar: outputs within 1e-3 of the oracle's verification attention (which
walks every sequence's own table), within 2.5e-5 of pkv_paged_attn_verify
on the same inputs (only the order of the fp32 sums differs). Members whose
query tokens reach into the prefix, sequences outside the member range,
query lengths 1 .. 33, more than 16 rows per KV head and both head sizes are
covered; an empty prefix is pkv_paged_attn_verify bit for bit; a member whose
table does not start with the prefix is caught on the device; scores that
rise and fall by many log2 units (tests/rescale_cases.py) drive the online
softmax's rescale and the merge of far-apart partials through this path too.
"""
import numpy as np
import pytest

import rescale_cases as rc
import workload as w
from gpu_util import TOL, max_abs, to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu

CROSS = 2.5e-5   # GPU against GPU, two fp32 summation orders


@pytest.fixture(scope="module")
def pkv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import paged_kv_cache_468_amd as lib
    return lib


def _shape(n_q, n_kv, d, prefix):
    return w.Shape(f"{n_q}/{n_kv} d{d}", 1, n_q, n_kv, d, 1, 1, 1, prefix_tokens=prefix)


def _run(pkv, hc, qv, scale, prefix=None, first=0, count=None, table=None):
    """pkv_paged_attn_verify_prefix (prefix=True) or pkv_paged_attn_verify."""
    import torch
    B = qv.shape[0]
    out = torch.full(qv.shape, float("nan"), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    args = (out, to_dev_bf16(qv), to_dev_bf16(hc.k_pool), to_dev_bf16(hc.v_pool),
            to_dev_i32(hc.tables.block_tables), to_dev_i32(hc.tables.context_lens), scale,
            int(hc.tables.context_lens.max()))
    if prefix:
        count = B - first if count is None else count
        pt = to_dev_i32(hc.tables.prefix_phys if table is None else table)
        pkv.pkv_paged_attn_verify_prefix(*args, pt, first, count, err_flag=err)
    else:
        pkv.pkv_paged_attn_verify(*args, err_flag=err)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), int(err.item())


CASES = [
    # n_q, n_kv, d, prefix tokens, q_len, context lengths (some with query
    # tokens inside the prefix)
    (32, 8, 128, 256, 5, [100, 256, 260, 261, 300, 1000, 2048, 4000, 17, 272]),
    (20, 4, 64, 48, 3, [17, 40, 51, 52, 77, 130, 300, 64]),
    (16, 16, 128, 64, 1, [65, 80, 200, 1000, 64, 3]),
    (64, 8, 128, 128, 5, [133, 500, 2000, 8000, 60]),
    (32, 1, 128, 32, 2, [34, 40, 90, 33, 1200]),        # 64 rows per KV head
    (4, 4, 64, 1024, 12, [1036, 2000, 3000, 4096]),    # a long prefix
    (8, 2, 128, 160, 33, [193, 200, 1500, 600, 190]),  # 33 query tokens: 132 rows per KV head
]


def _case(i):
    n_q, n_kv, d, prefix, q_len, ctx = CASES[i]
    hc = w.host_case(_shape(n_q, n_kv, d, prefix), 500 + i, context_lens=ctx, share=True)
    qv = w.normal_bf16(w.rng(500 + i, 8), (len(ctx), q_len, n_q, d))
    return hc, qv


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("members", ["all", "inner"])
def test_verify_prefix_parity(pkv, orc, case, members):
    hc, qv = _case(case)
    B = qv.shape[0]
    first, count = (0, B) if members == "all" else (1, B - 2)
    print(f"case {CASES[case][:5]} members {members}", flush=True)
    got, err = _run(pkv, hc, qv, hc.shape.scale, prefix=True, first=first, count=count)
    ref, err_r = _run(pkv, hc, qv, hc.shape.scale)
    assert err == 0 and err_r == 0
    assert np.isfinite(got).all()
    want, rc_ = orc.verify(qv, hc.k_pool, hc.v_pool, hc.tables.block_tables,
                           hc.tables.context_lens, hc.shape.n_kv, hc.shape.scale)
    assert rc_ == 0
    e_o, e_v = max_abs(got, want), max_abs(got, ref)
    print(f"  vs oracle {e_o:.2e}, vs pkv_paged_attn_verify {e_v:.2e}")
    assert e_o <= TOL
    assert e_v <= CROSS


def test_verify_prefix_member_table_mismatch(pkv, orc):
    """A member past the prefix whose table holds another block inside the
    prefix range: its rows are NaN and PKV_DEVERR_PREFIX is set; the other
    rows match the oracle on the same tables."""
    hc, qv = _case(0)
    bt = hc.tables.block_tables
    s, t = 5, 7                      # contexts 1000 and 4000: both past the prefix
    bt[s, 3] = bt[t, 40]
    assert bt[s, 3] != hc.tables.prefix_phys[3]
    got, err = _run(pkv, hc, qv, hc.shape.scale, prefix=True)
    assert err == pkv.PKV_DEVERR_PREFIX
    assert np.isnan(got[s]).all()
    others = np.arange(qv.shape[0]) != s
    assert np.isfinite(got[others]).all()
    want, rc_ = orc.verify(qv, hc.k_pool, hc.v_pool, bt, hc.tables.context_lens, hc.shape.n_kv,
                           hc.shape.scale)
    assert rc_ == 0
    assert max_abs(got[others], want[others]) <= TOL


def test_verify_empty_prefix_is_verify(pkv):
    """No members, or no prefix blocks: pkv_paged_attn_verify's computation,
    bit for bit."""
    hc, qv = _case(0)
    ref, _ = _run(pkv, hc, qv, hc.shape.scale)
    got, err = _run(pkv, hc, qv, hc.shape.scale, prefix=True, first=0, count=0)
    assert err == 0 and np.array_equal(got, ref)
    got, err = _run(pkv, hc, qv, hc.shape.scale, prefix=True, table=np.zeros(0, np.int32))
    assert err == 0 and np.array_equal(got, ref)


def test_verify_prefix_host_errors(pkv):
    import torch
    hc, qv = _case(1)
    B = qv.shape[0]
    with pytest.raises(pkv.PkvError) as info:      # member range past the batch
        _run(pkv, hc, qv, hc.shape.scale, prefix=True, first=2, count=B)
    assert info.value.status == pkv.PKV_EINVAL
    small = torch.empty(64, dtype=torch.uint8, device="cuda")
    out = torch.empty(qv.shape, dtype=torch.float32, device="cuda")
    with pytest.raises(pkv.PkvError) as info:
        pkv.pkv_paged_attn_verify_prefix(
            out, to_dev_bf16(qv), to_dev_bf16(hc.k_pool), to_dev_bf16(hc.v_pool),
            to_dev_i32(hc.tables.block_tables), to_dev_i32(hc.tables.context_lens),
            hc.shape.scale, int(hc.tables.context_lens.max()),
            to_dev_i32(hc.tables.prefix_phys), 0, B, workspace=small)
    assert info.value.status == pkv.PKV_EWORKSPACE


@pytest.mark.parametrize("profile", rc.PROFILES)
def test_verify_prefix_rescale(pkv, orc, profile):
    """Scores shaped as in rescale_cases (a 12-block prefix shared by six
    members, two sequences ending inside it), 5 query tokens per sequence
    (fewer if a context is shorter)."""
    d = 128
    case, pre, first, count = rc.prefix_case(profile, d, 310 + rc.PROFILES.index(profile))
    hc = case.hc
    q_len = min(5, int(hc.tables.context_lens.min()))   # every context holds its query tokens
    qv = w.normal_bf16(w.rng(77010, rc.PROFILES.index(profile)), (hc.q.shape[0], q_len) + hc.q.shape[1:])
    if not profile.startswith("scale_"):
        rc.shrink_query_noise(qv)
        rc.set_query_dim0(qv)
    print(f"verify prefix {profile}", flush=True)
    got, err = _run(pkv, hc, qv, case.scale, prefix=True, first=first, count=count)
    assert err == 0 and np.isfinite(got).all()
    want, rc_ = orc.verify(qv, hc.k_pool, hc.v_pool, hc.tables.block_tables,
                           hc.tables.context_lens, hc.shape.n_kv, case.scale)
    assert rc_ == 0
    vcase = rc.Case(hc, profile, case.scale, case.offs, qv, append=False)
    keep = rc.conditioned_rows(vcase)
    assert (~keep).sum() <= 0.2 * keep.size
    e = max_abs(got[keep], want[keep])
    print(f"  max-abs {e:.2e} ({int((~keep).sum())} rows left out)")
    assert e <= TOL
